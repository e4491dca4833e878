// bf16 MFMA state spine (placeholder until the kernel lands).
#include "gdn_internal.h"

namespace gdn {

bool prefill_mfma_accepts(const PrefillArgs&) { return false; }

Geometry prefill_mfma_geometry(const PrefillArgs& a)
{
    Geometry g{"gdn_prefill_mfma_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u}, 256u, 0u};
    return g;
}

hipError_t launch_prefill_mfma(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn

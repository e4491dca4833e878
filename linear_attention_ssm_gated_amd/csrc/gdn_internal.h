// Internal declarations shared by the HIP sources of libgdn.so.  Not part of
// the C ABI (include/gdn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Arguments of one prefill call after host validation.
struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_g;
    const float* beta;
    const float* h0;
    void* out;
    float* h_final;
    int B, T, Hk, Hv, dk, dv, chunk;
    const int32_t* cu_seqlens;
    int io_dtype, out_dtype;
    void* workspace;
    size_t workspace_bytes;
    bool segmented;   // the segment-scan route where it applies (gdn_chunk_prefill_segmented)
};

struct VerifyArgs {
    float* const* h_table;
    const void* q;
    const void* k;
    const void* v;
    const float* gate;
    const float* beta;
    void* out;
    float* stash;
    int B, Hk, Hv, dk, dv;
    int qk_stride, v_stride, gb_stride, stash_seq_floats;
    uint32_t* engaged_flag;
    int io_dtype, out_dtype;
    int k_rows;
};

struct FoldArgs {
    float* const* h_table;
    const float* stash;
    const int32_t* na_tab;
    const uint32_t* engaged_flag;
    int B, Hk, Hv, dk, dv, stash_seq_floats;
    int io_dtype;
    int k_rows;
};

// The parent-mode verify: the verify's arguments (engaged_flag NULL: the
// word is left alone) and the per-sequence slab tables.
struct ParentArgs {
    VerifyArgs v;
    float* const* hi_tables;
    int slab_entries;
};

struct StepArgs {
    float* const* h_table;
    const void* q;
    const void* k;
    const void* v;
    const float* gate;
    const float* beta;
    void* out;
    int B, Hk, Hv, dk, dv;
    int qk_stride, v_stride, gb_stride;
    int io_dtype, out_dtype;
};

// Arguments of one gate/beta producer call after host validation.
struct BaArgs {
    const void* input;       // bf16 [m][k_stride]
    const void* ba_weight;   // bf16 [n][k]
    const float* a_log;
    const float* dt_bias;
    float* gate_out;         // fp32 [m][gate_stride]: gate [0, nv), beta [nv, 2 nv)
    int m, n, k, k_stride, gate_stride, nv, vheads_per_group;
    void* workspace;
    size_t workspace_bytes;
};

constexpr int kMaxVerifyRows = 8;   // draft rows a verify takes

// Launch geometry a launcher reports for the route line.
struct Geometry {
    const char* entry;
    unsigned grid[3];
    unsigned block;
    unsigned lds_bytes;
};

// Kernel choice and geometry of a prefill call (no launch).
bool prefill_mfma_accepts(const PrefillArgs& a);
size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv, bool packed, bool segmented);
// Workspace bytes one prefill call needs: the plain route's, or with
// segmented the segment scan's where it is taken (which covers the plain one).
size_t prefill_workspace_need(int B, int T, int Hk, int Hv, int dk, int dv, int chunk, int io_dtype,
                              bool packed, bool segmented);
Geometry prefill_generic_geometry(const PrefillArgs& a);
Geometry prefill_mfma_geometry(const PrefillArgs& a);
int prefill_mfma_segments(const PrefillArgs& a);   // segments per sequence of the segment scan, 0 = plain spine
Geometry verify_geometry(const VerifyArgs& a);
Geometry fold_geometry(const FoldArgs& a);
Geometry step_geometry(const StepArgs& a);
Geometry flag_clear_geometry();
Geometry parent_geometry(const ParentArgs& a);
Geometry restore_geometry(const FoldArgs& a);
size_t ba_gates_workspace_bytes(int m, int n, int k);
Geometry ba_gates_geometry(const BaArgs& a);

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);
hipError_t launch_fold(const FoldArgs& a, hipStream_t s);
hipError_t launch_step(const StepArgs& a, hipStream_t s);
hipError_t launch_flag_clear(uint32_t* flag, hipStream_t s);
hipError_t launch_parent(const ParentArgs& a, hipStream_t s);
hipError_t launch_restore(const FoldArgs& a, float* const* hi_tables, hipStream_t s);
hipError_t launch_ba_gates(const BaArgs& a, hipStream_t s);

// Per-v-head stash floats of a k_rows-row verify: delta [k_rows][dv] fp32,
// G [k_rows] fp32, then the keys [k_rows][dk] as fp32 or as packed bf16 bits
// (rounded up to whole floats).
__host__ __device__ inline size_t stash_head_floats(int dk, int dv, int io_dtype, int k_rows) {
    const size_t kd = (size_t)k_rows * dk;
    return (size_t)k_rows * dv + k_rows + (io_dtype == 1 ? (kd + 1) / 2 : kd);
}

// Route-line helpers of the C ABI layer (gdn_api.hip) for the other entry
// files: a refusal of a call whose scratch exceeds the static scratch, and a
// failed runtime call.  Both return the status to hand back.
int refuse_noalloc(size_t need);
int hip_failure(const char* what, hipError_t e);

// ---- element helpers ------------------------------------------------------
// bf16 is carried as its 16 raw bits; widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// States reached through a device pointer table are plain (generic) pointers
// to the compiler, which then issues flat loads and stores; flat accesses count
// on the LDS counter as well, so every LDS wait would also wait for them.
// Naming the global address space gives global accesses.
#define GDN_GLOBAL __attribute__((address_space(1)))
typedef float gdn_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_global4(const float* p) {
    const gdn_f4 x = *(const GDN_GLOBAL gdn_f4*)p;
    return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void store_global4(float* p, float4 v) {
    *(GDN_GLOBAL gdn_f4*)p = gdn_f4{v.x, v.y, v.z, v.w};
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    __device__ __forceinline__ static void store(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }
};

}  // namespace gdn

// C ABI of libgdn.so (declared in include/gdn.h): host-side validation that
// names every refusal, the kernel choice, the route line, and the launches.
//
// The route line follows the pages' rule that a log must name the entry that
// actually launched, with its geometry (ssm_gdn_tc_route.rs, the route-line
// functions and their tests), and that a fast path refused by a shape guard
// names the guard (ssm_ba_gates_hopper.rs, doc of its reject function).
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <set>
#include <string>

namespace {

thread_local char t_route[512] = "no call yet";

// GDN_LOG_ROUTE=1: each distinct route line goes to stderr once per process.
bool log_routes()
{
    static const bool on = [] {
        const char* e = getenv("GDN_LOG_ROUTE");
        return e && e[0] == '1' && e[1] == 0;
    }();
    return on;
}

void log_route_once(const char* line)
{
    static std::mutex mu;
    static std::set<std::string> seen;
    std::lock_guard<std::mutex> lock(mu);
    if (seen.insert(line).second) fprintf(stderr, "[gdn route] %s\n", line);
}

void set_route(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void set_route(const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_route, sizeof(t_route), fmt, ap);
    va_end(ap);
    if (log_routes()) log_route_once(t_route);
}

int refuse(int status, const char* who, const char* why)
{
    set_route("%s refused: %s (%s)", who, gdn_status_string(status), why);
    return status;
}

bool bad_dtype(int d) { return d != GDN_F32 && d != GDN_BF16; }

void route_geometry(const gdn::Geometry& g, const char* note)
{
    set_route("%s grid=[%u,%u,%u] block=%u lds=%uB%s%s", g.entry, g.grid[0], g.grid[1], g.grid[2],
              g.block, g.lds_bytes, note && *note ? " " : "", note ? note : "");
}

// Validation shared by gdn_chunk_prefill and its plan.  On success *mfma tells
// which kernel runs and *why names the guard that sent it to the generic one.
int check_prefill(const gdn::PrefillArgs& a, bool* mfma, const char** why)
{
    const char* who = "gdn_chunk_prefill";
    if (bad_dtype(a.io_dtype) || bad_dtype(a.out_dtype))
        return refuse(GDN_ERR_DTYPE, who, "io_dtype/out_dtype must be GDN_F32 or GDN_BF16");
    if (a.B < 1 || a.T < 0 || a.Hk < 1 || a.Hv < 1 || a.dk < 1 || a.dv < 1 || a.chunk < 1)
        return refuse(GDN_ERR_SHAPE, who, "need B, Hk, Hv, dk, dv, chunk >= 1 and T >= 0");
    if (a.B > 65535 || a.Hv > 65535)
        return refuse(GDN_ERR_SHAPE, who, "B or Hv > 65535 (grid y limit)");
    if (a.Hv % a.Hk != 0)
        return refuse(GDN_ERR_HEAD_GROUPS, who, "Hv must be a multiple of Hk");
    if (a.dk > 128 || a.dv > 128 || a.chunk > 64)
        return refuse(GDN_ERR_DIM_LIMIT, who, "dk, dv <= 128 and chunk <= 64");
    if (a.T > 0 && (!a.q || !a.k || !a.v || !a.log_g || !a.beta || !a.out))
        return refuse(GDN_ERR_NULL, who, "q, k, v, log_g, beta and out are required when T > 0");
    const size_t need = gdn::prefill_workspace_need(a.B, a.T, a.Hk, a.Hv, a.dk, a.dv, a.chunk, a.io_dtype,
                                                    a.cu_seqlens != nullptr, a.segmented);
    if (need > 0 && (!a.workspace || a.workspace_bytes < need))
        return refuse(GDN_ERR_WORKSPACE, who, "workspace smaller than gdn_prefill_workspace_bytes()");
    *why = "";
    if (a.io_dtype != GDN_BF16) *why = "(generic: io dtype is f32; the MFMA spine takes bf16)";
    else if (a.dk != 128 || a.dv != 128) *why = "(generic: the MFMA spine takes dk = dv = 128)";
    else if (a.chunk != 64) *why = "(generic: the MFMA spine takes chunk = 64)";
    *mfma = gdn::prefill_mfma_accepts(a) && !**why;
    if (!*mfma && !**why) *why = "(generic: MFMA spine not built)";
    return GDN_OK;
}

// Validation of a verify; the parent verify (need_flag false) leaves the word
// alone and takes no flag.
int check_verify(const gdn::VerifyArgs& a, const char* who = "gdn_decode_verify", bool need_flag = true)
{
    if (bad_dtype(a.io_dtype) || bad_dtype(a.out_dtype))
        return refuse(GDN_ERR_DTYPE, who, "io_dtype/out_dtype must be GDN_F32 or GDN_BF16");
    if (!a.h_table || !a.stash || (need_flag && !a.engaged_flag))
        return refuse(GDN_ERR_NULL, who, need_flag ? "null table/stash/flag" : "null table/stash");
    if (!a.q || !a.k || !a.v || !a.gate || !a.beta || !a.out)
        return refuse(GDN_ERR_NULL, who, "q, k, v, gate, beta and out are required");
    if (a.B < 1 || a.Hk < 1 || a.Hv < 1 || a.dk < 1 || a.dv < 1)
        return refuse(GDN_ERR_SHAPE, who, "need B, Hk, Hv, dk, dv >= 1");
    if (a.B > 65535) return refuse(GDN_ERR_SHAPE, who, "B > 65535 (grid y limit)");
    if (a.Hv % a.Hk != 0) return refuse(GDN_ERR_HEAD_GROUPS, who, "Hv must be a multiple of Hk");
    if (a.dk > 128 || a.dv > 128 || a.dv % 4 != 0)
        return refuse(GDN_ERR_DIM_LIMIT, who, "dk <= 128, dv <= 128 and dv a multiple of 4");
    if ((long)a.qk_stride < (long)a.Hk * a.dk || (long)a.v_stride < (long)a.Hv * a.dv ||
        (long)a.gb_stride < (long)a.Hv)
        return refuse(GDN_ERR_STRIDE, who, "a row stride is shorter than its row");
    if (a.k_rows < 1 || a.k_rows > gdn::kMaxVerifyRows)
        return refuse(GDN_ERR_K_ROWS, who, "k_rows must be 1..8");
    if ((size_t)a.stash_seq_floats < gdn_stash_seq_floats(a.Hv, a.dk, a.dv, a.k_rows, a.io_dtype))
        return refuse(GDN_ERR_STASH, who, "stash_seq_floats < gdn_stash_seq_floats()");
    return GDN_OK;
}

int check_fold(const gdn::FoldArgs& a, float* const* hi_tables, int slab_entries)
{
    const char* who = "gdn_fold";
    if (bad_dtype(a.io_dtype)) return refuse(GDN_ERR_DTYPE, who, "io_dtype must be GDN_F32 or GDN_BF16");
    if (a.k_rows < 1 || a.k_rows > gdn::kMaxVerifyRows)
        return refuse(GDN_ERR_K_ROWS, who, "k_rows must be 1..8");
    if (hi_tables && slab_entries < a.k_rows)
        return refuse(GDN_ERR_SLABS, who, "slab_entries < k_rows: the restore reads slabs 0 .. k_rows - 1");
    if (!a.h_table || !a.stash || !a.na_tab || !a.engaged_flag)
        return refuse(GDN_ERR_NULL, who, "null table/stash/na_tab/flag");
    if (a.B < 1 || a.Hk < 1 || a.Hv < 1 || a.dk < 1 || a.dv < 1)
        return refuse(GDN_ERR_SHAPE, who, "need B, Hk, Hv, dk, dv >= 1");
    if (a.B > 65535) return refuse(GDN_ERR_SHAPE, who, "B > 65535 (grid y limit)");
    if (a.Hv % a.Hk != 0) return refuse(GDN_ERR_HEAD_GROUPS, who, "Hv must be a multiple of Hk");
    if (a.dk > 128 || a.dv > 128 || a.dv % 4 != 0)
        return refuse(GDN_ERR_DIM_LIMIT, who, "dk <= 128, dv <= 128 and dv a multiple of 4");
    if ((size_t)a.stash_seq_floats < gdn_stash_seq_floats(a.Hv, a.dk, a.dv, a.k_rows, a.io_dtype))
        return refuse(GDN_ERR_STASH, who, "stash_seq_floats < gdn_stash_seq_floats()");
    return GDN_OK;
}

int check_step(const gdn::StepArgs& a)
{
    const char* who = "gdn_decode_step";
    if (bad_dtype(a.io_dtype) || bad_dtype(a.out_dtype))
        return refuse(GDN_ERR_DTYPE, who, "io_dtype/out_dtype must be GDN_F32 or GDN_BF16");
    if (!a.h_table || !a.q || !a.k || !a.v || !a.gate || !a.beta || !a.out)
        return refuse(GDN_ERR_NULL, who, "h_table, q, k, v, gate, beta and out are required");
    if (a.B < 1 || a.Hk < 1 || a.Hv < 1 || a.dk < 1 || a.dv < 1)
        return refuse(GDN_ERR_SHAPE, who, "need B, Hk, Hv, dk, dv >= 1");
    if (a.B > 65535) return refuse(GDN_ERR_SHAPE, who, "B > 65535 (grid y limit)");
    if (a.Hv % a.Hk != 0) return refuse(GDN_ERR_HEAD_GROUPS, who, "Hv must be a multiple of Hk");
    if (a.dk > 128 || a.dv > 128 || a.dv % 4 != 0)
        return refuse(GDN_ERR_DIM_LIMIT, who, "dk <= 128, dv <= 128 and dv a multiple of 4");
    if ((long)a.qk_stride < (long)a.Hk * a.dk || (long)a.v_stride < (long)a.Hv * a.dv ||
        (long)a.gb_stride < (long)a.Hv)
        return refuse(GDN_ERR_STRIDE, who, "a row stride is shorter than its row");
    return GDN_OK;
}

int launched(hipError_t e)
{
    if (e == hipSuccess) return GDN_OK;
    size_t n = strlen(t_route);
    snprintf(t_route + n, sizeof(t_route) - n, " -- launch failed: %s", hipGetErrorString(e));
    if (log_routes()) log_route_once(t_route);
    return GDN_ERR_HIP;
}

gdn::PrefillArgs make_prefill(const void* q, const void* k, const void* v, const float* log_g,
                              const float* beta, const float* h0, void* out, float* h_final, int B,
                              int T, int Hk, int Hv, int dk, int dv, int chunk,
                              const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                              void* workspace, size_t workspace_bytes)
{
    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta; a.h0 = h0; a.out = out;
    a.h_final = h_final; a.B = B; a.T = T; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv;
    a.chunk = chunk; a.cu_seqlens = cu_seqlens; a.io_dtype = io_dtype; a.out_dtype = out_dtype;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.segmented = false;
    return a;
}

}  // namespace

namespace gdn {
int refuse_noalloc(size_t need)
{
    char why[160];
    snprintf(why, sizeof(why), "the call needs %zu bytes of device scratch, more than the %zu-byte static scratch",
             need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    return refuse(GDN_ERR_WORKSPACE, "gdn_chunk_prefill_noalloc", why);
}
int hip_failure(const char* what, hipError_t e)
{
    set_route("%s failed: %s", what, hipGetErrorString(e));
    return GDN_ERR_HIP;
}
}  // namespace gdn

extern "C" {

const char* gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size is out of range";
    case GDN_ERR_HEAD_GROUPS: return "GDN_ERR_HEAD_GROUPS: Hv is not a multiple of Hk";
    case GDN_ERR_DIM_LIMIT: return "GDN_ERR_DIM_LIMIT: dk, dv or chunk beyond what any kernel takes";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype code";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace too small";
    case GDN_ERR_STASH: return "GDN_ERR_STASH: stash_seq_floats too small";
    case GDN_ERR_K_ROWS: return "GDN_ERR_K_ROWS: k_rows must be 1..8";
    case GDN_ERR_STRIDE: return "GDN_ERR_STRIDE: a row stride is shorter than its row";
    case GDN_ERR_SLABS: return "GDN_ERR_SLABS: slab_entries smaller than k_rows";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime refused a launch";
    default: return "unknown gdn status";
    }
}

const char* gdn_last_route(void) { return t_route; }

size_t gdn_prefill_workspace_bytes(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                   int io_dtype, int packed)
{
    // enough for either entry point
    return gdn::prefill_workspace_need(B, T, Hk, Hv, dk, dv, chunk, io_dtype, packed != 0, true);
}

int gdn_chunk_prefill_plan(const void* q, const void* k, const void* v, const float* log_g,
                           const float* beta, const float* h0, void* out, float* h_final, int B,
                           int T, int Hk, int Hv, int dk, int dv, int chunk,
                           const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                           void* workspace, size_t workspace_bytes)
{
    gdn::PrefillArgs a = make_prefill(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv,
                                      chunk, cu_seqlens, io_dtype, out_dtype, workspace,
                                      workspace_bytes);
    bool mfma = false;
    const char* why = "";
    int st = check_prefill(a, &mfma, &why);
    if (st != GDN_OK) return st;
    route_geometry(mfma ? gdn::prefill_mfma_geometry(a) : gdn::prefill_generic_geometry(a), why);
    return GDN_OK;
}

int gdn_chunk_prefill(const void* q, const void* k, const void* v, const float* log_g,
                      const float* beta, const float* h0, void* out, float* h_final, int B, int T,
                      int Hk, int Hv, int dk, int dv, int chunk, const int32_t* cu_seqlens,
                      int io_dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    gdn::PrefillArgs a = make_prefill(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv,
                                      chunk, cu_seqlens, io_dtype, out_dtype, workspace,
                                      workspace_bytes);
    bool mfma = false;
    const char* why = "";
    int st = check_prefill(a, &mfma, &why);
    if (st != GDN_OK) return st;
    route_geometry(mfma ? gdn::prefill_mfma_geometry(a) : gdn::prefill_generic_geometry(a), why);
    return launched(mfma ? gdn::launch_prefill_mfma(a, stream) : gdn::launch_prefill_generic(a, stream));
}

// The segment-scan twin: the same validation and routes, and on the MFMA
// route the segment scan where segment_cut takes it (dense input, few spine
// workgroups); the route line names the route that runs.
static int prefill_segmented(bool launch, const void* q, const void* k, const void* v, const float* log_g,
                             const float* beta, const float* h0, void* out, float* h_final, int B, int T,
                             int Hk, int Hv, int dk, int dv, int chunk, const int32_t* cu_seqlens,
                             int io_dtype, int out_dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    gdn::PrefillArgs a = make_prefill(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv,
                                      chunk, cu_seqlens, io_dtype, out_dtype, workspace,
                                      workspace_bytes);
    a.segmented = true;
    bool mfma = false;
    const char* why = "";
    int st = check_prefill(a, &mfma, &why);
    if (st != GDN_OK) return st;
    if (mfma && gdn::prefill_mfma_segments(a) == 0)
        why = cu_seqlens ? "(plain spine: the segment scan takes dense input)"
                         : "(plain spine: the spine's workgroups fill the chip, or too few chunks)";
    route_geometry(mfma ? gdn::prefill_mfma_geometry(a) : gdn::prefill_generic_geometry(a), why);
    if (!launch) return GDN_OK;
    return launched(mfma ? gdn::launch_prefill_mfma(a, stream) : gdn::launch_prefill_generic(a, stream));
}

int gdn_chunk_prefill_segmented(const void* q, const void* k, const void* v, const float* log_g,
                                const float* beta, const float* h0, void* out, float* h_final, int B,
                                int T, int Hk, int Hv, int dk, int dv, int chunk,
                                const int32_t* cu_seqlens, int io_dtype, int out_dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    return prefill_segmented(true, q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                             cu_seqlens, io_dtype, out_dtype, workspace, workspace_bytes, stream);
}

int gdn_chunk_prefill_segmented_plan(const void* q, const void* k, const void* v, const float* log_g,
                                     const float* beta, const float* h0, void* out, float* h_final,
                                     int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                     const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                                     void* workspace, size_t workspace_bytes)
{
    return prefill_segmented(false, q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                             cu_seqlens, io_dtype, out_dtype, workspace, workspace_bytes, nullptr);
}

size_t gdn_stash_seq_floats(int Hv, int dk, int dv, int k_rows, int io_dtype)
{
    if (Hv < 1 || dk < 1 || dv < 1 || k_rows < 1 || k_rows > gdn::kMaxVerifyRows) return 0;
    return (size_t)Hv * gdn::stash_head_floats(dk, dv, io_dtype == GDN_BF16 ? 1 : 0, k_rows);
}

int gdn_flag_clear(uint32_t* engaged_flag, hipStream_t stream)
{
    if (!engaged_flag) return refuse(GDN_ERR_NULL, "gdn_flag_clear", "null flag");
    route_geometry(gdn::flag_clear_geometry(), "");
    return launched(gdn::launch_flag_clear(engaged_flag, stream));
}

static gdn::VerifyArgs make_verify(float* const* h_table, const void* q, const void* k, const void* v,
                                   const float* gate, const float* beta, void* out, float* stash,
                                   int B, int Hk, int Hv, int dk, int dv, int k_rows,
                                   int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                                   uint32_t* engaged_flag, int io_dtype, int out_dtype)
{
    gdn::VerifyArgs a;
    a.k_rows = k_rows;
    a.h_table = h_table; a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.out = out;
    a.stash = stash; a.B = B; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.qk_stride = qk_stride;
    a.v_stride = v_stride; a.gb_stride = gb_stride; a.stash_seq_floats = stash_seq_floats;
    a.engaged_flag = engaged_flag; a.io_dtype = io_dtype; a.out_dtype = out_dtype;
    return a;
}

int gdn_decode_verify_plan(float* const* h_table, const void* q, const void* k, const void* v,
                           const float* gate, const float* beta, void* out, float* stash, int B,
                           int Hk, int Hv, int dk, int dv, int k_rows, int qk_stride, int v_stride,
                           int gb_stride, int stash_seq_floats, uint32_t* engaged_flag, int io_dtype,
                           int out_dtype)
{
    gdn::VerifyArgs a = make_verify(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, k_rows,
                                    qk_stride, v_stride, gb_stride, stash_seq_floats, engaged_flag,
                                    io_dtype, out_dtype);
    int st = check_verify(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::verify_geometry(a), "");
    return GDN_OK;
}

int gdn_decode_verify(float* const* h_table, const void* q, const void* k, const void* v,
                      const float* gate, const float* beta, void* out, float* stash, int B, int Hk,
                      int Hv, int dk, int dv, int k_rows, int qk_stride, int v_stride, int gb_stride,
                      int stash_seq_floats, uint32_t* engaged_flag, int io_dtype, int out_dtype,
                      hipStream_t stream)
{
    gdn::VerifyArgs a = make_verify(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, k_rows,
                                    qk_stride, v_stride, gb_stride, stash_seq_floats, engaged_flag,
                                    io_dtype, out_dtype);
    int st = check_verify(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::verify_geometry(a), "");
    return launched(gdn::launch_verify(a, stream));
}

int gdn_decode_verify_k4_plan(float* const* h_table, const void* q, const void* k, const void* v,
                              const float* gate, const float* beta, void* out, float* stash, int B,
                              int Hk, int Hv, int dk, int dv, int qk_stride, int v_stride,
                              int gb_stride, int stash_seq_floats, uint32_t* engaged_flag,
                              int io_dtype, int out_dtype)
{
    return gdn_decode_verify_plan(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, 4,
                                  qk_stride, v_stride, gb_stride, stash_seq_floats, engaged_flag,
                                  io_dtype, out_dtype);
}

int gdn_decode_verify_k4(float* const* h_table, const void* q, const void* k, const void* v,
                         const float* gate, const float* beta, void* out, float* stash, int B,
                         int Hk, int Hv, int dk, int dv, int qk_stride, int v_stride, int gb_stride,
                         int stash_seq_floats, uint32_t* engaged_flag, int io_dtype, int out_dtype,
                         hipStream_t stream)
{
    return gdn_decode_verify(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, 4, qk_stride,
                             v_stride, gb_stride, stash_seq_floats, engaged_flag, io_dtype, out_dtype,
                             stream);
}

static gdn::FoldArgs make_fold(float* const* h_table, const float* stash, const int32_t* na_tab,
                               const uint32_t* engaged_flag, int k_rows, int B, int Hk, int Hv,
                               int dk, int dv, int stash_seq_floats, int io_dtype)
{
    gdn::FoldArgs a;
    a.k_rows = k_rows;
    a.h_table = h_table; a.stash = stash; a.na_tab = na_tab; a.engaged_flag = engaged_flag;
    a.B = B; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.stash_seq_floats = stash_seq_floats;
    a.io_dtype = io_dtype;
    return a;
}

int gdn_fold_plan(float* const* h_table, const float* stash, const int32_t* na_tab,
                  float* const* hi_tables, int slab_entries, const uint32_t* engaged_flag,
                  int k_rows, int B, int Hk, int Hv, int dk, int dv, int stash_seq_floats,
                  int io_dtype)
{
    gdn::FoldArgs a = make_fold(h_table, stash, na_tab, engaged_flag, k_rows, B, Hk, Hv, dk, dv,
                                stash_seq_floats, io_dtype);
    int st = check_fold(a, hi_tables, slab_entries);
    if (st != GDN_OK) return st;
    route_geometry(gdn::fold_geometry(a), hi_tables ? "(+gdn_restore_kernel: word clear restores slab na)" : "");
    return GDN_OK;
}

int gdn_fold(float* const* h_table, const float* stash, const int32_t* na_tab,
             float* const* hi_tables, int slab_entries, const uint32_t* engaged_flag, int k_rows,
             int B, int Hk, int Hv, int dk, int dv, int stash_seq_floats, int io_dtype,
             hipStream_t stream)
{
    gdn::FoldArgs a = make_fold(h_table, stash, na_tab, engaged_flag, k_rows, B, Hk, Hv, dk, dv,
                                stash_seq_floats, io_dtype);
    int st = check_fold(a, hi_tables, slab_entries);
    if (st != GDN_OK) return st;
    route_geometry(gdn::fold_geometry(a), hi_tables ? "(+gdn_restore_kernel: word clear restores slab na)" : "");
    // each kernel reads the word: the restore acts when it is clear, the fold
    // when it is set
    if (hi_tables) {
        st = launched(gdn::launch_restore(a, hi_tables, stream));
        if (st != GDN_OK) return st;
    }
    return launched(gdn::launch_fold(a, stream));
}

// Validation of a parent verify (shared by the call and its plan).
static int check_parent(const gdn::ParentArgs& p)
{
    const char* who = "gdn_decode_verify_parent";
    int st = check_verify(p.v, who, false);
    if (st != GDN_OK) return st;
    if (!p.hi_tables) return refuse(GDN_ERR_NULL, who, "null hi_tables");
    if (p.slab_entries < p.v.k_rows)
        return refuse(GDN_ERR_SLABS, who, "slab_entries < k_rows: the verify writes slabs 0 .. k_rows - 1");
    return GDN_OK;
}

static gdn::ParentArgs make_parent(float* const* h_table, float* const* hi_tables, int slab_entries,
                                   const void* q, const void* k, const void* v, const float* gate,
                                   const float* beta, void* out, float* stash, int B, int Hk, int Hv,
                                   int dk, int dv, int k_rows, int qk_stride, int v_stride,
                                   int gb_stride, int stash_seq_floats, int io_dtype, int out_dtype)
{
    gdn::ParentArgs p;
    p.v = make_verify(h_table, q, k, v, gate, beta, out, stash, B, Hk, Hv, dk, dv, k_rows, qk_stride,
                      v_stride, gb_stride, stash_seq_floats, nullptr, io_dtype, out_dtype);
    p.hi_tables = hi_tables;
    p.slab_entries = slab_entries;
    return p;
}

int gdn_decode_verify_parent_plan(float* const* h_table, float* const* hi_tables, int slab_entries,
                                  const void* q, const void* k, const void* v, const float* gate,
                                  const float* beta, void* out, float* stash, int B, int Hk, int Hv,
                                  int dk, int dv, int k_rows, int qk_stride, int v_stride,
                                  int gb_stride, int stash_seq_floats, int io_dtype, int out_dtype)
{
    gdn::ParentArgs p = make_parent(h_table, hi_tables, slab_entries, q, k, v, gate, beta, out, stash, B,
                                    Hk, Hv, dk, dv, k_rows, qk_stride, v_stride, gb_stride,
                                    stash_seq_floats, io_dtype, out_dtype);
    int st = check_parent(p);
    if (st != GDN_OK) return st;
    route_geometry(gdn::parent_geometry(p), "");
    return GDN_OK;
}

int gdn_decode_verify_parent(float* const* h_table, float* const* hi_tables, int slab_entries,
                             const void* q, const void* k, const void* v, const float* gate,
                             const float* beta, void* out, float* stash, int B, int Hk, int Hv, int dk,
                             int dv, int k_rows, int qk_stride, int v_stride, int gb_stride,
                             int stash_seq_floats, int io_dtype, int out_dtype, hipStream_t stream)
{
    gdn::ParentArgs p = make_parent(h_table, hi_tables, slab_entries, q, k, v, gate, beta, out, stash, B,
                                    Hk, Hv, dk, dv, k_rows, qk_stride, v_stride, gb_stride,
                                    stash_seq_floats, io_dtype, out_dtype);
    int st = check_parent(p);
    if (st != GDN_OK) return st;
    route_geometry(gdn::parent_geometry(p), "");
    return launched(gdn::launch_parent(p, stream));
}

// Validation of a gate/beta producer call (shared by the call and its plan).
static int check_ba(const gdn::BaArgs& a)
{
    const char* who = "gdn_ba_gates";
    if (a.m < 0 || a.nv < 1 || a.vheads_per_group < 1 || a.k < 1)
        return refuse(GDN_ERR_SHAPE, who, "need m >= 0, nv, vheads_per_group and k >= 1");
    if (a.n != 2 * a.nv) return refuse(GDN_ERR_SHAPE, who, "n must be 2 * nv");
    if (a.nv % a.vheads_per_group != 0)
        return refuse(GDN_ERR_HEAD_GROUPS, who, "nv must be a multiple of vheads_per_group");
    if (a.n > 128 || a.k % 64 != 0)
        return refuse(GDN_ERR_DIM_LIMIT, who, "n <= 128 and k a multiple of 64");
    if (a.k_stride < a.k || a.k_stride % 8 != 0 || a.gate_stride < 2 * a.nv)
        return refuse(GDN_ERR_STRIDE, who, "k_stride >= k (a multiple of 8) and gate_stride >= 2 * nv");
    if ((long)a.m * a.k_stride >= (1L << 30) || (long)a.n * a.k >= (1L << 30))
        return refuse(GDN_ERR_SHAPE, who, "m * k_stride and n * k must stay below 2^30");
    if (a.m > 0 && (!a.input || !a.ba_weight || !a.a_log || !a.dt_bias || !a.gate_out))
        return refuse(GDN_ERR_NULL, who, "input, ba_weight, a_log, dt_bias and gate_out are required when m > 0");
    if (a.m > 0 && (!a.workspace || a.workspace_bytes < gdn::ba_gates_workspace_bytes(a.m, a.n, a.k)))
        return refuse(GDN_ERR_WORKSPACE, who, "workspace smaller than gdn_ba_gates_workspace_bytes()");
    return GDN_OK;
}

static gdn::StepArgs make_step(float* const* h_table, const void* q, const void* k, const void* v,
                               const float* gate, const float* beta, void* out, int B, int Hk, int Hv,
                               int dk, int dv, int qk_stride, int v_stride, int gb_stride,
                               int io_dtype, int out_dtype)
{
    gdn::StepArgs a;
    a.h_table = h_table; a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.out = out;
    a.B = B; a.Hk = Hk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.qk_stride = qk_stride;
    a.v_stride = v_stride; a.gb_stride = gb_stride; a.io_dtype = io_dtype; a.out_dtype = out_dtype;
    return a;
}

int gdn_decode_step_plan(float* const* h_table, const void* q, const void* k, const void* v,
                         const float* gate, const float* beta, void* out, int B, int Hk, int Hv,
                         int dk, int dv, int qk_stride, int v_stride, int gb_stride, int io_dtype,
                         int out_dtype)
{
    gdn::StepArgs a = make_step(h_table, q, k, v, gate, beta, out, B, Hk, Hv, dk, dv, qk_stride,
                                v_stride, gb_stride, io_dtype, out_dtype);
    int st = check_step(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::step_geometry(a), "");
    return GDN_OK;
}

int gdn_decode_step(float* const* h_table, const void* q, const void* k, const void* v,
                    const float* gate, const float* beta, void* out, int B, int Hk, int Hv, int dk,
                    int dv, int qk_stride, int v_stride, int gb_stride, int io_dtype, int out_dtype,
                    hipStream_t stream)
{
    gdn::StepArgs a = make_step(h_table, q, k, v, gate, beta, out, B, Hk, Hv, dk, dv, qk_stride,
                                v_stride, gb_stride, io_dtype, out_dtype);
    int st = check_step(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::step_geometry(a), "");
    return launched(gdn::launch_step(a, stream));
}

size_t gdn_ba_gates_workspace_bytes(int m, int n, int k)
{
    if (m < 0 || n < 1 || k < 1) return 0;
    return gdn::ba_gates_workspace_bytes(m, n, k);
}

int gdn_ba_gates_plan(const void* input, const void* ba_weight, const float* a_log,
                      const float* dt_bias, float* gate_out, int m, int n, int k, int k_stride,
                      int gate_stride, int nv, int vheads_per_group, void* workspace,
                      size_t workspace_bytes)
{
    gdn::BaArgs a{input, ba_weight, a_log, dt_bias, gate_out, m, n, k, k_stride, gate_stride, nv,
                  vheads_per_group, workspace, workspace_bytes};
    int st = check_ba(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::ba_gates_geometry(a), "");
    return GDN_OK;
}

int gdn_ba_gates(const void* input, const void* ba_weight, const float* a_log,
                 const float* dt_bias, float* gate_out, int m, int n, int k, int k_stride,
                 int gate_stride, int nv, int vheads_per_group, void* workspace,
                 size_t workspace_bytes, hipStream_t stream)
{
    gdn::BaArgs a{input, ba_weight, a_log, dt_bias, gate_out, m, n, k, k_stride, gate_stride, nv,
                  vheads_per_group, workspace, workspace_bytes};
    int st = check_ba(a);
    if (st != GDN_OK) return st;
    route_geometry(gdn::ba_gates_geometry(a), "");
    return launched(gdn::launch_ba_gates(a, stream));
}

}  // extern "C"

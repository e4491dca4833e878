/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library (libgdn.so).
 *
 * The method: the Gated DeltaNet recurrence (Yang, Kautz, Hatamizadeh, "Gated
 * Delta Networks", ICLR 2025), whose kernels the pages name gated_delta_rule_*
 * (ssm_gdn_tc_route.rs, module doc and the spine entry constants):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t,
 *
 * with alpha_t = exp(log_g_t) (log_g <= 0), no scale on q, and S_t a dv x dk
 * matrix per (sequence, v-head).  States cross this ABI as h = S^T: dk rows of
 * dv fp32 values, row-major ("dk*dv fp32 per head", ssm_gdn_woa.rs, the
 * shared-memory size of the verify launch).  V-head vh reads k-head
 * vh / (Hv / Hk) (ssm_ba_gates_hopper.rs, the v-head grouping of its index model).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (the caller allocates them; the
 *    library never allocates, frees or synchronises).  h_table/hi_tables are
 *    device arrays of device pointers.
 *  - Shapes and pointers are validated on the host before anything is
 *    launched; a refusal returns a named status (gdn_status_string) and
 *    launches nothing.  A refused fast path is never silent: either the
 *    generic kernel runs and gdn_last_route() names it, or an error returns.
 *  - Work is enqueued on `stream` and the call returns without waiting.
 *  - Floating-point inputs are read as given; bf16 values are widened exactly.
 *  - Entry points are reentrant and thread-safe; gdn_last_route() is
 *    thread-local.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q/k/v (io_dtype) and of the output (out_dtype). */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Return codes.  0 = success; every refusal has its own code and text. */
typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,          /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,         /* B < 1, T < 0, a head count, dk, dv or chunk < 1; B or Hv > 65535 */
    GDN_ERR_HEAD_GROUPS = 3,   /* Hv is not a multiple of Hk */
    GDN_ERR_DIM_LIMIT = 4,     /* dk or dv > 128, or chunk > 64: no kernel here takes it */
    GDN_ERR_DTYPE = 5,         /* unknown dtype code */
    GDN_ERR_WORKSPACE = 6,     /* workspace smaller than gdn_prefill_workspace_bytes() */
    GDN_ERR_STASH = 7,         /* stash_seq_floats smaller than gdn_stash_seq_floats() */
    GDN_ERR_K_ROWS = 8,        /* k_rows outside 1..8 */
    GDN_ERR_STRIDE = 9,        /* a row stride shorter than the heads it must hold */
    GDN_ERR_SLABS = 10,        /* slab_entries smaller than k_rows (parent verify, fold restore) */
    GDN_ERR_HIP = 11           /* the HIP runtime refused a launch (text: gdn_last_route()) */
} gdn_status;

/* Static text naming a status.  Never NULL.  Every refusal names its reason
 * rather than failing silently, as the pages' launchers do with their checked
 * errors on null pointers and bad shapes (ssm_gdn_woa.rs, the argument checks
 * of the verify, fold and flag-clear launchers; ssm_ba_gates_hopper.rs, doc of
 * the reject function: a refused fast path names the guard that refused it). */
const char* gdn_status_string(int status);

/* Thread-local route line of the last call on this thread: the kernel entry
 * that was launched (or would be, for the *_plan functions), its grid, block
 * and LDS bytes, or the reason for a refusal.  Never NULL; valid until the
 * next call on the same thread.  The rule that a log line names the entry that
 * actually ran, with its launch geometry, is the pages' (ssm_gdn_tc_route.rs,
 * the route-line functions and their tests).  With the environment variable
 * GDN_LOG_ROUTE=1 (read once per process), each distinct route line is also
 * written once to stderr, the first time a call produces it (the pages log
 * each branch once, ssm_ba_gates_hopper.rs, its once-per-branch logging). */
const char* gdn_last_route(void);

/* ------------------------------------------------------------------------ */
/* Chunked prefill.
 *
 * The pages' "state spine" (ssm_gdn_tc_route.rs, doc of the spine entry
 * constants): sequences are cut into chunks of `chunk` tokens; inside a chunk
 * the delta rule is solved in closed form (WY/UT form: T = (I + A)^-1 with
 * A = strict_lower(diag(beta) (Gamma o K K^T)), U = T diag(beta) V,
 * W = T diag(beta gamma) K) and the fp32 state walks the chunks in order,
 * h <- gamma_L h + K~^T (U - W h) ("h stays f32", same page, the route line
 * of the tensor-core spine), while each chunk's outputs are
 * O = diag(gamma) Q h + (lower_incl(Q K^T) o Gamma)(U - W h).
 *
 * Layouts (row-major, element strides implied by the shapes):
 *   dense  (cu_seqlens == NULL): q, k [B][T][Hk][dk];  v, out [B][T][Hv][dv];
 *                                log_g, beta [B][T][Hv]
 *   packed (cu_seqlens != NULL): the B sequences' rows concatenated, T = total
 *                                rows: q, k [T][Hk][dk]; v, out [T][Hv][dv];
 *                                log_g, beta [T][Hv]; cu_seqlens: device int32
 *                                [B+1], cu[0] = 0, non-decreasing, cu[B] = T
 *                                (values outside [0, T] are clamped into it).
 *   h0, h_final: [B][Hv][dk][dv] fp32.  h0 == NULL means zero states;
 *   h_final == NULL means the final states are not written; h0 == h_final is
 *   allowed (updated in place).  q, k, v: io_dtype; out: out_dtype; log_g
 *   (natural log of the decay, <= 0, finite) and beta: fp32.  Any finite
 *   gates are taken: every decay factor either kernel forms is exp of a
 *   non-positive difference of cumulative log decays.
 *
 * Kernels: io_dtype == GDN_BF16 with dk == dv == 128 and chunk == 64 runs the
 * bf16-MFMA spine (fp32 state and accumulators).  Every other accepted shape
 * runs the generic fp32-arithmetic chunked kernel (dk, dv <= 128, chunk <= 64).
 * gdn_last_route() names the one that ran.
 * workspace: device scratch of at least gdn_prefill_workspace_bytes() bytes
 * (may be NULL when that is 0), asked with the same B, T, shapes and io_dtype,
 * and packed = (cu_seqlens != NULL).  The MFMA route keeps a chunk table of
 * packed sequences (their first chunks, and for up to 256 sequences their
 * order by length, longest first, in which the state walks are dispatched),
 * and for every (chunk, v-head) T_e = diag(exp(G_L - G)) T diag(beta), with
 * T = (I + A)^-1, and PT = (Gamma o lower_incl(Q K^T)) T diag(beta), each as
 * 64 x 64 bf16 in MFMA fragment order (6 KiB; the granules above their
 * diagonals are never written or read) followed by the chunk's per-row decay
 * factors exp(G_r) (and exp(G_L) after T_e), 7 KiB per matrix; the generic
 * route needs none.  The size returned covers gdn_chunk_prefill_segmented
 * too: where its segment scan is taken, 3 fp32 128 x 128 matrices per
 * (segment, v-head) follow the slots (gdn_chunk_prefill itself asks only the
 * slots, and gdn_chunk_prefill_noalloc uses only those).
 * The library reads and writes the workspace only inside the call's stream
 * order; its contents need no initialisation.
 */
size_t gdn_prefill_workspace_bytes(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                   int io_dtype, int packed);

int gdn_chunk_prefill(const void* q, const void* k, const void* v,
                      const float* log_g, const float* beta,
                      const float* h0, void* out, float* h_final,
                      int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                      const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Validation and kernel choice of gdn_chunk_prefill without launching
 * anything: same return codes; gdn_last_route() holds the route.  Pointers are
 * only compared with NULL. */
int gdn_chunk_prefill_plan(const void* q, const void* k, const void* v,
                           const float* log_g, const float* beta,
                           const float* h0, void* out, float* h_final,
                           int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                           const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                           void* workspace, size_t workspace_bytes);

/* gdn_chunk_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * Same arguments, kernels, results and route line as gdn_chunk_prefill, minus
 * the workspace: the device scratch lives in a static array inside the library
 * (GDN_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on that
 * GPU until the process ends).  The call allocates and frees nothing; the first
 * call on a device looks the array's device address up once (the caller's
 * current device must be the device of `stream`).  A call whose scratch,
 * gdn_prefill_workspace_bytes(...), exceeds GDN_NOALLOC_SCRATCH_BYTES returns
 * GDN_ERR_WORKSPACE and launches nothing (e.g. a 4576-token call at Hv = 48
 * fits; a 29k-token packed call does not).  Every call on one GPU shares that
 * GPU's scratch, so two calls that overlap on one GPU (different streams or
 * threads without ordering between them) race; calls in one stream's order do
 * not.  The scratch needs no clearing between calls.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                              const float* log_g, const float* beta,
                              const float* h0, void* out, float* h_final,
                              int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                              const int32_t* cu_seqlens, int io_dtype, int out_dtype,
                              hipStream_t stream);

/* Segment-scan prefill (ssm_gdn_tc_route.rs, doc of the spine entries: the
 * spine walks the chunk states S_c in order, and the map from one chunk's
 * start state to the next is affine in the state).  Same arguments, layouts,
 * workspace (gdn_prefill_workspace_bytes covers both routes) and results as
 * gdn_chunk_prefill, to rounding: on the MFMA route, for dense input
 * (cu_seqlens == NULL) whose spine workgroups (B * Hv * 4) would fill at most
 * a third of the 256 compute units, each sequence is cut into S segments of
 * whole chunks (3 <= S <= 10, the most whose 2 S - 3 map walks per sequence
 * fit in 256 workgroups).  One spine launch walks segment 0 from h0 (its end
 * state N_0) and segments 1 .. S-2 both from zero (N_s) and from the identity
 * with V read as zero (the linear part M_s); a combine kernel applies the
 * maps in order per sequence (start(1) = N_0, start(s) = M_{s-1} start(s-1) +
 * N_{s-1}, in products of bf16 splits of the fp32 operands, about 16 bits
 * each); a second spine launch walks every segment from its start state,
 * writing the outputs, the last segment writing h_final.  Elsewhere it runs
 * the route gdn_chunk_prefill would, and the route line says why.
 * Deterministic run to run; not bitwise equal to gdn_chunk_prefill. */
int gdn_chunk_prefill_segmented(const void* q, const void* k, const void* v,
                                const float* log_g, const float* beta, const float* h0,
                                void* out, float* h_final, int B, int T, int Hk, int Hv,
                                int dk, int dv, int chunk, const int32_t* cu_seqlens,
                                int io_dtype, int out_dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

int gdn_chunk_prefill_segmented_plan(const void* q, const void* k, const void* v,
                                     const float* log_g, const float* beta, const float* h0,
                                     void* out, float* h_final, int B, int T, int Hk, int Hv,
                                     int dk, int dv, int chunk, const int32_t* cu_seqlens,
                                     int io_dtype, int out_dtype, void* workspace,
                                     size_t workspace_bytes);

/* ------------------------------------------------------------------------ */
/* Write-on-accept decode verify of K draft rows (the pages' K = 4, and any K
 * in 1..8 from the same chunk algebra), its fold, and the engaged word
 * (ssm_gdn_woa.rs: docs of gdn_decode_wy4_woa, gdn_wy4_fold and
 * gdn_wy4_flag_clear).  Protocol, on one stream: gdn_flag_clear, then
 * gdn_decode_verify (or gdn_decode_verify_k4) (writes outputs and the stash,
 * marks the word, writes NO state), then the caller writes na_tab, then
 * gdn_fold with the same k_rows (if the word is set, applies the first
 * na_tab[b] stashed rows to each state, reading and writing it once).
 *
 * Verify rows: row r (0..K-1) of sequence b is global row b*K + r.
 *   q, k : row at q + (b*K + r)*qk_stride, k-head kh at + kh*dk   (io_dtype)
 *   v    : row at v + (b*K + r)*v_stride,  v-head vh at + vh*dv   (io_dtype)
 *   gate, beta: fp32 at (b*K + r)*gb_stride + vh; gate is log-space like log_g
 *   out  : dense [B][K][Hv][dv] (out_dtype)
 *   h_table[b]: device pointer to sequence b's states [Hv][dk][dv] fp32
 *   stash: sequence b at stash + b*stash_seq_floats; per v-head vh, at
 *          vh*(K*dv + K + kfl) floats: delta [K][dv] fp32, G [K] fp32 (the
 *          within-verify cumulative log decay), then the K keys [K][dk] as
 *          kfl = K*dk floats (fp32 io) or ceil(K*dk/2) floats of packed bf16
 *          bits (bf16 io).  The fold receives no q/k/v/gate, so the stash
 *          carries them.
 *   engaged_flag: one device uint32; verify sets it to 1.
 * Fold:
 *   na_tab: device int32 [B], accepted rows per sequence, clamped to 0..K;
 *           na = 0 leaves the state's bytes unchanged.
 *   hi_tables / slab_entries: the restore branch, for a verify that ran in
 *           parent mode (gdn_decode_verify_parent below, which leaves the
 *           word clear).  NULL: with the word clear the fold changes nothing.
 *           Otherwise, with the word clear, na = na_tab[b] < K puts back
 *           slab na of sequence b (the state after its first na rows) as a
 *           bitwise copy, and na = K keeps the state (which the parent verify
 *           advanced through all K rows); with the word set the slabs are not
 *           read.  slab_entries >= k_rows, else GDN_ERR_SLABS.
 *   k_rows: K of the verify that filled the stash, 1..8.
 * Errors: GDN_ERR_K_ROWS for k_rows outside 1..8; the others as below.
 */
size_t gdn_stash_seq_floats(int Hv, int dk, int dv, int k_rows, int io_dtype);

int gdn_flag_clear(uint32_t* engaged_flag, hipStream_t stream);

int gdn_decode_verify(float* const* h_table, const void* q, const void* k, const void* v,
                      const float* gate, const float* beta, void* out, float* stash,
                      int B, int Hk, int Hv, int dk, int dv, int k_rows,
                      int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                      uint32_t* engaged_flag, int io_dtype, int out_dtype, hipStream_t stream);

/* gdn_decode_verify with k_rows = 4 (the pages' K). */
int gdn_decode_verify_k4(float* const* h_table, const void* q, const void* k, const void* v,
                         const float* gate, const float* beta, void* out, float* stash,
                         int B, int Hk, int Hv, int dk, int dv,
                         int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                         uint32_t* engaged_flag, int io_dtype, int out_dtype, hipStream_t stream);

int gdn_fold(float* const* h_table, const float* stash, const int32_t* na_tab,
             float* const* hi_tables, int slab_entries, const uint32_t* engaged_flag,
             int k_rows, int B, int Hk, int Hv, int dk, int dv, int stash_seq_floats,
             int io_dtype, hipStream_t stream);

/* Parent-mode verify (ssm_gdn_woa.rs, doc of gdn_wy4_fold: when the engaged
 * word is clear "the parent kernel ran, and a partial accept (na < k_rows)
 * restores Hi(na - 1) from hi_tables").  The pages give neither the parent
 * kernel nor the slab layout; this library's reading, with Hi(r) the state
 * after rows 0..r:
 *   - it writes the outputs and the stash exactly as gdn_decode_verify does,
 *     and leaves the engaged word alone (the caller clears it first, so the
 *     fold takes the restore branch);
 *   - it writes slab j = Hi(j - 1), the state after the first j rows, for
 *     j = 0 .. k_rows - 1 (slab 0 is a copy of the state before the verify);
 *   - it advances each state in place to Hi(k_rows - 1), the state after all
 *     k_rows rows (the full accept).
 *   hi_tables: device array [B] of device pointers; slab j of sequence b,
 *           v-head vh, is the [dk][dv] fp32 block at
 *           hi_tables[b] + (j*Hv + vh)*dk*dv floats (slabs laid out as states).
 *   slab_entries: slabs behind each hi_tables[b]; at least k_rows
 *           (GDN_ERR_SLABS otherwise).
 * Every other argument as gdn_decode_verify.  The caller owns the slabs; the
 * library writes slabs 0 .. k_rows - 1 of each sequence and nothing else. */
int gdn_decode_verify_parent(float* const* h_table, float* const* hi_tables, int slab_entries,
                             const void* q, const void* k, const void* v, const float* gate,
                             const float* beta, void* out, float* stash, int B, int Hk, int Hv,
                             int dk, int dv, int k_rows, int qk_stride, int v_stride, int gb_stride,
                             int stash_seq_floats, int io_dtype, int out_dtype, hipStream_t stream);

/* Validation of the calls above without launching (same return codes). */
int gdn_decode_verify_parent_plan(float* const* h_table, float* const* hi_tables, int slab_entries,
                                  const void* q, const void* k, const void* v, const float* gate,
                                  const float* beta, void* out, float* stash, int B, int Hk, int Hv,
                                  int dk, int dv, int k_rows, int qk_stride, int v_stride,
                                  int gb_stride, int stash_seq_floats, int io_dtype, int out_dtype);

int gdn_decode_verify_plan(float* const* h_table, const void* q, const void* k,
                           const void* v, const float* gate, const float* beta, void* out,
                           float* stash, int B, int Hk, int Hv, int dk, int dv, int k_rows,
                           int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                           uint32_t* engaged_flag, int io_dtype, int out_dtype);

int gdn_decode_verify_k4_plan(float* const* h_table, const void* q, const void* k,
                              const void* v, const float* gate, const float* beta, void* out,
                              float* stash, int B, int Hk, int Hv, int dk, int dv,
                              int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                              uint32_t* engaged_flag, int io_dtype, int out_dtype);

int gdn_fold_plan(float* const* h_table, const float* stash, const int32_t* na_tab,
                  float* const* hi_tables, int slab_entries, const uint32_t* engaged_flag,
                  int k_rows, int B, int Hk, int Hv, int dk, int dv, int stash_seq_floats,
                  int io_dtype);

/* ------------------------------------------------------------------------ */
/* Single-token decode step (K = 1), in place: the chunk algebra with L = 1
 * (one row of the token recurrence) applied to each state,
 *   alpha = exp(gate), delta = beta (v - alpha h^T k),
 *   out = alpha h^T q + (q . k) delta,  h <- alpha h + k delta^T,
 * so out is the new state applied to q.  Row b of q, k, v, gate, beta is
 * sequence b's token (layouts as in the verify with K = 1); out is dense
 * [B][Hv][dv]; h_table[b] points at sequence b's states [Hv][dk][dv] fp32,
 * which are read and written once.  dk, dv <= 128, dv a multiple of 4.
 * Returns GDN_OK or one of the GDN_ERR_* codes (nothing launched on error).
 */
int gdn_decode_step(float* const* h_table, const void* q, const void* k, const void* v,
                    const float* gate, const float* beta, void* out,
                    int B, int Hk, int Hv, int dk, int dv,
                    int qk_stride, int v_stride, int gb_stride,
                    int io_dtype, int out_dtype, hipStream_t stream);

int gdn_decode_step_plan(float* const* h_table, const void* q, const void* k, const void* v,
                         const float* gate, const float* beta, void* out,
                         int B, int Hk, int Hv, int dk, int dv,
                         int qk_stride, int v_stride, int gb_stride,
                         int io_dtype, int out_dtype);

/* ------------------------------------------------------------------------ */
/* Gate/beta producer (the BA projection ahead of the recurrence).
 *
 * Follows the launcher of the BA-gates kernels and their index model in
 * ssm_ba_gates_hopper.rs (dense_gemm_ba_gates_prefill_hopper, ba_gates_slot):
 * token t's activation row (input + t*k_stride, k bf16 values) is multiplied
 * by the n = 2*nv weight rows (ba_weight, bf16 [n][k] row-major) in fp32, and
 * output o is placed in the token's fp32 row gate_out + t*gate_stride, laid
 * out [gate(nv) | beta(nv)]: with G = vheads_per_group, group = o / (2G) and
 * w = o % (2G), w < G is beta of v-head group*G + w and w >= G the gate of
 * v-head group*G + (w - G).  The gating, a reading of the a_log and dt_bias
 * arguments (the pages do not print it):
 *     gate = -exp(a_log[vh]) * softplus(y + dt_bias[vh])   (natural log of alpha,
 *                                                            the log_g of the prefill)
 *     beta = 1 / (1 + exp(-y)),   softplus(z) = log(1 + exp(z)).
 * a_log, dt_bias: fp32 [nv].  All pointers are device pointers owned by the
 * caller; gate_out must not overlap the inputs.
 * Shapes: m >= 0 tokens; nv >= 1 with nv % vheads_per_group == 0; n == 2*nv
 * <= 128; k a positive multiple of 64; k_stride >= k and a multiple of 8;
 * gate_stride >= 2*nv; m*k_stride and n*k below 2^30 elements.
 * workspace: device scratch of at least gdn_ba_gates_workspace_bytes(m, n, k)
 * bytes (fp32 partial sums of the k splits; no initialisation needed), used
 * only in the stream's order.
 * Returns GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_HEAD_GROUPS (nv not a
 * multiple of vheads_per_group), GDN_ERR_DIM_LIMIT (n > 128 or k not a multiple
 * of 64), GDN_ERR_STRIDE, GDN_ERR_WORKSPACE or GDN_ERR_HIP; nothing is
 * launched on error.  m = 0 launches nothing and returns GDN_OK.
 */
size_t gdn_ba_gates_workspace_bytes(int m, int n, int k);

int gdn_ba_gates(const void* input, const void* ba_weight, const float* a_log,
                 const float* dt_bias, float* gate_out, int m, int n, int k, int k_stride,
                 int gate_stride, int nv, int vheads_per_group, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

int gdn_ba_gates_plan(const void* input, const void* ba_weight, const float* a_log,
                      const float* dt_bias, float* gate_out, int m, int n, int k, int k_stride,
                      int gate_stride, int nv, int vheads_per_group, void* workspace,
                      size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

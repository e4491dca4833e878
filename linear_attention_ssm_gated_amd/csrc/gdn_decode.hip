// Decode: the write-on-accept verify of K draft rows (K = 1..8, the pages'
// K = 4 among them), its post-verdict fold, the clear of the engaged word
// (ssm_gdn_woa.rs: docs of gdn_decode_wy4_woa, gdn_wy4_fold and
// gdn_wy4_flag_clear), the parent-mode verify with its per-prefix state slabs
// and the fold's restore branch (the same page, doc of gdn_wy4_fold: when the
// word is clear the parent kernel ran, and a partial accept restores
// Hi(na - 1) from hi_tables), and the single-token (K = 1) decode step that
// updates the state in place.
//
// Verify, per (v-head, sequence): the K draft rows are one chunk of the
// chunked form with L = K and start state h0 = *(h_table[b]) + vh*dk*dv:
//   p_s = h0^T k_s,  y_r = h0^T q_r                       (2K reductions over dk)
//   G = cumsum(gate), A_rs = beta_r exp(G_r - G_s) k_r.k_s (s < r)
//   Delta = (I + A)^-1 diag(beta) (V - diag(exp(G)) P)     (KxK forward solve)
//   o_r = exp(G_r) y_r + sum_{s<=r} exp(G_r - G_s) (q_r.k_s) Delta_s
// It writes the outputs and stashes Delta, G and the keys; it writes no state.
// Fold: h <- exp(G_{na-1}) h0 + sum_{s<na} exp(G_{na-1} - G_s) k_s Delta_s^T,
// the state after the first na rows, reading and writing the state once.
// Parent verify: the verify above (outputs and stash, the word left alone),
// then one pass over each state that writes slab j = the state after the
// first j rows (j = 0 .. K-1; slab 0 is the state before the verify) and
// advances the state itself through all K rows:
//   x_r = exp(G_r - G_{r-1}) x_{r-1} + k_r Delta_r^T,  x_{-1} = h0,  G_{-1} = 0.
// Restore (fold, word clear): na < K puts back slab na, a bitwise copy.
// Step (K = 1): the verify and the fold of its one row in one pass,
//   delta = beta (v - alpha h^T k),  o = alpha h^T q + (q.k) delta,
//   h <- alpha h + k delta^T,        alpha = exp(gate).
//
// All of these are HBM-bound (a few flop per state byte): the state is
// streamed once with 16-byte coalesced loads and the dk reductions are split
// over 8 row slices per workgroup.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSlices = 8;      // dk row slices per workgroup
constexpr int kColGroups = 32;  // float4 column groups per slice (dv <= 128)
constexpr int kMaxD = 128;

template <typename TIn>
__device__ __forceinline__ void load_key_row(float* dst, const TIn* src, int n, int tid) {
    for (int i = tid; i < n; i += kThreads) dst[i] = Elem<TIn>::load(src + i);
}

// ---------------------------------------------------------------------------
// Any dk, dv <= 128 (dv a multiple of 4): the correctness path for head sizes
// other than 128.

template <typename TIn, typename TOut, int KR>
__global__ void __launch_bounds__(kThreads)
gdn_verify_kernel(float* const* __restrict__ h_table, const TIn* __restrict__ q,
                  const TIn* __restrict__ k, const TIn* __restrict__ v,
                  const float* __restrict__ gate, const float* __restrict__ beta,
                  TOut* __restrict__ out, float* __restrict__ stash, int Hk, int Hv, int dk, int dv,
                  int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                  uint32_t* __restrict__ engaged_flag)
{
    __shared__ float sk[KR][kMaxD];
    __shared__ float sq[KR][kMaxD];
    __shared__ float sv[KR][kMaxD];
    __shared__ float4 part[kSlices][2 * KR][kColGroups];  // partial p_s, y_r
    __shared__ float sG[KR], sBeta[KR], sA[KR][KR], sQK[KR][KR];

    const int tid = threadIdx.x;
    const int vh = blockIdx.x;
    const int b = blockIdx.y;
    const int kh = vh / (Hv / Hk);

    for (int r = 0; r < KR; ++r) {
        const size_t row = (size_t)b * KR + r;
        load_key_row(sk[r], k + row * qk_stride + (size_t)kh * dk, dk, tid);
        load_key_row(sq[r], q + row * qk_stride + (size_t)kh * dk, dk, tid);
        load_key_row(sv[r], v + row * v_stride + (size_t)vh * dv, dv, tid);
    }
    if (tid < KR) {
        const size_t off = ((size_t)b * KR + tid) * gb_stride + vh;
        sG[tid] = gate[off];
        sBeta[tid] = beta[off];
    }
    __syncthreads();

    // Partial reductions over this thread's dk slice, 4 columns at a time.
    const float* h0 = h_table[b] + (size_t)vh * dk * dv;
    const int cg = tid % kColGroups;
    const int sl = tid / kColGroups;
    const int ncg = dv / 4;
    if (cg < ncg) {
        float4 acc[2 * KR];
#pragma unroll
        for (int m = 0; m < 2 * KR; ++m) acc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = sl; i < dk; i += kSlices) {
            const float4 h = load_global4(h0 + (size_t)i * dv + 4 * cg);
#pragma unroll
            for (int r = 0; r < KR; ++r) {
                const float kk = sk[r][i], qq = sq[r][i];
                acc[r].x += h.x * kk; acc[r].y += h.y * kk; acc[r].z += h.z * kk; acc[r].w += h.w * kk;
                acc[KR + r].x += h.x * qq; acc[KR + r].y += h.y * qq;
                acc[KR + r].z += h.z * qq; acc[KR + r].w += h.w * qq;
            }
        }
#pragma unroll
        for (int m = 0; m < 2 * KR; ++m) part[sl][m][cg] = acc[m];
    }
    // Scalars of the KxK chunk: cumulative decay, A and Q K^T.
    if (tid < KR * KR) {
        const int r = tid / KR, s = tid % KR;
        float kk = 0.f, qk = 0.f;
        if (s <= r)
            for (int i = 0; i < dk; ++i) { kk += sk[r][i] * sk[s][i]; qk += sq[r][i] * sk[s][i]; }
        sA[r][s] = kk;   // raw k_r.k_s for now
        sQK[r][s] = qk;
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < KR; ++r) { acc += sG[r]; sG[r] = acc; }
        for (int r = 0; r < KR; ++r)
            for (int s = 0; s < KR; ++s) {
                const float gam = s <= r ? __expf(sG[r] - sG[s]) : 0.f;
                sA[r][s] = s < r ? sBeta[r] * gam * sA[r][s] : 0.f;
                sQK[r][s] = gam * sQK[r][s];
            }
    }
    __syncthreads();

    // One thread per dv column: finish the reductions, solve, write.
    float* st = stash + (size_t)b * stash_seq_floats +
                (size_t)vh * stash_head_floats(dk, dv, sizeof(TIn) == 2, KR);
    for (int j = tid; j < dv; j += kThreads) {
        float p[KR], y[KR];
        for (int r = 0; r < KR; ++r) { p[r] = 0.f; y[r] = 0.f; }
        const int g = j / 4, c = j % 4;
        for (int s2 = 0; s2 < kSlices; ++s2)
            for (int r = 0; r < KR; ++r) {
                const float4 a = part[s2][r][g], w = part[s2][KR + r][g];
                p[r] += c == 0 ? a.x : c == 1 ? a.y : c == 2 ? a.z : a.w;
                y[r] += c == 0 ? w.x : c == 1 ? w.y : c == 2 ? w.z : w.w;
            }
        float d[KR];
        for (int r = 0; r < KR; ++r) {
            float x = sBeta[r] * (sv[r][j] - __expf(sG[r]) * p[r]);
            for (int m = 0; m < r; ++m) x -= sA[r][m] * d[m];
            d[r] = x;
        }
        for (int r = 0; r < KR; ++r) {
            float o = __expf(sG[r]) * y[r];
            for (int s = 0; s <= r; ++s) o += sQK[r][s] * d[s];
            Elem<TOut>::store(out + (((size_t)b * KR + r) * Hv + vh) * dv + j, o);
            st[r * dv + j] = d[r];
        }
    }
    if (tid < KR) st[KR * dv + tid] = sG[tid];
    float* sk_out = st + KR * dv + KR;
    if (sizeof(TIn) == 2) {
        // keys as packed bf16 bits, exactly as read
        uint16_t* kb = reinterpret_cast<uint16_t*>(sk_out);
        for (int e = tid; e < KR * dk; e += kThreads) {
            const int r = e / dk, i = e % dk;
            kb[e] = *reinterpret_cast<const uint16_t*>(k + ((size_t)b * KR + r) * qk_stride + (size_t)kh * dk + i);
        }
    } else {
        for (int e = tid; e < KR * dk; e += kThreads) sk_out[e] = sk[e / dk][e % dk];
    }
    if (engaged_flag && vh == 0 && b == 0 && tid == 0) engaged_flag[0] = 1u;
}

template <bool kBf16Keys, int KR>
__global__ void __launch_bounds__(kThreads)
gdn_fold_kernel(float* const* __restrict__ h_table, const float* __restrict__ stash,
                const int32_t* __restrict__ na_tab, const uint32_t* __restrict__ engaged_flag,
                int dk, int dv, int stash_seq_floats)
{
    __shared__ float sk[KR][kMaxD];
    __shared__ float sd[KR][kMaxD];
    __shared__ float sc[KR + 1];

    if (engaged_flag[0] == 0u) return;   // the write-on-accept verify did not run
    const int vh = blockIdx.x;
    const int b = blockIdx.y;
    const int na = min(max(na_tab[b], 0), KR);
    if (na == 0) return;                 // nothing accepted: the state is left as it is
    const int tid = threadIdx.x;
    const float* st = stash + (size_t)b * stash_seq_floats + (size_t)vh * stash_head_floats(dk, dv, kBf16Keys, KR);
    for (int e = tid; e < na * dv; e += kThreads) sd[e / dv][e % dv] = st[e];
    const float* sk_in = st + KR * dv + KR;
    for (int e = tid; e < na * dk; e += kThreads) {
        float x;
        if (kBf16Keys) x = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sk_in)[e]);
        else x = sk_in[e];
        sk[e / dk][e % dk] = x;
    }
    if (tid <= na) {
        const float gl = st[KR * dv + na - 1];
        sc[tid] = tid < na ? __expf(gl - st[KR * dv + tid]) : __expf(gl);
    }
    __syncthreads();

    float* h = h_table[b] + (size_t)vh * dk * dv;
    const int ncg = dv / 4;
    const float gam = sc[na];
    for (int e = tid; e < dk * ncg; e += kThreads) {
        const int i = e / ncg, c4 = (e % ncg) * 4;
        float4 x = load_global4(h + (size_t)i * dv + c4);
        x.x *= gam; x.y *= gam; x.z *= gam; x.w *= gam;
        for (int s = 0; s < na; ++s) {
            const float ks = sc[s] * sk[s][i];
            x.x += ks * sd[s][c4]; x.y += ks * sd[s][c4 + 1];
            x.z += ks * sd[s][c4 + 2]; x.w += ks * sd[s][c4 + 3];
        }
        store_global4(h + (size_t)i * dv + c4, x);
    }
}

// K = 1 step, any dk, dv <= 128: two passes over the state (reduce, then
// update in place), with a barrier between them.
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads)
gdn_step_kernel(float* const* __restrict__ h_table, const TIn* __restrict__ q,
                const TIn* __restrict__ k, const TIn* __restrict__ v,
                const float* __restrict__ gate, const float* __restrict__ beta,
                TOut* __restrict__ out, int Hk, int Hv, int dk, int dv, int qk_stride,
                int v_stride, int gb_stride)
{
    __shared__ float sk[kMaxD], sq[kMaxD], sv[kMaxD], sd[kMaxD];
    __shared__ float4 part[kSlices][2][kColGroups];
    __shared__ float skq;

    const int tid = threadIdx.x;
    const int vh = blockIdx.x, b = blockIdx.y;
    const int kh = vh / (Hv / Hk);
    load_key_row(sk, k + (size_t)b * qk_stride + (size_t)kh * dk, dk, tid);
    load_key_row(sq, q + (size_t)b * qk_stride + (size_t)kh * dk, dk, tid);
    load_key_row(sv, v + (size_t)b * v_stride + (size_t)vh * dv, dv, tid);
    const float alpha = __expf(gate[(size_t)b * gb_stride + vh]);
    const float bt = beta[(size_t)b * gb_stride + vh];
    __syncthreads();

    float* h = h_table[b] + (size_t)vh * dk * dv;
    const int cg = tid % kColGroups, sl = tid / kColGroups, ncg = dv / 4;
    if (cg < ncg) {
        float4 p = make_float4(0.f, 0.f, 0.f, 0.f), y = p;
        for (int i = sl; i < dk; i += kSlices) {
            const float4 x = load_global4(h + (size_t)i * dv + 4 * cg);
            const float kk = sk[i], qq = sq[i];
            p.x += x.x * kk; p.y += x.y * kk; p.z += x.z * kk; p.w += x.w * kk;
            y.x += x.x * qq; y.y += x.y * qq; y.z += x.z * qq; y.w += x.w * qq;
        }
        part[sl][0][cg] = p;
        part[sl][1][cg] = y;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int i = 0; i < dk; ++i) a += sq[i] * sk[i];
        skq = a;
    }
    __syncthreads();
    for (int j = tid; j < dv; j += kThreads) {
        float p = 0.f, y = 0.f;
        const int g = j / 4, c = j % 4;
        for (int s2 = 0; s2 < kSlices; ++s2) {
            const float4 a = part[s2][0][g], w = part[s2][1][g];
            p += c == 0 ? a.x : c == 1 ? a.y : c == 2 ? a.z : a.w;
            y += c == 0 ? w.x : c == 1 ? w.y : c == 2 ? w.z : w.w;
        }
        const float d = bt * (sv[j] - alpha * p);
        sd[j] = d;
        Elem<TOut>::store(out + ((size_t)b * Hv + vh) * dv + j, alpha * y + skq * d);
    }
    __syncthreads();
    for (int e = tid; e < dk * ncg; e += kThreads) {
        const int i = e / ncg, c4 = (e % ncg) * 4;
        float4 x = load_global4(h + (size_t)i * dv + c4);
        const float ki = sk[i];
        x.x = alpha * x.x + ki * sd[c4]; x.y = alpha * x.y + ki * sd[c4 + 1];
        x.z = alpha * x.z + ki * sd[c4 + 2]; x.w = alpha * x.w + ki * sd[c4 + 3];
        store_global4(h + (size_t)i * dv + c4, x);
    }
}

// ---------------------------------------------------------------------------
// dk = dv = 128: one workgroup per (v-head, sequence), three per compute
// unit.  Thread t owns rows t/32 + 8 m (m = 0..15) of column group t%32 (4
// columns): a wave's row load covers two adjacent rows (1 KiB) and the
// workgroup's m-th load step the 4 KiB of rows 8m .. 8m+7, so the state is
// read front to back.
//
// While the memory system is saturated, a wave cannot issue a load until the
// queue in front of it drains, so a wave that issues all of its loads first
// sits at the last issue for most of the stream and only then computes.  The
// state loads are therefore software-pipelined: the small rows (keys,
// queries, values, gates) and the first kLookahead state rows go out first,
// and each later step issues row m + kLookahead and then takes row m, so the
// dot products run between issues.  The k.k / q.k products and the KxK
// scalars are formed while the first rows are in flight.  The two row slices
// of a wave are added with a cross-half lane swap, the four wave partials
// through LDS.  The state is read with nontemporal loads (it is read once).
constexpr int kLookahead = 4;       // state rows in flight per thread: verify, fold
constexpr int kLookaheadStep = 8;   // and in the K = 1 step (measured best for each)
// The fold's workgroups per state (each takes 128 / kFoldSplit of its rows):
// the accepted sequences are an uneven share of the grid, and finer
// workgroups spread them evenly over the compute units (measured: 4 beats 1
// and 2 on the B = 16, Hv = 48 fold).
constexpr int kFoldSplit = 4;
constexpr int kD = 128;
constexpr int kKP = kD + 16;    // key rows padded: rows read together fall in different banks
constexpr int kSP = 20;         // keys of slice s at [s][m] = row s + 8 m, padded

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Empty fences that fix the order of the pipelined loads and arithmetic: the
// first keeps memory operations on their side of it, the second makes the
// accumulators complete before it (so their arithmetic cannot sink past the
// next load issue).
__device__ __forceinline__ void mem_fence_here() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void pin(float4& a, float4& b)
{
    asm volatile("" : "+v"(a.x), "+v"(a.y), "+v"(a.z), "+v"(a.w), "+v"(b.x), "+v"(b.y), "+v"(b.z), "+v"(b.w));
}

__device__ __forceinline__ float4 state_row(rsrc_t r, int row, int cg)
{
    const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(
        r, (uint32_t)((row * kD + 4 * cg) * sizeof(float)), 0u, /*nontemporal*/ 2);
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                       __uint_as_float(x.w));
}

__device__ __forceinline__ void state_store(rsrc_t r, int row, int cg, float4 x)
{
    const u32x4v o = {__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)};
    __builtin_amdgcn_raw_buffer_store_b128(o, r, (uint32_t)((row * kD + 4 * cg) * sizeof(float)), 0u,
                                           /*nontemporal*/ 2);
}

__device__ __forceinline__ float4 f4_of(const float* p) { return *reinterpret_cast<const float4*>(p); }

// (q, k, v, gate and beta are not declared __restrict__: the order fences
// then keep their loads ahead of the state's.)
template <typename TIn, typename TOut, int KR>
__global__ void __launch_bounds__(kThreads)
gdn_verify_d128_kernel(float* const* __restrict__ h_table, const TIn* q, const TIn* k,
                       const TIn* v, const float* gate, const float* beta,
                       TOut* __restrict__ out, float* __restrict__ stash, int Hk, int Hv,
                       int qk_stride, int v_stride, int gb_stride, int stash_seq_floats,
                       uint32_t* __restrict__ engaged_flag)
{
    constexpr int D = kD, SP = kSP;
    constexpr int NS = 3 * KR * D;                        // small-row elements
    constexpr int NSU = (NS + kThreads - 1) / kThreads;   // per thread
    __shared__ __attribute__((aligned(16))) float sk[KR][kKP];
    __shared__ __attribute__((aligned(16))) float sq[KR][kKP];
    __shared__ __attribute__((aligned(16))) float sk2[KR][kSlices * SP];
    __shared__ __attribute__((aligned(16))) float sq2[KR][kSlices * SP];
    __shared__ __attribute__((aligned(16))) float sv[KR][D];
    __shared__ float4 part[kThreads / 64][2 * KR][kColGroups];
    __shared__ __attribute__((aligned(16))) float red[2 * KR][D];
    __shared__ float sG[KR], sBeta[KR], sA[KR][KR], sQK[KR][KR];

    const int tid = threadIdx.x;
    const int sl = tid >> 5, cg = tid & 31;
    const int vh = blockIdx.x, b = blockIdx.y;
    const int kh = vh / (Hv / Hk);

    // small rows, as raw elements (widened later): element tid + 256 u of
    // [k | q | v] (KR rows of 128 each; a thread past the end re-reads the
    // last element); every thread reads a gate and a beta so that the loads
    // stay outside any branch
    TIn small[NSU];
#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int idx = min(tid + kThreads * u, NS - 1);
        const int which = idx / (KR * D), r = (idx / D) % KR, i = idx % D;
        const size_t row = (size_t)b * KR + r;
        const TIn* src = which == 0 ? k + row * qk_stride + (size_t)kh * D + i
                       : which == 1 ? q + row * qk_stride + (size_t)kh * D + i
                                    : v + row * v_stride + (size_t)vh * D + i;
        small[u] = *src;
    }
    const size_t goff = ((size_t)b * KR + (tid % KR)) * gb_stride + vh;
    const float g_in = gate[goff], b_in = beta[goff];
    mem_fence_here();
    // the state pointer is read after the small rows are on their way, so
    // that their loads do not wait for it
    float* const hb = h_table[b];
    asm volatile("" ::"s"(hb));
    const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(hb + (size_t)vh * D * D, (short)0,
                                                        D * D * (int)sizeof(float), 0x00020000);

    float4 hv[16];
#pragma unroll
    for (int m = 0; m < kLookahead; ++m) hv[m] = state_row(rs, sl + 8 * m, cg);
    mem_fence_here();

#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int idx = tid + kThreads * u;
        if (NS % kThreads == 0 || idx < NS) {
            const int which = idx / (KR * D), r = (idx / D) % KR, i = idx % D;
            const float x = Elem<TIn>::load(&small[u]);
            const int i2 = (i & 7) * SP + (i >> 3);
            if (which == 2) sv[r][i] = x;
            else if (which == 1) { sq[r][i] = x; sq2[r][i2] = x; }
            else { sk[r][i] = x; sk2[r][i2] = x; }
        }
    }
    if (tid < KR) { sG[tid] = g_in; sBeta[tid] = b_in; }
    __syncthreads();

    // k_r . k_s and q_r . k_s: pair tid/16 (+ 16 per round) sums elements
    // tid%16 + 16 e; the KxK decay-weighted scalars are finished by the
    // lane-0 threads of the pairs
    for (int pr = tid >> 4; pr < KR * KR; pr += kThreads / 16) {
        const int seg = tid & 15, r = pr / KR, s2 = pr % KR;
        float kk = 0.f, qk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = seg + 16 * e;
            const float ks = sk[s2][i];
            kk += sk[r][i] * ks;
            qk += sq[r][i] * ks;
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            kk += __shfl_xor(kk, off, 16);
            qk += __shfl_xor(qk, off, 16);
        }
        if (seg == 0) {
            float Gr = 0.f, Gs = 0.f;
            for (int t = 0; t < KR; ++t) {
                if (t <= r) Gr += sG[t];
                if (t <= s2) Gs += sG[t];
            }
            const float gam = s2 <= r ? __expf(Gr - Gs) : 0.f;
            sA[r][s2] = s2 < r ? sBeta[r] * gam * kk : 0.f;
            sQK[r][s2] = gam * qk;
        }
    }

    // partial h0^T k_r and h0^T q_r over this thread's 16 rows, 4 rows a step,
    // each step first issuing the rows kLookahead ahead
    float4 acc[2 * KR];
#pragma unroll
    for (int m = 0; m < 2 * KR; ++m) acc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e + kLookahead;
            if (m < 16) hv[m] = state_row(rs, sl + 8 * m, cg);
        }
        mem_fence_here();
        float kk[KR][4], qq[KR][4];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const float4 a4 = f4_of(&sk2[r][sl * SP + 4 * m4]);
            const float4 c4 = f4_of(&sq2[r][sl * SP + 4 * m4]);
            kk[r][0] = a4.x; kk[r][1] = a4.y; kk[r][2] = a4.z; kk[r][3] = a4.w;
            qq[r][0] = c4.x; qq[r][1] = c4.y; qq[r][2] = c4.z; qq[r][3] = c4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 h = hv[4 * m4 + e];
#pragma unroll
            for (int r = 0; r < KR; ++r) {
                const float a = kk[r][e], c = qq[r][e];
                acc[r].x += h.x * a; acc[r].y += h.y * a; acc[r].z += h.z * a; acc[r].w += h.w * a;
                acc[KR + r].x += h.x * c; acc[KR + r].y += h.y * c;
                acc[KR + r].z += h.z * c; acc[KR + r].w += h.w * c;
            }
        }
#pragma unroll
        for (int r = 0; r < KR; ++r) pin(acc[r], acc[KR + r]);
    }
    // add the wave's two slices (lanes l and l+32): after the swap, lanes
    // 0..31 hold the k-vector sums (acc 0..KR-1), lanes 32..63 the q-vector sums
    {
        const int hi = (tid >> 5) & 1;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            float* a = &acc[r].x;
            float* c = &acc[KR + r].x;
            float4 s4;
            float* sp = &s4.x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[e]), __float_as_uint(c[e]),
                                                                 false, false);
                sp[e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            part[tid >> 6][hi * KR + r][cg] = s4;
        }
    }
    __syncthreads();

    // sum the 4 wave partials: thread -> (vector tid/32 + 8 per round, column group tid%32)
    for (int vec = tid >> 5; vec < 2 * KR; vec += kThreads / 32) {
        float4 t = part[0][vec][cg];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            const float4 u4 = part[w][vec][cg];
            t.x += u4.x; t.y += u4.y; t.z += u4.z; t.w += u4.w;
        }
        *reinterpret_cast<float4*>(&red[vec][4 * cg]) = t;
    }
    __syncthreads();

    // Outputs and stash: every thread solves column tid%128 (the two halves
    // of the workgroup redundantly) and writes rows half, half + 2, ... of it
    // with buffer stores; lanes with nothing to write use an offset past the
    // range.
    {
        const int j = tid & (D - 1), half = tid >> 7;
        const size_t hs = stash_head_floats(D, D, sizeof(TIn) == 2, KR);
        const size_t row_out = (size_t)Hv * D;   // out elements between rows r and r+1
        const rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            out + ((size_t)b * KR * Hv + vh) * D, (short)0,
            (int)(((KR - 1) * row_out + D) * sizeof(TOut)), 0x00020000);
        const rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
            stash + (size_t)b * stash_seq_floats + (size_t)vh * hs, (short)0, (int)(hs * sizeof(float)),
            0x00020000);
        float G[KR], a = 0.f;
#pragma unroll
        for (int r = 0; r < KR; ++r) { a += sG[r]; G[r] = a; }
        float d[KR], o[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            float x = sBeta[r] * (sv[r][j] - __expf(G[r]) * red[r][j]);
#pragma unroll
            for (int m = 0; m < r; ++m) x -= sA[r][m] * d[m];
            d[r] = x;
        }
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            float y = __expf(G[r]) * red[KR + r][j];
#pragma unroll
            for (int s2 = 0; s2 <= r; ++s2) y += sQK[r][s2] * d[s2];
            o[r] = y;
        }
#pragma unroll
        for (int u = 0; u < (KR + 1) / 2; ++u) {
            // rows 2u (first half) and 2u + 1 (second half)
            const int r = 2 * u + half;
            const float ov = half && 2 * u + 1 < KR ? o[2 * u + 1] : o[2 * u];
            const float dv_ = half && 2 * u + 1 < KR ? d[2 * u + 1] : d[2 * u];
            const bool live = r < KR;
            const uint32_t oo = live ? (uint32_t)((r * row_out + j) * sizeof(TOut)) : 0x7fffffffu;
            const uint32_t so = live ? (uint32_t)((r * D + j) * sizeof(float)) : 0x7fffffffu;
            if (sizeof(TOut) == 2)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(ov), ro, oo, 0u, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, oo, 0u, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dv_), rst, so, 0u, 0);
        }
        // the cumulative log decay G_0..G_{KR-1} (threads 0..KR-1)
        float gsel = G[0];
#pragma unroll
        for (int r = 1; r < KR; ++r) gsel = (tid % KR) == r ? G[r] : gsel;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gsel), rst,
                                              tid < KR ? (uint32_t)((KR * D + tid) * sizeof(float)) : 0x7fffffffu,
                                              0u, 0);
        // the keys, element tid + 256 u of [KR][dk]
        const uint32_t kbase = (uint32_t)((KR * D + KR) * sizeof(float));
#pragma unroll
        for (int u = 0; u < (KR * D + kThreads - 1) / kThreads; ++u) {
            const int e = tid + kThreads * u;
            const int ec = min(e, KR * D - 1), r = ec / D, i = ec % D;
            const float x = sk[r][i];
            const bool live = e < KR * D;
            if (sizeof(TIn) == 2)   // the widened bf16 key: its high half is the bits as read
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(__float_as_uint(x) >> 16), rst,
                                                      live ? kbase + 2u * e : 0x7fffffffu, 0u, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rst,
                                                      live ? kbase + 4u * e : 0x7fffffffu, 0u, 0);
        }
    }
    if (engaged_flag && vh == 0 && b == 0 && tid == 0) engaged_flag[0] = 1u;
}

// dk = dv = 128 fold: laid out like the verify (thread t updates rows
// t/32 + 8 m of column group t%32).  The stash reads (deltas, decays, keys)
// go out first, then the state rows, pipelined kLookahead rows ahead of the
// update; each row is written back as soon as it is updated.  The state is
// read and written with nontemporal accesses.
template <bool kBf16Keys, int KR, int S>
__global__ void __launch_bounds__(kThreads)
gdn_fold_d128_kernel(float* const* __restrict__ h_table, const float* stash,
                     const int32_t* __restrict__ na_tab, const uint32_t* __restrict__ engaged_flag,
                     int stash_seq_floats)
{
    constexpr int D = kD, SP = kSP;
    constexpr int NKU = (KR * D + kThreads - 1) / kThreads;   // key elements per thread
    __shared__ __attribute__((aligned(16))) float sk2[KR][kSlices * SP];

    const int vh = blockIdx.x, b = blockIdx.y;
    constexpr int NM = 16 / S;                   // state rows per thread: this workgroup's share
    static_assert(16 % S == 0 && NM % 4 == 0, "the row loop takes whole groups of four rows per thread");
    constexpr int LA = kLookahead < NM ? kLookahead : NM;
    const int m0 = (int)blockIdx.z * NM;
    // the word, the accept count and the state pointer are independent loads:
    // issue all three before the first branch, so that their latencies overlap
    const uint32_t engaged = engaged_flag[0];
    const int na_in = na_tab[b];
    float* const hb = h_table[b];
    asm volatile("" ::"s"(engaged), "s"(na_in), "s"(hb));   // all three loaded here, one wait
    const int na = min(max(na_in, 0), KR);
    // the write-on-accept verify did not run, or nothing was accepted: the
    // state keeps its bytes
    if (engaged == 0u || na == 0) return;
    const int tid = threadIdx.x;
    const int sl = tid >> 5, cg = tid & 31;
    const float* st = stash + (size_t)b * stash_seq_floats + (size_t)vh * stash_head_floats(D, D, kBf16Keys, KR);
    const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(hb + (size_t)vh * D * D, (short)0,
                                                        D * D * (int)sizeof(float), 0x00020000);

    // stash: this thread's 4 delta columns of every row, the KR decays, and
    // key elements tid + 256 u of [KR][dk]
    float dl[KR][4];
#pragma unroll
    for (int r = 0; r < KR; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) dl[r][c] = st[r * D + 4 * cg + c];
    float G[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) G[r] = st[KR * D + r];
    float kraw[NKU];
#pragma unroll
    for (int u = 0; u < NKU; ++u) {
        const int e = min(tid + kThreads * u, KR * D - 1);
        if (kBf16Keys) kraw[u] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(st + KR * D + KR)[e]);
        else kraw[u] = st[KR * D + KR + e];
    }
    mem_fence_here();

    float4 hv[NM];
#pragma unroll
    for (int m = 0; m < LA; ++m) hv[m] = state_row(rs, sl + 8 * (m0 + m), cg);
    mem_fence_here();

#pragma unroll
    for (int u = 0; u < NKU; ++u) {
        const int e = tid + kThreads * u, r = e / D, i = e % D;
        if ((KR * D) % kThreads == 0 || e < KR * D) sk2[r][(i & 7) * SP + (i >> 3)] = kraw[u];
    }
    // c_s = exp(G_{na-1} - G_s) for the accepted rows, gamma = exp(G_{na-1})
    float gl = G[0];
#pragma unroll
    for (int r = 1; r < KR; ++r) gl = na - 1 == r ? G[r] : gl;
    float cs[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) cs[r] = r < na ? __expf(gl - G[r]) : 0.f;
    const float gam = __expf(gl);
    __syncthreads();

#pragma unroll
    for (int m4 = 0; m4 < NM / 4; ++m4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e + LA;
            if (m < NM) hv[m] = state_row(rs, sl + 8 * (m0 + m), cg);
        }
        mem_fence_here();
        float kk[KR][4];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const float4 a4 = f4_of(&sk2[r][sl * SP + m0 + 4 * m4]);
            kk[r][0] = a4.x; kk[r][1] = a4.y; kk[r][2] = a4.z; kk[r][3] = a4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e;
            float4 x = hv[m];
            x.x *= gam; x.y *= gam; x.z *= gam; x.w *= gam;
#pragma unroll
            for (int s2 = 0; s2 < KR; ++s2) {
                if (s2 < na) {
                    const float ks = cs[s2] * kk[s2][e];
                    x.x += ks * dl[s2][0]; x.y += ks * dl[s2][1]; x.z += ks * dl[s2][2]; x.w += ks * dl[s2][3];
                }
            }
            state_store(rs, sl + 8 * (m0 + m), cg, x);
        }
        mem_fence_here();
    }
}

// dk = dv = 128 step (K = 1): the verify's layout and pipelining for the two
// reductions h^T k and h^T q; the state rows stay in registers until delta is
// known, then each is updated and written back (nontemporal) in place.
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads)
gdn_step_d128_kernel(float* const* __restrict__ h_table, const TIn* q, const TIn* k, const TIn* v,
                     const float* gate, const float* beta, TOut* __restrict__ out, int Hk, int Hv,
                     int qk_stride, int v_stride, int gb_stride)
{
    constexpr int D = kD, SP = kSP;
    constexpr int NS = 3 * D;                             // k, q, v rows
    constexpr int NSU = (NS + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) float sk[D];
    __shared__ __attribute__((aligned(16))) float sq[D];
    __shared__ __attribute__((aligned(16))) float sk2[kSlices * SP];
    __shared__ __attribute__((aligned(16))) float sq2[kSlices * SP];
    __shared__ __attribute__((aligned(16))) float sv[D];
    __shared__ float4 part[kThreads / 64][2][kColGroups];
    __shared__ __attribute__((aligned(16))) float red[2][D];
    __shared__ float skq;

    const int tid = threadIdx.x;
    const int sl = tid >> 5, cg = tid & 31;
    const int vh = blockIdx.x, b = blockIdx.y;
    const int kh = vh / (Hv / Hk);
    const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(h_table[b] + (size_t)vh * D * D, (short)0,
                                                        D * D * (int)sizeof(float), 0x00020000);
    TIn small[NSU];
#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int idx = min(tid + kThreads * u, NS - 1);
        const int which = idx / D, i = idx % D;
        const TIn* src = which == 0 ? k + (size_t)b * qk_stride + (size_t)kh * D + i
                       : which == 1 ? q + (size_t)b * qk_stride + (size_t)kh * D + i
                                    : v + (size_t)b * v_stride + (size_t)vh * D + i;
        small[u] = *src;
    }
    const float g_in = gate[(size_t)b * gb_stride + vh], b_in = beta[(size_t)b * gb_stride + vh];
    mem_fence_here();

    float4 hv[16];
#pragma unroll
    for (int m = 0; m < kLookaheadStep; ++m) hv[m] = state_row(rs, sl + 8 * m, cg);
    mem_fence_here();

#pragma unroll
    for (int u = 0; u < NSU; ++u) {
        const int idx = tid + kThreads * u;
        if (idx < NS) {
            const int which = idx / D, i = idx % D;
            const float x = Elem<TIn>::load(&small[u]);
            const int i2 = (i & 7) * SP + (i >> 3);
            if (which == 2) sv[i] = x;
            else if (which == 1) { sq[i] = x; sq2[i2] = x; }
            else { sk[i] = x; sk2[i2] = x; }
        }
    }
    __syncthreads();
    if (tid < 16) {   // q . k
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += sq[tid + 16 * e] * sk[tid + 16 * e];
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) a += __shfl_xor(a, off, 16);
        if (tid == 0) skq = a;
    }

    float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e + kLookaheadStep;
            if (m < 16) hv[m] = state_row(rs, sl + 8 * m, cg);
        }
        mem_fence_here();
        const float4 a4 = f4_of(&sk2[sl * SP + 4 * m4]);
        const float4 c4 = f4_of(&sq2[sl * SP + 4 * m4]);
        const float kk[4] = {a4.x, a4.y, a4.z, a4.w}, qq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 h = hv[4 * m4 + e];
            acc[0].x += h.x * kk[e]; acc[0].y += h.y * kk[e]; acc[0].z += h.z * kk[e]; acc[0].w += h.w * kk[e];
            acc[1].x += h.x * qq[e]; acc[1].y += h.y * qq[e]; acc[1].z += h.z * qq[e]; acc[1].w += h.w * qq[e];
        }
        pin(acc[0], acc[1]);
    }
    {   // lanes 0..31: h^T k sums, lanes 32..63: h^T q sums
        float4 s4;
        float* sp = &s4.x;
        float* a = &acc[0].x;
        float* c = &acc[1].x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[e]), __float_as_uint(c[e]),
                                                             false, false);
            sp[e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        part[tid >> 6][(tid >> 5) & 1][cg] = s4;
    }
    __syncthreads();
    if (tid < 64) {
        const int vec = tid >> 5;
        float4 t = part[0][vec][cg];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            const float4 u4 = part[w][vec][cg];
            t.x += u4.x; t.y += u4.y; t.z += u4.z; t.w += u4.w;
        }
        *reinterpret_cast<float4*>(&red[vec][4 * cg]) = t;
    }
    __syncthreads();

    const float alpha = __expf(g_in);
    const float4 p4 = f4_of(&red[0][4 * cg]), v4 = f4_of(&sv[4 * cg]);
    float4 d4;
    d4.x = b_in * (v4.x - alpha * p4.x); d4.y = b_in * (v4.y - alpha * p4.y);
    d4.z = b_in * (v4.z - alpha * p4.z); d4.w = b_in * (v4.w - alpha * p4.w);
    if (sl == 0) {
        const float4 y4 = f4_of(&red[1][4 * cg]);
        const float kq = skq;
        TOut* o = out + ((size_t)b * Hv + vh) * D + 4 * cg;
        Elem<TOut>::store(o + 0, alpha * y4.x + kq * d4.x);
        Elem<TOut>::store(o + 1, alpha * y4.y + kq * d4.y);
        Elem<TOut>::store(o + 2, alpha * y4.z + kq * d4.z);
        Elem<TOut>::store(o + 3, alpha * y4.w + kq * d4.w);
    }
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
        const float4 a4 = f4_of(&sk2[sl * SP + 4 * m4]);
        const float kk[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * m4 + e;
            const float4 h = hv[m];
            float4 x;
            x.x = alpha * h.x + kk[e] * d4.x; x.y = alpha * h.y + kk[e] * d4.y;
            x.z = alpha * h.z + kk[e] * d4.z; x.w = alpha * h.w + kk[e] * d4.w;
            state_store(rs, sl + 8 * m, cg, x);
        }
    }
}

__global__ void __launch_bounds__(64) gdn_flag_clear_kernel(uint32_t* flag)
{
    if (threadIdx.x == 0) flag[0] = 0u;
}

// ---------------------------------------------------------------------------
// The parent verify's slabs, from the stash its verify just wrote (row deltas,
// cumulative log decays G, keys): slab j of sequence b, v-head vh, at
// hi_tables[b] + (j Hv + vh) dk dv floats, laid out as the state.  Thread t
// takes float4 column group t % (dv / 4) of rows t / (dv / 4) + m (256 / (dv / 4));
// every state element is read once and written K + 1 times.  Any dk, dv <= 128
// with dv a multiple of 4.
template <bool kBf16Keys, int KR>
__global__ void __launch_bounds__(kThreads)
gdn_slab_kernel(float* const* __restrict__ h_table, float* const* __restrict__ hi_tables,
                const float* __restrict__ stash, int Hv, int dk, int dv, int stash_seq_floats)
{
    __shared__ float sk[KR][kMaxD];
    __shared__ float sd[KR][kMaxD];
    __shared__ float sa[KR];
    const int vh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const float* st = stash + (size_t)b * stash_seq_floats + (size_t)vh * stash_head_floats(dk, dv, kBf16Keys, KR);
    for (int e = tid; e < KR * dv; e += kThreads) sd[e / dv][e % dv] = st[e];
    const float* sk_in = st + KR * dv + KR;
    for (int e = tid; e < KR * dk; e += kThreads) {
        float x;
        if (kBf16Keys) x = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sk_in)[e]);
        else x = sk_in[e];
        sk[e / dk][e % dk] = x;
    }
    // the decay of row r: exp(G_r - G_{r-1}) = exp(gate_r) <= 1
    if (tid < KR) sa[tid] = __expf(st[KR * dv + tid] - (tid > 0 ? st[KR * dv + tid - 1] : 0.f));
    __syncthreads();

    float* h = h_table[b] + (size_t)vh * dk * dv;
    float* slab = hi_tables[b] + (size_t)vh * dk * dv;
    const size_t sstride = (size_t)Hv * dk * dv;
    const int ncg = dv / 4;
    for (int e = tid; e < dk * ncg; e += kThreads) {
        const int i = e / ncg, c4 = (e % ncg) * 4;
        const size_t off = (size_t)i * dv + c4;
        float4 x = load_global4(h + off);
        store_global4(slab + off, x);
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const float a = sa[r], kr = sk[r][i];
            x.x = fmaf(a, x.x, kr * sd[r][c4]);
            x.y = fmaf(a, x.y, kr * sd[r][c4 + 1]);
            x.z = fmaf(a, x.z, kr * sd[r][c4 + 2]);
            x.w = fmaf(a, x.w, kr * sd[r][c4 + 3]);
            if (r + 1 < KR) store_global4(slab + (size_t)(r + 1) * sstride + off, x);
        }
        store_global4(h + off, x);
    }
}

// The fold's restore branch.  With the word clear (the parent verify ran, not
// the write-on-accept one), a partial accept na < K puts back slab na, the
// state after the first na rows, as a bitwise copy; na = K keeps the state,
// which the parent verify advanced through all K rows.  With the word set it
// does nothing (the write-on-accept fold applies the stashed rows).
__global__ void __launch_bounds__(kThreads)
gdn_restore_kernel(float* const* __restrict__ h_table, float* const* __restrict__ hi_tables,
                   const int32_t* __restrict__ na_tab, const uint32_t* __restrict__ engaged_flag,
                   int k_rows, int Hv, int dk, int dv)
{
    const int vh = blockIdx.x, b = blockIdx.y;
    if (engaged_flag[0] != 0u) return;
    const int na = min(max(na_tab[b], 0), k_rows);
    if (na == k_rows) return;
    const float* src = hi_tables[b] + ((size_t)na * Hv + vh) * dk * dv;
    float* dst = h_table[b] + (size_t)vh * dk * dv;
    for (int e = threadIdx.x; e < dk * dv / 4; e += kThreads)
        store_global4(dst + 4 * (size_t)e, load_global4(src + 4 * (size_t)e));
}

// ---- launchers -------------------------------------------------------------

template <typename TIn, typename TOut, int KR>
hipError_t launch_verify_rows(const VerifyArgs& a, hipStream_t s)
{
    if (a.dk == kD && a.dv == kD)
        hipLaunchKernelGGL((gdn_verify_d128_kernel<TIn, TOut, KR>), dim3(a.Hv, a.B), dim3(kThreads), 0, s,
                           a.h_table, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta,
                           (TOut*)a.out, a.stash, a.Hk, a.Hv, a.qk_stride, a.v_stride, a.gb_stride,
                           a.stash_seq_floats, a.engaged_flag);
    else
        hipLaunchKernelGGL((gdn_verify_kernel<TIn, TOut, KR>), dim3(a.Hv, a.B), dim3(kThreads), 0, s,
                           a.h_table, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta,
                           (TOut*)a.out, a.stash, a.Hk, a.Hv, a.dk, a.dv, a.qk_stride, a.v_stride,
                           a.gb_stride, a.stash_seq_floats, a.engaged_flag);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_verify_typed(const VerifyArgs& a, hipStream_t s)
{
    switch (a.k_rows) {
    case 1: return launch_verify_rows<TIn, TOut, 1>(a, s);
    case 2: return launch_verify_rows<TIn, TOut, 2>(a, s);
    case 3: return launch_verify_rows<TIn, TOut, 3>(a, s);
    case 4: return launch_verify_rows<TIn, TOut, 4>(a, s);
    case 5: return launch_verify_rows<TIn, TOut, 5>(a, s);
    case 6: return launch_verify_rows<TIn, TOut, 6>(a, s);
    case 7: return launch_verify_rows<TIn, TOut, 7>(a, s);
    case 8: return launch_verify_rows<TIn, TOut, 8>(a, s);
    default: return hipErrorInvalidValue;   // refused on the host before this point
    }
}

template <bool kBf16Keys, int KR>
hipError_t launch_fold_rows(const FoldArgs& a, hipStream_t s)
{
    if (a.dk == kD && a.dv == kD)
        hipLaunchKernelGGL((gdn_fold_d128_kernel<kBf16Keys, KR, kFoldSplit>), dim3(a.Hv, a.B, kFoldSplit), dim3(kThreads), 0, s,
                           a.h_table, a.stash, a.na_tab, a.engaged_flag, a.stash_seq_floats);
    else
        hipLaunchKernelGGL((gdn_fold_kernel<kBf16Keys, KR>), dim3(a.Hv, a.B), dim3(kThreads), 0, s,
                           a.h_table, a.stash, a.na_tab, a.engaged_flag, a.dk, a.dv, a.stash_seq_floats);
    return hipGetLastError();
}

template <bool kBf16Keys>
hipError_t launch_fold_typed(const FoldArgs& a, hipStream_t s)
{
    switch (a.k_rows) {
    case 1: return launch_fold_rows<kBf16Keys, 1>(a, s);
    case 2: return launch_fold_rows<kBf16Keys, 2>(a, s);
    case 3: return launch_fold_rows<kBf16Keys, 3>(a, s);
    case 4: return launch_fold_rows<kBf16Keys, 4>(a, s);
    case 5: return launch_fold_rows<kBf16Keys, 5>(a, s);
    case 6: return launch_fold_rows<kBf16Keys, 6>(a, s);
    case 7: return launch_fold_rows<kBf16Keys, 7>(a, s);
    case 8: return launch_fold_rows<kBf16Keys, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename TIn, typename TOut>
hipError_t launch_step_typed(const StepArgs& a, hipStream_t s)
{
    if (a.dk == kD && a.dv == kD)
        hipLaunchKernelGGL((gdn_step_d128_kernel<TIn, TOut>), dim3(a.Hv, a.B), dim3(kThreads), 0, s,
                           a.h_table, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta,
                           (TOut*)a.out, a.Hk, a.Hv, a.qk_stride, a.v_stride, a.gb_stride);
    else
        hipLaunchKernelGGL((gdn_step_kernel<TIn, TOut>), dim3(a.Hv, a.B), dim3(kThreads), 0, s,
                           a.h_table, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta,
                           (TOut*)a.out, a.Hk, a.Hv, a.dk, a.dv, a.qk_stride, a.v_stride, a.gb_stride);
    return hipGetLastError();
}

template <bool kBf16Keys, int KR>
hipError_t launch_slab_rows(const ParentArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL((gdn_slab_kernel<kBf16Keys, KR>), dim3(a.v.Hv, a.v.B), dim3(kThreads), 0, s,
                       a.v.h_table, a.hi_tables, a.v.stash, a.v.Hv, a.v.dk, a.v.dv, a.v.stash_seq_floats);
    return hipGetLastError();
}

template <bool kBf16Keys>
hipError_t launch_slab_typed(const ParentArgs& a, hipStream_t s)
{
    switch (a.v.k_rows) {
    case 1: return launch_slab_rows<kBf16Keys, 1>(a, s);
    case 2: return launch_slab_rows<kBf16Keys, 2>(a, s);
    case 3: return launch_slab_rows<kBf16Keys, 3>(a, s);
    case 4: return launch_slab_rows<kBf16Keys, 4>(a, s);
    case 5: return launch_slab_rows<kBf16Keys, 5>(a, s);
    case 6: return launch_slab_rows<kBf16Keys, 6>(a, s);
    case 7: return launch_slab_rows<kBf16Keys, 7>(a, s);
    case 8: return launch_slab_rows<kBf16Keys, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// Static LDS of the kernels above, for the route line.
unsigned verify_lds(int kr, bool d128)
{
    if (d128)
        return (unsigned)(sizeof(float) * (2 * kr * kKP + 2 * kr * kSlices * kSP + kr * kD + 2 * kr * kD +
                                           2 * kr + 2 * kr * kr) +
                          sizeof(float4) * (kThreads / 64) * 2 * kr * kColGroups);
    return (unsigned)(sizeof(float) * (3 * kr * kMaxD + 2 * kr + 2 * kr * kr) +
                      sizeof(float4) * kSlices * 2 * kr * kColGroups);
}

}  // namespace

Geometry verify_geometry(const VerifyArgs& a)
{
    const bool d128 = a.dk == kD && a.dv == kD;
    Geometry g{d128 ? "gdn_verify_d128_kernel" : "gdn_verify_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u},
               kThreads, verify_lds(a.k_rows, d128)};
    return g;
}

Geometry fold_geometry(const FoldArgs& a)
{
    if (a.dk == kD && a.dv == kD) {
        Geometry g{"gdn_fold_d128_kernel", {(unsigned)a.Hv, (unsigned)a.B, (unsigned)kFoldSplit}, kThreads,
                   (unsigned)(sizeof(float) * a.k_rows * kSlices * kSP)};
        return g;
    }
    Geometry g{"gdn_fold_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u}, kThreads,
               (unsigned)(sizeof(float) * (2 * a.k_rows * kMaxD + a.k_rows + 1))};
    return g;
}

Geometry step_geometry(const StepArgs& a)
{
    if (a.dk == kD && a.dv == kD) {
        Geometry g{"gdn_step_d128_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u}, kThreads,
                   (unsigned)(sizeof(float) * (3 * kD + 2 * kSlices * kSP + 2 * kD + 1) +
                              sizeof(float4) * (kThreads / 64) * 2 * kColGroups)};
        return g;
    }
    Geometry g{"gdn_step_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u}, kThreads,
               (unsigned)(sizeof(float) * (4 * kMaxD + 1) + sizeof(float4) * kSlices * 2 * kColGroups)};
    return g;
}

Geometry flag_clear_geometry()
{
    Geometry g{"gdn_flag_clear_kernel", {1u, 1u, 1u}, 64u, 0u};
    return g;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s)
{
    if (a.io_dtype == 0 && a.out_dtype == 0) return launch_verify_typed<float, float>(a, s);
    if (a.io_dtype == 0 && a.out_dtype == 1) return launch_verify_typed<float, uint16_t>(a, s);
    if (a.io_dtype == 1 && a.out_dtype == 0) return launch_verify_typed<uint16_t, float>(a, s);
    return launch_verify_typed<uint16_t, uint16_t>(a, s);
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t s)
{
    return a.io_dtype == 1 ? launch_fold_typed<true>(a, s) : launch_fold_typed<false>(a, s);
}

hipError_t launch_step(const StepArgs& a, hipStream_t s)
{
    if (a.io_dtype == 0 && a.out_dtype == 0) return launch_step_typed<float, float>(a, s);
    if (a.io_dtype == 0 && a.out_dtype == 1) return launch_step_typed<float, uint16_t>(a, s);
    if (a.io_dtype == 1 && a.out_dtype == 0) return launch_step_typed<uint16_t, float>(a, s);
    return launch_step_typed<uint16_t, uint16_t>(a, s);
}

Geometry parent_geometry(const ParentArgs& a)
{
    Geometry g = verify_geometry(a.v);
    g.entry = a.v.dk == kD && a.v.dv == kD ? "gdn_verify_d128_kernel+gdn_slab_kernel" : "gdn_verify_kernel+gdn_slab_kernel";
    return g;
}

Geometry restore_geometry(const FoldArgs& a)
{
    Geometry g{"gdn_restore_kernel", {(unsigned)a.Hv, (unsigned)a.B, 1u}, kThreads, 0u};
    return g;
}

hipError_t launch_parent(const ParentArgs& a, hipStream_t s)
{
    hipError_t e = launch_verify(a.v, s);   // a.v.engaged_flag is NULL: the word is left alone
    if (e != hipSuccess) return e;
    return a.v.io_dtype == 1 ? launch_slab_typed<true>(a, s) : launch_slab_typed<false>(a, s);
}

hipError_t launch_restore(const FoldArgs& a, float* const* hi_tables, hipStream_t s)
{
    hipLaunchKernelGGL(gdn_restore_kernel, dim3(a.Hv, a.B), dim3(kThreads), 0, s, a.h_table, hi_tables,
                       a.na_tab, a.engaged_flag, a.k_rows, a.Hv, a.dk, a.dv);
    return hipGetLastError();
}

hipError_t launch_flag_clear(uint32_t* flag, hipStream_t s)
{
    hipLaunchKernelGGL(gdn_flag_clear_kernel, dim3(1), dim3(64), 0, s, flag);
    return hipGetLastError();
}

}  // namespace gdn

// Generic chunked prefill of the gated delta rule: fp32 arithmetic on fp32 or
// bf16 inputs, any dk, dv <= 128 and chunk <= 64.  It is the route for fp32
// I/O and for shapes the bf16 MFMA spine does not take.
//
// One workgroup walks one (sequence, v-head, 32-column slice of dv) through
// its chunks in order -- the pages' state spine, one workgroup per (v-head,
// batch) (ssm_gdn_tc_route.rs, grid of the tensor-core spine route line),
// split along dv as the SPLIT variants split it (same page, the vtile/vfused
// entry constants).  Columns of the state evolve independently, so the slices
// need no exchange.  Per chunk of L rows with start state h (dk x TV slice):
//   G = cumsum(log_g), gamma = exp(G), Gamma_rs = exp(G_r - G_s) (s <= r)
//   A_rs = beta_r Gamma_rs k_r.k_s (s < r),  P_rs = Gamma_rs q_r.k_s (s <= r)
//   R = diag(beta) (V - diag(gamma) K h)        [= U - W h before the solve]
//   Delta = (I + A)^-1 R                        (forward substitution)
//   O = diag(gamma) Q h + P Delta
//   h <- gamma_L h + sum_s exp(G_L - G_s) k_s Delta_s^T
// Everything stays in LDS in fp32.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxC = 64;
constexpr int kMaxD = 128;
constexpr int kTV = 32;  // dv columns per workgroup

template <typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads)
gdn_prefill_generic_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                           const TIn* __restrict__ v, const float* __restrict__ log_g,
                           const float* __restrict__ beta, const float* h0, TOut* __restrict__ out,
                           float* h_final, int T, int Hk, int Hv, int dk, int dv, int C,
                           const int32_t* __restrict__ cu, int n_tiles)
{
    __shared__ float sK[kMaxC][kMaxD + 1];
    __shared__ float sQ[kMaxC][kMaxD + 1];
    __shared__ float sA[kMaxC][kMaxC + 1];
    __shared__ float sP[kMaxC][kMaxC + 1];
    __shared__ float sH[kMaxD][kTV + 1];
    __shared__ float sV[kMaxC][kTV + 1];
    __shared__ float sX[kMaxC][kTV + 1];   // R, then Delta
    __shared__ float sY[kMaxC][kTV + 1];   // gamma * Q h
    __shared__ float sG[kMaxC];
    __shared__ float sB[kMaxC];
    __shared__ float sE[kMaxC];            // exp(G_L - G_s)

    const int tid = threadIdx.x;
    const int vh = blockIdx.x / n_tiles;
    const int j0 = (blockIdx.x % n_tiles) * kTV;
    const int tv = min(kTV, dv - j0);
    const int b = blockIdx.y;
    const int kh = vh / (Hv / Hk);

    long row0, len;
    if (cu) {
        long a = min(max((long)cu[b], 0L), (long)T);
        long e = min(max((long)cu[b + 1], a), (long)T);
        row0 = a;
        len = e - a;
    } else {
        row0 = (long)b * T;
        len = T;
    }

    const size_t hoff = ((size_t)b * Hv + vh) * (size_t)dk * dv;
    for (int e = tid; e < dk * tv; e += kThreads) {
        int i = e / tv, j = e % tv;
        sH[i][j] = h0 ? h0[hoff + (size_t)i * dv + j0 + j] : 0.0f;
    }

    for (long t0 = 0; t0 < len; t0 += C) {
        const int L = (int)min((long)C, len - t0);
        __syncthreads();  // previous chunk's readers of sK/sQ/sX are done
        for (int e = tid; e < L * dk; e += kThreads) {
            int r = e / dk, i = e % dk;
            size_t off = ((size_t)(row0 + t0 + r) * Hk + kh) * dk + i;
            sK[r][i] = Elem<TIn>::load(k + off);
            sQ[r][i] = Elem<TIn>::load(q + off);
        }
        for (int e = tid; e < L * tv; e += kThreads) {
            int r = e / tv, j = e % tv;
            sV[r][j] = Elem<TIn>::load(v + ((size_t)(row0 + t0 + r) * Hv + vh) * dv + j0 + j);
        }
        if (tid < L) {
            size_t off = (size_t)(row0 + t0 + tid) * Hv + vh;
            sG[tid] = log_g[off];
            sB[tid] = beta[off];
        }
        __syncthreads();
        if (tid == 0) {  // within-chunk cumulative log decay
            float acc = 0.0f;
            for (int r = 0; r < L; ++r) { acc += sG[r]; sG[r] = acc; }
            for (int r = 0; r < L; ++r) sE[r] = __expf(acc - sG[r]);
        }
        __syncthreads();

        // Gram terms A (strictly lower) and P (lower incl. diagonal).
        for (int e = tid; e < L * L; e += kThreads) {
            int r = e / L, s = e % L;
            float a = 0.0f, p = 0.0f;
            if (s <= r) {
                float kk = 0.0f, qk = 0.0f;
                for (int i = 0; i < dk; ++i) {
                    kk += sK[r][i] * sK[s][i];
                    qk += sQ[r][i] * sK[s][i];
                }
                float gam = __expf(sG[r] - sG[s]);
                p = gam * qk;
                if (s < r) a = sB[r] * gam * kk;
            }
            sA[r][s] = a;
            sP[r][s] = p;
        }
        // R = beta (V - gamma K h) and gamma Q h.
        for (int e = tid; e < L * tv; e += kThreads) {
            int r = e / tv, j = e % tv;
            float x = 0.0f, y = 0.0f;
            for (int i = 0; i < dk; ++i) {
                x += sK[r][i] * sH[i][j];
                y += sQ[r][i] * sH[i][j];
            }
            float gam = __expf(sG[r]);
            sX[r][j] = sB[r] * (sV[r][j] - gam * x);
            sY[r][j] = gam * y;
        }
        __syncthreads();

        // Delta = (I + A)^-1 R: one thread per column walks the rows in order.
        if (tid < tv) {
            const int j = tid;
            for (int r = 1; r < L; ++r) {
                float acc = sX[r][j];
                for (int m = 0; m < r; ++m) acc -= sA[r][m] * sX[m][j];
                sX[r][j] = acc;
            }
        }
        __syncthreads();

        // Outputs of the chunk, and the state carried to the next chunk.
        for (int e = tid; e < L * tv; e += kThreads) {
            int r = e / tv, j = e % tv;
            float o = sY[r][j];
            for (int s = 0; s <= r; ++s) o += sP[r][s] * sX[s][j];
            Elem<TOut>::store(out + ((size_t)(row0 + t0 + r) * Hv + vh) * dv + j0 + j, o);
        }
        const float gL = sG[L - 1];
        const float gamL = __expf(gL);
        for (int e = tid; e < dk * tv; e += kThreads) {
            int i = e / tv, j = e % tv;
            float h = gamL * sH[i][j];
            for (int s = 0; s < L; ++s) h += sE[s] * sK[s][i] * sX[s][j];
            sH[i][j] = h;
        }
    }
    __syncthreads();
    if (h_final) {
        for (int e = tid; e < dk * tv; e += kThreads) {
            int i = e / tv, j = e % tv;
            h_final[hoff + (size_t)i * dv + j0 + j] = sH[i][j];
        }
    }
}

template <typename TIn, typename TOut>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t s)
{
    const int n_tiles = (a.dv + kTV - 1) / kTV;
    dim3 grid(a.Hv * n_tiles, a.B);
    hipLaunchKernelGGL((gdn_prefill_generic_kernel<TIn, TOut>), grid, dim3(kThreads), 0, s,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.log_g, a.beta, a.h0,
                       (TOut*)a.out, a.h_final, a.T, a.Hk, a.Hv, a.dk, a.dv, a.chunk,
                       a.cu_seqlens, n_tiles);
    return hipGetLastError();
}

}  // namespace

Geometry prefill_generic_geometry(const PrefillArgs& a)
{
    const int n_tiles = (a.dv + kTV - 1) / kTV;
    Geometry g;
    g.entry = "gdn_prefill_generic_kernel";
    g.grid[0] = (unsigned)(a.Hv * n_tiles);
    g.grid[1] = (unsigned)a.B;
    g.grid[2] = 1;
    g.block = kThreads;
    g.lds_bytes = (unsigned)(sizeof(float) * (2 * kMaxC * (kMaxD + 1) + 2 * kMaxC * (kMaxC + 1) +
                                              kMaxD * (kTV + 1) + 3 * kMaxC * (kTV + 1) + 3 * kMaxC));
    return g;
}

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t s)
{
    if (a.io_dtype == 0 && a.out_dtype == 0) return launch_typed<float, float>(a, s);
    if (a.io_dtype == 0 && a.out_dtype == 1) return launch_typed<float, uint16_t>(a, s);
    if (a.io_dtype == 1 && a.out_dtype == 0) return launch_typed<uint16_t, float>(a, s);
    return launch_typed<uint16_t, uint16_t>(a, s);
}

}  // namespace gdn

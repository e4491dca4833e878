// bf16 MFMA chunked prefill for dk = dv = 128, chunk = 64 (gfx950).
//
// Two kernels on the caller's stream:
//
// gdn_wy_prep_kernel, one workgroup per (chunk, v-head), all chunks at once:
//   the intra-chunk terms that do not depend on the state (the pages' W/U
//   producer behind the spine, ssm_gdn_tc_route.rs, doc of the pipe spine):
//     G = cumsum(log_g), Gamma_rs = exp(G_r - G_s) for s <= r
//     A = strict_lower(diag(beta) (Gamma o K K^T)),  T = (I + A)^-1
//     P = lower_incl(Gamma o Q K^T)
//   K K^T and Q K^T run on bf16 MFMA with fp32 accumulation; T is solved in
//   fp32 (16x16 diagonal blocks by forward substitution on VALU, the blocks
//   below them on fp32 MFMA); T and P are stored as bf16 in the workspace.
//
// gdn_spine_kernel, one workgroup per (sequence, v-head, 32 dv columns), two
//   waves of 16 columns each, walking the chunks in order: the state spine
//   (same page, the tensor-core spine: bf16 MFMA operands, the fp32
//   accumulators are the recurrent state, h stays f32).  Per chunk:
//     X = K h, Y = Q h                       (state as the bf16 B operand)
//     R = diag(beta) (V - diag(gamma) X)
//     Delta = T R                            (= U - W h of the WY form)
//     O = diag(gamma) Y + P Delta
//     h <- gamma_L h + K^T diag(exp(G_L - G)) Delta
//   Columns of h evolve independently (the dv split of the pages' SPLIT
//   variants), so the waves never exchange data.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16, 64 lanes, lane = 16 g + i):
// the hardware pairs element e of A in lane 16g+m with element e of B in lane
// 16g+n and sums over (g, e).  We assign the 32 k indices of one k-step as
//     k(g, e) = 4g + e        for e < 4
//     k(g, e) = 16 + 4g + e-4 for e >= 4
// so that a 16x16 fp32 accumulator tile (lane 16g+n holds rows 4g..4g+3 of
// column n) of two consecutive k-blocks IS a B operand after rounding to bf16,
// and an A operand is two 8-byte LDS reads of its row.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;        // chunk rows
constexpr int D = 128;       // dk = dv
constexpr int LDK = D + 8;   // LDS row stride (bf16) of K and Q
constexpr int LDC = C + 8;   // LDS row stride (bf16) of T, P and K^T
constexpr int LDF = C + 4;   // LDS row stride (fp32) of A and the fp32 T
constexpr int TILE_COLS = 32;            // dv columns per spine workgroup
constexpr int N_TILES = D / TILE_COLS;   // 4
constexpr int SLOT_ELEMS = 2 * C * C;    // T then P, bf16, per (chunk, v-head)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// A operand of one 32-wide k-step: row `row` of a bf16 LDS matrix, columns
// k0 + 4g .. +3 and k0 + 16 + 4g .. +3.
__device__ __forceinline__ s16x8 frag_a(const uint16_t* base, int ld, int row, int k0, int g) {
    const uint16_t* p = base + row * ld + k0 + 4 * g;
    s16x4 lo = *reinterpret_cast<const s16x4*>(p);
    s16x4 hi = *reinterpret_cast<const s16x4*>(p + 16);
    return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ short bf16_bits(float x) {
    return (short)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// B operand from two accumulator tiles of consecutive k-blocks.
__device__ __forceinline__ s16x8 frag_b(f32x4 lo, f32x4 hi) {
    return s16x8{bf16_bits(lo[0]), bf16_bits(lo[1]), bf16_bits(lo[2]), bf16_bits(lo[3]),
                 bf16_bits(hi[0]), bf16_bits(hi[1]), bf16_bits(hi[2]), bf16_bits(hi[3])};
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Rows of sequence b: [row0, row0 + len).
__device__ __forceinline__ void seq_rows(const int32_t* cu, int b, int T, long* row0, long* len) {
    if (cu) {
        long a = min(max((long)cu[b], 0L), (long)T);
        long e = min(max((long)cu[b + 1], a), (long)T);
        *row0 = a;
        *len = e - a;
    } else {
        *row0 = (long)b * T;
        *len = T;
    }
}

// ---------------------------------------------------------------------------
// Chunk table for packed sequences: base[b] = sum_{b' < b} ceil(len_b' / C).
__global__ void __launch_bounds__(256)
gdn_chunk_table_kernel(const int32_t* __restrict__ cu, int B, int T, int32_t* __restrict__ base)
{
    __shared__ int32_t part[256];
    const int tid = threadIdx.x;
    const int per = (B + 255) / 256;
    const int b0 = tid * per, b1 = min(B, b0 + per);
    int32_t s = 0;
    for (int b = b0; b < b1; ++b) {
        long r0, len;
        seq_rows(cu, b, T, &r0, &len);
        s += (int32_t)((len + C - 1) / C);
    }
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int i = 0; i < 256; ++i) { int32_t v = part[i]; part[i] = acc; acc += v; }
        base[B] = acc;
    }
    __syncthreads();
    s = part[tid];
    for (int b = b0; b < b1; ++b) {
        base[b] = s;
        long r0, len;
        seq_rows(cu, b, T, &r0, &len);
        s += (int32_t)((len + C - 1) / C);
    }
}

// Loads rows [row0, row0 + L) of one head of a [rows][H][128] bf16 tensor into
// a [C][LDK] LDS tile, zero-filling rows >= L.  256 or 128 threads.
template <int NT>
__device__ __forceinline__ void load_rows_128(uint16_t* dst, const uint16_t* src, long row0, int L,
                                              int H, int head, int tid)
{
    for (int idx = tid; idx < C * (D / 8); idx += NT) {
        const int r = idx >> 4, c8 = (idx & 15) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < L) v = *reinterpret_cast<const uint4*>(src + ((size_t)(row0 + r) * H + head) * D + c8);
        *reinterpret_cast<uint4*>(dst + r * LDK + c8) = v;
    }
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
gdn_wy_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const float* __restrict__ log_g, const float* __restrict__ beta,
                   uint16_t* __restrict__ slots, int B, int T, int Hk, int Hv,
                   const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_base,
                   int nc_dense)
{
    __shared__ __attribute__((aligned(16))) uint16_t sK[C * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[C * LDK];
    __shared__ __attribute__((aligned(16))) float sA[C * LDF];
    __shared__ __attribute__((aligned(16))) float sT[C * LDF];
    __shared__ __attribute__((aligned(16))) uint16_t sP[C * LDC];
    __shared__ float sG[C], sB[C];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int x = blockIdx.x, vh = blockIdx.y;
    const int kh = vh / (Hv / Hk);

    // which sequence and chunk this workgroup serves
    int b, c;
    if (!cu) {
        b = x / nc_dense;
        c = x % nc_dense;
    } else {
        if (x >= chunk_base[B]) return;   // beyond the last chunk
        int lo = 0, hi = B - 1;  // last b with chunk_base[b] <= x
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (chunk_base[mid] <= x) lo = mid; else hi = mid - 1;
        }
        b = lo;
        c = x - chunk_base[b];
    }
    long row0, len;
    seq_rows(cu, b, T, &row0, &len);
    row0 += (long)c * C;
    const int L = (int)min((long)C, len - (long)c * C);

    load_rows_128<256>(sK, k, row0, L, Hk, kh, tid);
    load_rows_128<256>(sQ, q, row0, L, Hk, kh, tid);
    for (int e = tid; e < C * LDF; e += 256) sT[e] = 0.f;
    if (w == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < L) {
            gv = log_g[(size_t)(row0 + lane) * Hv + vh];
            bv = beta[(size_t)(row0 + lane) * Hv + vh];
        }
        sG[lane] = wave_inclusive_sum(gv, lane);
        sB[lane] = bv;
    }
    __syncthreads();

    // K K^T -> A (fp32, strictly lower, beta_r Gamma_rs folded in) and
    // Q K^T -> P (bf16, lower incl. diagonal); 16x16 tiles, 20 lower ones.
    for (int t = w; t < 32; t += 4) {
        const bool is_kk = t < 16;
        const int tt = t & 15;
        const int rb = tt >> 2, cb = tt & 3;
        if (cb > rb) {
            if (!is_kk)  // upper P tiles are zero
                for (int r = 0; r < 4; ++r) sP[(16 * rb + 4 * g + r) * LDC + 16 * cb + n] = 0;
            continue;
        }
        const uint16_t* a_src = is_kk ? sK : sQ;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            acc = mfma_bf16(frag_a(a_src, LDK, 16 * rb + n, 32 * kk, g),
                            frag_a(sK, LDK, 16 * cb + n, 32 * kk, g), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * g + r, col = 16 * cb + n;
            if (is_kk) {
                sA[row * LDF + col] = col < row ? sB[row] * __expf(sG[row] - sG[col]) * acc[r] : 0.f;
            } else {
                const float p = col <= row ? __expf(sG[row] - sG[col]) * acc[r] : 0.f;
                sP[row * LDC + col] = __builtin_bit_cast(uint16_t, (__bf16)p);
            }
        }
    }
    __syncthreads();

    // T_ii = (I + A_ii)^-1 for the four 16x16 diagonal blocks: wave w, lane j
    // walks column j of block w by forward substitution.
    if (lane < 16) {
        const int j = lane, o = 16 * w;
        float xcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xcol[r] = r == j ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) s += sA[(o + r) * LDF + o + m] * xcol[m];
            if (r > j) xcol[r] = -s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(o + r) * LDF + o + j] = xcol[r];
    }
    __syncthreads();

    // Blocks below the diagonal, by distance d:  T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
    for (int d = 1; d < 4; ++d) {
        if (w < 4 - d) {
            const int i = w + d, j = w;
            f32x4 acc = zero4();
            for (int m = j; m < i; ++m)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = mfma_f32(sA[(16 * i + n) * LDF + 16 * m + 4 * s + g],
                                   sT[(16 * m + 4 * s + g) * LDF + 16 * j + n], acc);
            // acc (lane 16g+n, reg r) holds M[4g + r][n]; use it as the B operand
            // with k = 4g + s at step s.
            f32x4 t = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s)
                t = mfma_f32(sT[(16 * i + n) * LDF + 16 * i + 4 * g + s], acc[s], t);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * g + r) * LDF + 16 * j + n] = -t[r];
        }
        __syncthreads();
    }

    // Store T then P as bf16 rows of 64.
    uint16_t* dstT = slots + ((size_t)x * Hv + vh) * SLOT_ELEMS;
    uint16_t* dstP = dstT + C * C;
    for (int idx = tid; idx < C * C / 8; idx += 256) {
        const int r = idx >> 3, c8 = (idx & 7) * 8;
        s16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_bits(sT[r * LDF + c8 + e]);
        *reinterpret_cast<s16x8*>(dstT + r * C + c8) = v;
        *reinterpret_cast<uint4*>(dstP + r * C + c8) = *reinterpret_cast<const uint4*>(sP + r * LDC + c8);
    }
}

// ---------------------------------------------------------------------------
template <bool kOutF32>
__global__ void __launch_bounds__(128)
gdn_spine_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const float* __restrict__ log_g,
                 const float* __restrict__ beta, const float* h0, void* __restrict__ out,
                 float* h_final, const uint16_t* __restrict__ slots, int T, int Hk, int Hv,
                 const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_base,
                 int nc_dense, long n_slots)
{
    __shared__ __attribute__((aligned(16))) uint16_t sK[C * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[C * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[D * LDC];
    __shared__ __attribute__((aligned(16))) uint16_t sT[C * LDC];
    __shared__ __attribute__((aligned(16))) uint16_t sP[C * LDC];
    __shared__ __attribute__((aligned(16))) uint16_t sV[C * (TILE_COLS + 8)];
    __shared__ float sGam[C], sEL[C], sB[C];
    __shared__ float sGamL;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int vh = blockIdx.x / N_TILES;
    const int tile = blockIdx.x % N_TILES;
    const int b = blockIdx.y;
    const int kh = vh / (Hv / Hk);
    const int col = tile * TILE_COLS + 16 * w + n;   // this lane's dv column

    long row0, len;
    seq_rows(cu, b, T, &row0, &len);
    const long slot0 = cu ? (long)chunk_base[b] : (long)b * nc_dense;
    const int nc = (int)((len + C - 1) / C);

    // the state: h[16 db + 4 g + r][col] in acc tile db, register r
    f32x4 h[8];
    const size_t hoff = ((size_t)b * Hv + vh) * D * D;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            h[db][r] = h0 ? h0[hoff + (size_t)(16 * db + 4 * g + r) * D + col] : 0.f;

    for (int c = 0; c < nc; ++c) {
        // Only reachable when cu_seqlens decreases somewhere (a broken
        // precondition): never read past the workspace.  Uniform per workgroup.
        if (slot0 + c >= n_slots) break;
        const long r0 = row0 + (long)c * C;
        const int L = (int)min((long)C, len - (long)c * C);
        __syncthreads();  // the previous chunk is done with the LDS tiles

        // K (both layouts), Q, V columns of this workgroup, T, P
        for (int idx = tid; idx < C * (D / 8); idx += 128) {
            const int r = idx >> 4, c8 = (idx & 15) * 8;
            uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
            if (r < L) {
                const size_t off = ((size_t)(r0 + r) * Hk + kh) * D + c8;
                kv = *reinterpret_cast<const uint4*>(k + off);
                qv = *reinterpret_cast<const uint4*>(q + off);
            }
            *reinterpret_cast<uint4*>(sK + r * LDK + c8) = kv;
            *reinterpret_cast<uint4*>(sQ + r * LDK + c8) = qv;
            const uint16_t* ke = reinterpret_cast<const uint16_t*>(&kv);
#pragma unroll
            for (int e = 0; e < 8; ++e) sKt[(c8 + e) * LDC + r] = ke[e];
        }
        const uint16_t* slot = slots + ((size_t)(slot0 + c) * Hv + vh) * SLOT_ELEMS;
        for (int idx = tid; idx < C * C / 8; idx += 128) {
            const int r = idx >> 3, c8 = (idx & 7) * 8;
            *reinterpret_cast<uint4*>(sT + r * LDC + c8) = *reinterpret_cast<const uint4*>(slot + r * C + c8);
            *reinterpret_cast<uint4*>(sP + r * LDC + c8) = *reinterpret_cast<const uint4*>(slot + C * C + r * C + c8);
        }
        for (int idx = tid; idx < C * (TILE_COLS / 8); idx += 128) {
            const int r = idx >> 2, c8 = (idx & 3) * 8;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (r < L) vv = *reinterpret_cast<const uint4*>(v + ((size_t)(r0 + r) * Hv + vh) * D + tile * TILE_COLS + c8);
            *reinterpret_cast<uint4*>(sV + r * (TILE_COLS + 8) + c8) = vv;
        }
        if (w == 0) {
            float gv = 0.f, bv = 0.f;
            if (lane < L) {
                gv = log_g[(size_t)(r0 + lane) * Hv + vh];
                bv = beta[(size_t)(r0 + lane) * Hv + vh];
            }
            const float G = wave_inclusive_sum(gv, lane);
            const float GL = __shfl(G, 63, 64);
            sGam[lane] = __expf(G);
            sEL[lane] = __expf(GL - G);
            sB[lane] = bv;
            if (lane == 0) sGamL = __expf(GL);
        }
        __syncthreads();

        // X = K h and Y = Q h for this wave's 16 columns
        s16x8 hb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) hb[kk] = frag_b(h[2 * kk], h[2 * kk + 1]);
        f32x4 X[4], Y[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            X[cb] = zero4();
            Y[cb] = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                X[cb] = mfma_bf16(frag_a(sK, LDK, 16 * cb + n, 32 * kk, g), hb[kk], X[cb]);
                Y[cb] = mfma_bf16(frag_a(sQ, LDK, 16 * cb + n, 32 * kk, g), hb[kk], Y[cb]);
            }
        }
        // R = beta (V - gamma X), in place
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * cb + 4 * g + r;
                const float vv = bf16_bits_to_f32(sV[row * (TILE_COLS + 8) + 16 * w + n]);
                X[cb][r] = sB[row] * (vv - sGam[row] * X[cb][r]);
                Y[cb][r] *= sGam[row];
            }
        const s16x8 rb0 = frag_b(X[0], X[1]), rb1 = frag_b(X[2], X[3]);
        // Delta = T R (T is lower triangular: rows < 32 need only k < 32)
        f32x4 Dl[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            Dl[cb] = mfma_bf16(frag_a(sT, LDC, 16 * cb + n, 0, g), rb0, zero4());
            if (cb >= 2) Dl[cb] = mfma_bf16(frag_a(sT, LDC, 16 * cb + n, 32, g), rb1, Dl[cb]);
        }
        const s16x8 db0 = frag_b(Dl[0], Dl[1]), db1 = frag_b(Dl[2], Dl[3]);
        // O = gamma Y + P Delta, written for the rows of the chunk
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 o = mfma_bf16(frag_a(sP, LDC, 16 * cb + n, 0, g), db0, Y[cb]);
            if (cb >= 2) o = mfma_bf16(frag_a(sP, LDC, 16 * cb + n, 32, g), db1, o);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * cb + 4 * g + r;
                if (row < L) {
                    const size_t off = ((size_t)(r0 + row) * Hv + vh) * D + col;
                    if (kOutF32) reinterpret_cast<float*>(out)[off] = o[r];
                    else reinterpret_cast<uint16_t*>(out)[off] = f32_to_bf16_bits(o[r]);
                }
            }
        }
        // h <- gamma_L h + K^T (exp(G_L - G) Delta)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Dl[cb][r] *= sEL[16 * cb + 4 * g + r];
        const s16x8 ds0 = frag_b(Dl[0], Dl[1]), ds1 = frag_b(Dl[2], Dl[3]);
        const float gl = sGamL;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            f32x4 acc = h[db] * gl;
            acc = mfma_bf16(frag_a(sKt, LDC, 16 * db + n, 0, g), ds0, acc);
            acc = mfma_bf16(frag_a(sKt, LDC, 16 * db + n, 32, g), ds1, acc);
            h[db] = acc;
        }
    }

    if (h_final) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h_final[hoff + (size_t)(16 * db + 4 * g + r) * D + col] = h[db][r];
    }
}

size_t table_bytes(int B) { return ((size_t)(B + 1) * sizeof(int32_t) + 255) & ~(size_t)255; }

long slot_count(int B, int T, bool packed) {
    return packed ? (long)(T + C - 1) / C + B : (long)B * ((T + C - 1) / C);
}

}  // namespace

size_t prefill_mfma_workspace_bytes(int B, int T, int Hv, bool packed)
{
    return table_bytes(B) + (size_t)slot_count(B, T, packed) * Hv * SLOT_ELEMS * sizeof(uint16_t);
}

bool prefill_mfma_accepts(const PrefillArgs& a)
{
    return a.io_dtype == 1 && a.dk == D && a.dv == D && a.chunk == C;
}

Geometry prefill_mfma_geometry(const PrefillArgs& a)
{
    Geometry g{"gdn_wy_prep_kernel+gdn_spine_kernel", {(unsigned)(a.Hv * N_TILES), (unsigned)a.B, 1u}, 128u,
               (unsigned)(sizeof(uint16_t) * (2 * C * LDK + D * LDC + 2 * C * LDC + C * (TILE_COLS + 8)) +
                          sizeof(float) * (3 * C + 1))};
    return g;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s)
{
    const bool packed = a.cu_seqlens != nullptr;
    int32_t* base = reinterpret_cast<int32_t*>(a.workspace);
    uint16_t* slots = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(a.workspace) + table_bytes(a.B));
    const int nc_dense = (a.T + C - 1) / C;
    const long n_slots = slot_count(a.B, a.T, packed);
    if (packed) {
        hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.B, a.T, base);
    }
    if (n_slots > 0) {
        hipLaunchKernelGGL(gdn_wy_prep_kernel, dim3((unsigned)n_slots, a.Hv), dim3(256), 0, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, a.log_g, a.beta, slots, a.B,
                           a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense);
    }
    dim3 grid(a.Hv * N_TILES, a.B);
    if (a.out_dtype == 0)
        hipLaunchKernelGGL((gdn_spine_kernel<true>), grid, dim3(128), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, slots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense, n_slots);
    else
        hipLaunchKernelGGL((gdn_spine_kernel<false>), grid, dim3(128), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, slots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense, n_slots);
    return hipGetLastError();
}

}  // namespace gdn

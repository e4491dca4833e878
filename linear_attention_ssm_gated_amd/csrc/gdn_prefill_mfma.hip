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
// LDS row strides.  A fragment read is 16 lanes x 8 bytes from 16 consecutive
// rows; rows that start 8 bytes apart modulo 128 put those 16 reads on
// distinct banks, so bf16 rows are padded by 4 elements (8 bytes).
constexpr int LDK = D + 4;   // LDS row stride (bf16) of K and Q: 264 bytes
constexpr int LDC = C + 4;   // LDS row stride (bf16) of T, P, K^T and V^T: 136 bytes
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

// 16 bytes to an LDS row that is only 8-byte aligned.
__device__ __forceinline__ void store16(uint16_t* dst, const uint4& v) {
    reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
    reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
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
// One workgroup per (chunk, k-head): K K^T and Q K^T once, then for each
// v-head of the group its decay, A, T and P.
__global__ void __launch_bounds__(256)
gdn_wy_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const float* __restrict__ log_g, const float* __restrict__ beta,
                   uint16_t* __restrict__ slots, int B, int T, int Hk, int Hv,
                   const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_base,
                   int nc_dense)
{
    // K and Q (bf16) while the Grams are formed; afterwards the same bytes
    // hold A and T (fp32) of the v-head being solved.
    constexpr size_t kRaw = 2 * C * LDF * sizeof(float) > 2 * C * LDK * sizeof(uint16_t)
                                ? 2 * C * LDF * sizeof(float) : 2 * C * LDK * sizeof(uint16_t);
    __shared__ __attribute__((aligned(16))) unsigned char sRaw[kRaw];
    __shared__ __attribute__((aligned(16))) float sKK[C * LDF];
    __shared__ __attribute__((aligned(16))) float sQK[C * LDF];
    __shared__ float sG[C], sB[C];
    uint16_t* sK = reinterpret_cast<uint16_t*>(sRaw);
    uint16_t* sQ = sK + C * LDK;
    float* sA = reinterpret_cast<float*>(sRaw);
    float* sT = sA + C * LDF;
    static_assert(2 * C * LDF * sizeof(float) <= sizeof(sRaw), "A and T must fit where K and Q were");

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int x = blockIdx.x, kh = blockIdx.y;
    const int G = Hv / Hk;

    int b, c;
    if (!cu) {
        b = x / nc_dense;
        c = x % nc_dense;
    } else {
        if (x >= chunk_base[B]) return;   // beyond the last chunk
        int lo = 0, hi = B - 1;           // last b with chunk_base[b] <= x
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

    {   // K and Q rows, all loads in flight before any store
        uint4 kr[4], qr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
            kr[i] = qr[i] = make_uint4(0, 0, 0, 0);
            if (r < L) {
                const size_t off = ((size_t)(row0 + r) * Hk + kh) * D + c8;
                kr[i] = *reinterpret_cast<const uint4*>(k + off);
                qr[i] = *reinterpret_cast<const uint4*>(q + off);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
            store16(sK + r * LDK + c8, kr[i]);
            store16(sQ + r * LDK + c8, qr[i]);
        }
    }
    __syncthreads();

    // raw Grams, lower 16x16 tiles (diagonal tiles whole)
    for (int t = w; t < 20; t += 4) {
        const bool is_kk = t < 10;
        int tt = is_kk ? t : t - 10, rb = 0;
        while (tt > rb) { tt -= rb + 1; ++rb; }
        const int cb = tt;
        const uint16_t* a_src = is_kk ? sK : sQ;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            acc = mfma_bf16(frag_a(a_src, LDK, 16 * rb + n, 32 * kk, g),
                            frag_a(sK, LDK, 16 * cb + n, 32 * kk, g), acc);
        float* dst = is_kk ? sKK : sQK;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * rb + 4 * g + r) * LDF + 16 * cb + n] = acc[r];
    }
    __syncthreads();

    for (int gi = 0; gi < G; ++gi) {
        const int vh = kh * G + gi;
        if (w == 0) {
            float gv = 0.f, bv = 0.f;
            if (lane < L) {
                gv = log_g[(size_t)(row0 + lane) * Hv + vh];
                bv = beta[(size_t)(row0 + lane) * Hv + vh];
            }
            sG[lane] = wave_inclusive_sum(gv, lane);
            sB[lane] = bv;
        } else {
            for (int e = tid - 64; e < C * LDF; e += 192) sT[e] = 0.f;
        }
        __syncthreads();

        uint16_t* dstT = slots + ((size_t)x * Hv + vh) * SLOT_ELEMS;
        uint16_t* dstP = dstT + C * C;
        // A (fp32, LDS) and P (bf16, straight to the workspace), 8 entries per step
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, r = idx >> 3, s0 = (idx & 7) * 8;
            const float gr = sG[r], br = sB[r];
            s16x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                // upper-triangle Gram entries were never written: select, never multiply
                const float gam = s <= r ? __expf(gr - sG[s]) : 0.f;
                sA[r * LDF + s] = s < r ? br * gam * sKK[r * LDF + s] : 0.f;
                pv[e] = s <= r ? bf16_bits(gam * sQK[r * LDF + s]) : (short)0;
            }
            *reinterpret_cast<s16x8*>(dstP + r * C + s0) = pv;
        }
        __syncthreads();

        // T_ii = (I + A_ii)^-1: wave w, lane j walks column j of block w.
        if (lane < 16) {
            const int j = lane, o = 16 * w;
            float xc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) xc[r] = r == j ? 1.f : 0.f;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                const float4* arow = reinterpret_cast<const float4*>(sA + (o + r) * LDF + o);
                float a[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 t4 = arow[q4];
                    a[4 * q4] = t4.x; a[4 * q4 + 1] = t4.y; a[4 * q4 + 2] = t4.z; a[4 * q4 + 3] = t4.w;
                }
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s += a[m] * xc[m];
                if (r > j) xc[r] = -s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(o + r) * LDF + o + j] = xc[r];
        }
        __syncthreads();

        // blocks below the diagonal, by distance d: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
        for (int d = 1; d < 4; ++d) {
            if (w < 4 - d) {
                const int i = w + d, j = w;
                f32x4 acc = zero4();
                for (int m = j; m < i; ++m)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc = mfma_f32(sA[(16 * i + n) * LDF + 16 * m + 4 * s + g],
                                       sT[(16 * m + 4 * s + g) * LDF + 16 * j + n], acc);
                // acc (lane 16g+n, reg r) = M[4g + r][n]: the B operand with k = 4g + s at step s
                f32x4 t = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    t = mfma_f32(sT[(16 * i + n) * LDF + 16 * i + 4 * g + s], acc[s], t);
#pragma unroll
                for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * g + r) * LDF + 16 * j + n] = -t[r];
            }
            __syncthreads();
        }

#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, r = idx >> 3, c8 = (idx & 7) * 8;
            s16x8 tv;
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[e] = bf16_bits(sT[r * LDF + c8 + e]);
            *reinterpret_cast<s16x8*>(dstT + r * C + c8) = tv;
        }
        __syncthreads();   // sG, sA and sT are rewritten by the next v-head
    }
}

// ---------------------------------------------------------------------------
// Operands of one chunk for the spine, as the compute waves read them.
struct alignas(16) SpineBuf {
    uint16_t K[C * LDK];        // K, row-major (A operand of K h)
    uint16_t Q[C * LDK];        // Q, row-major (A operand of Q h)
    uint16_t Kt[D * LDC];       // K^T (A operand of K^T Delta)
    uint16_t T[C * LDC];        // (I + A)^-1
    uint16_t P[C * LDC];        // lower_incl(Gamma o Q K^T)
    uint16_t Vt[TILE_COLS * LDC];  // this workgroup's 32 columns of V, transposed
    float gam[C];               // exp(G_r)
    float el[C];                // exp(G_L - G_r)
    float beta[C];
    float gamL;                 // exp(G_L)
};

// One chunk's worth of global data in a loader thread's registers.
struct SpineRegs {
    uint4 k[8], q[8], t[4], p[4], v[2];
    float g = 0.f, b = 0.f;
};

// Buffer resources (gfx9 family): a wave-uniform base in SGPRs, 32-bit lane
// byte offsets, and a byte range; reads beyond the range return 0 and writes
// beyond it are dropped, which is how partial chunks are masked.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4f(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Per-thread byte offsets of the loader's fetches within one chunk.
struct LoaderOffsets {
    uint32_t kq, kq_row;   // row 8 rb + i of K and Q at kq + i * kq_row
    uint32_t tp[4];        // T pieces (P at + C*C*2)
    uint32_t v[2];
    uint32_t gb;           // log_g / beta of row lt (first loader wave)
};

__device__ __forceinline__ LoaderOffsets loader_offsets(int lt, int Hk, int Hv)
{
    LoaderOffsets o;
    const int rb = lt >> 4, cb = lt & 15;
    o.kq_row = (uint32_t)Hk * D * 2u;
    o.kq = (uint32_t)(8 * rb) * o.kq_row + (uint32_t)(8 * cb) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = lt + 128 * i;
        o.tp[i] = (uint32_t)((idx >> 3) * C + (idx & 7) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = lt + 128 * i;
        o.v[i] = (uint32_t)(idx >> 2) * Hv * D * 2u + (uint32_t)((idx & 3) * 8) * 2u;
    }
    o.gb = (uint32_t)(lt & 63) * Hv * 4u;
    return o;
}

// Two loader waves (128 threads, lt = 0..127) fetch one chunk into registers;
// every load is issued before any is used.  Rows >= L read as zero.
__device__ __forceinline__ void spine_fetch(SpineRegs& R, const LoaderOffsets& o, rsrc_t rk,
                                            rsrc_t rq, rsrc_t rv, rsrc_t rg, rsrc_t rb_,
                                            rsrc_t rs, int lt)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        R.k[i] = buf_load16(rk, o.kq + i * o.kq_row);
        R.q[i] = buf_load16(rq, o.kq + i * o.kq_row);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        R.t[i] = buf_load16(rs, o.tp[i]);
        R.p[i] = buf_load16(rs, o.tp[i] + C * C * 2);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) R.v[i] = buf_load16(rv, o.v[i]);
    if (lt < 64) {   // wave-uniform
        R.g = buf_load4f(rg, o.gb);
        R.b = buf_load4f(rb_, o.gb);
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// Halves e of two packed bf16 words: (lo's, hi's) as one word.
__device__ __forceinline__ uint32_t pair_half(uint32_t lo, uint32_t hi, int e) {
    return (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
}

// Stores a fetched chunk into `sb`: K, Q and T, P rows as they are; K^T by
// transposing each thread's 8x8 block in registers; V transposed element-wise.
__device__ __forceinline__ void spine_store(SpineBuf& sb, const SpineRegs& R, int lt)
{
    const int rb = lt >> 4, cb = lt & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        store16(sb.K + (8 * rb + i) * LDK + 8 * cb, R.k[i]);
        store16(sb.Q + (8 * rb + i) * LDK + 8 * cb, R.q[i]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {   // column e of the block = row 8 cb + e of K^T
        uint4 o;
        o.x = pair_half(word_of(R.k[0], e >> 1), word_of(R.k[1], e >> 1), e);
        o.y = pair_half(word_of(R.k[2], e >> 1), word_of(R.k[3], e >> 1), e);
        o.z = pair_half(word_of(R.k[4], e >> 1), word_of(R.k[5], e >> 1), e);
        o.w = pair_half(word_of(R.k[6], e >> 1), word_of(R.k[7], e >> 1), e);
        store16(sb.Kt + (8 * cb + e) * LDC + 8 * rb, o);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = lt + 128 * i, r = idx >> 3, c8 = (idx & 7) * 8;
        store16(sb.T + r * LDC + c8, R.t[i]);
        store16(sb.P + r * LDC + c8, R.p[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = lt + 128 * i, r = idx >> 2, c8 = (idx & 3) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t wv = word_of(R.v[i], e >> 1);
            sb.Vt[(c8 + e) * LDC + r] = (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xffffu));
        }
    }
    if (lt < 64) {   // wave-uniform: the first loader wave
        const float Gr = wave_inclusive_sum(R.g, lt);
        const float GL = __shfl(Gr, 63, 64);
        sb.gam[lt] = __expf(Gr);
        sb.el[lt] = __expf(GL - Gr);
        sb.beta[lt] = R.b;
        if (lt == 0) sb.gamL = __expf(GL);
    }
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// One compute wave, one chunk, 16 columns (wave w of the workgroup).  LDS
// fragment reads are issued one group ahead of the MFMAs that consume them,
// so that a single wave per SIMD does not wait out each read's latency.
template <bool kOutF32>
__device__ __forceinline__ void spine_step(const SpineBuf& sb, f32x4 (&h)[8], void* __restrict__ out,
                                           long r0, int L, int Hv, int vh, int col, int w, int g, int n)
{
    s16x8 hb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) hb[kk] = frag_b(h[2 * kk], h[2 * kk + 1]);

    // X = K h, Y = Q h: 4 k-steps x 8 independent accumulators
    f32x4 X[4], Y[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) X[cb] = Y[cb] = zero4();
    s16x8 fa[8], fb[8];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        fa[cb] = frag_a(sb.K, LDK, 16 * cb + n, 0, g);
        fa[4 + cb] = frag_a(sb.Q, LDK, 16 * cb + n, 0, g);
    }
    float4 gm4[4], bt4[4], el4[4];
    uint2 vv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        s16x8 (&cur)[8] = (kk & 1) ? fb : fa;
        s16x8 (&nxt)[8] = (kk & 1) ? fa : fb;
        if (kk < 3) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                nxt[cb] = frag_a(sb.K, LDK, 16 * cb + n, 32 * (kk + 1), g);
                nxt[4 + cb] = frag_a(sb.Q, LDK, 16 * cb + n, 32 * (kk + 1), g);
            }
        } else {
            // per-row scalars of the next phases, and the first T fragments
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int row = 16 * cb + 4 * g;
                gm4[cb] = *reinterpret_cast<const float4*>(sb.gam + row);
                bt4[cb] = *reinterpret_cast<const float4*>(sb.beta + row);
                el4[cb] = *reinterpret_cast<const float4*>(sb.el + row);
                vv[cb] = *reinterpret_cast<const uint2*>(sb.Vt + (16 * w + n) * LDC + row);
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) nxt[cb] = frag_a(sb.T, LDC, 16 * cb + n, 0, g);
            nxt[4] = frag_a(sb.T, LDC, 32 + n, 32, g);
            nxt[5] = frag_a(sb.T, LDC, 48 + n, 32, g);
        }
        sched_fence();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            X[cb] = mfma_bf16(cur[cb], hb[kk], X[cb]);
            Y[cb] = mfma_bf16(cur[4 + cb], hb[kk], Y[cb]);
        }
        sched_fence();
    }
    s16x8 (&ft)[8] = fa;   // T fragments (the last k-step's "next" buffer)

    // R = beta (V - gamma X) in place of X; gamma Y in place of Y
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float gmr[4] = {gm4[cb].x, gm4[cb].y, gm4[cb].z, gm4[cb].w};
        const float btr[4] = {bt4[cb].x, bt4[cb].y, bt4[cb].z, bt4[cb].w};
        const float vr[4] = {bf16_bits_to_f32((uint16_t)(vv[cb].x & 0xffffu)), bf16_bits_to_f32((uint16_t)(vv[cb].x >> 16)),
                             bf16_bits_to_f32((uint16_t)(vv[cb].y & 0xffffu)), bf16_bits_to_f32((uint16_t)(vv[cb].y >> 16))};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            X[cb][r] = btr[r] * (vr[r] - gmr[r] * X[cb][r]);
            Y[cb][r] *= gmr[r];
        }
    }
    const s16x8 rb0 = frag_b(X[0], X[1]), rb1 = frag_b(X[2], X[3]);

    // Delta = T R (T lower triangular: rows < 32 need only k < 32); meanwhile
    // fetch the first half of the K^T fragments
    s16x8 fk[8];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        fk[2 * db] = frag_a(sb.Kt, LDC, 16 * db + n, 0, g);
        fk[2 * db + 1] = frag_a(sb.Kt, LDC, 16 * db + n, 32, g);
    }
    sched_fence();
    f32x4 Dl[4];
    Dl[0] = mfma_bf16(ft[0], rb0, zero4());
    Dl[1] = mfma_bf16(ft[1], rb0, zero4());
    Dl[2] = mfma_bf16(ft[2], rb0, zero4());
    Dl[3] = mfma_bf16(ft[3], rb0, zero4());
    Dl[2] = mfma_bf16(ft[4], rb1, Dl[2]);
    Dl[3] = mfma_bf16(ft[5], rb1, Dl[3]);
    sched_fence();
    const s16x8 db0 = frag_b(Dl[0], Dl[1]), db1 = frag_b(Dl[2], Dl[3]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        Dl[cb][0] *= el4[cb].x; Dl[cb][1] *= el4[cb].y;
        Dl[cb][2] *= el4[cb].z; Dl[cb][3] *= el4[cb].w;
    }
    const s16x8 ds0 = frag_b(Dl[0], Dl[1]), ds1 = frag_b(Dl[2], Dl[3]);

    // h <- gamma_L h + K^T (exp(G_L - G) Delta): two groups of 4 row blocks
    const float gl = sb.gamL;
    s16x8 fk2[8];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        fk2[2 * db] = frag_a(sb.Kt, LDC, 16 * (db + 4) + n, 0, g);
        fk2[2 * db + 1] = frag_a(sb.Kt, LDC, 16 * (db + 4) + n, 32, g);
    }
    sched_fence();
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        f32x4 acc = h[db] * gl;
        acc = mfma_bf16(fk[2 * db], ds0, acc);
        h[db] = mfma_bf16(fk[2 * db + 1], ds1, acc);
    }
    sched_fence();
    s16x8 fp[6];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) fp[cb] = frag_a(sb.P, LDC, 16 * cb + n, 0, g);
    fp[4] = frag_a(sb.P, LDC, 32 + n, 32, g);
    fp[5] = frag_a(sb.P, LDC, 48 + n, 32, g);
    sched_fence();
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        f32x4 acc = h[db + 4] * gl;
        acc = mfma_bf16(fk2[2 * db], ds0, acc);
        h[db + 4] = mfma_bf16(fk2[2 * db + 1], ds1, acc);
    }
    sched_fence();

    // O = gamma Y + P Delta, for the rows of the chunk
    f32x4 O[4];
    O[0] = mfma_bf16(fp[0], db0, Y[0]);
    O[1] = mfma_bf16(fp[1], db0, Y[1]);
    O[2] = mfma_bf16(fp[2], db0, Y[2]);
    O[3] = mfma_bf16(fp[3], db0, Y[3]);
    O[2] = mfma_bf16(fp[4], db1, O[2]);
    O[3] = mfma_bf16(fp[5], db1, O[3]);
    // hardware RNE conversion; stores through a buffer resource covering the
    // chunk's L rows, so rows beyond a partial chunk are dropped
    constexpr uint32_t es = kOutF32 ? 4u : 2u;
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)r0);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r0 >> 32));
    const size_t ru = ((size_t)rhi << 32) | rlo;
    const rsrc_t ro = make_rsrc(reinterpret_cast<char*>(out) + (ru * Hv + vh) * D * es,
                                __builtin_amdgcn_readfirstlane((uint32_t)L * Hv * D * es));
    const uint32_t rs = (uint32_t)Hv * D * es;
    const uint32_t lane_off = (uint32_t)(4 * g) * rs + (uint32_t)col * es;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = lane_off + (uint32_t)(16 * cb + r) * rs;
            const float val = O[cb][r];   // by value: never bit-cast a vector element in place
            if (kOutF32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_bits(val), ro, off, 0, 0);
        }
}

// Chunk c of the sequence at rows [row0, row0 + len): its buffer resources
// (rows beyond the chunk read as 0), fetched into the loader's registers.
__device__ __forceinline__ void spine_fetch_chunk(SpineRegs& R, const LoaderOffsets& lo,
                                                  const uint16_t* q, const uint16_t* k,
                                                  const uint16_t* v, const float* log_g,
                                                  const float* beta, const uint16_t* slot_base,
                                                  size_t slot_stride, long row0, long len, int c,
                                                  int Hk, int Hv, int kh, int vh, int tile, int lt)
{
    // all of these are wave-uniform; say so, so the resources live in SGPRs
    const long r = row0 + (long)c * C;
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)r);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r >> 32));
    const size_t ru = ((size_t)rhi << 32) | rlo;
    const uint32_t L = __builtin_amdgcn_readfirstlane((uint32_t)min((long)C, len - (long)c * C));
    spine_fetch(R, lo, make_rsrc(k + (ru * Hk + kh) * D, L * Hk * D * 2u),
                make_rsrc(q + (ru * Hk + kh) * D, L * Hk * D * 2u),
                make_rsrc(v + (ru * Hv + vh) * D + tile * TILE_COLS, L * Hv * D * 2u),
                make_rsrc(log_g + ru * Hv + vh, L * Hv * 4u), make_rsrc(beta + ru * Hv + vh, L * Hv * 4u),
                make_rsrc(slot_base + (size_t)c * slot_stride, SLOT_ELEMS * 2u), lt);
}

// One workgroup per (sequence, v-head, 32 dv columns): waves 0-1 compute
// (16 columns each, state in registers), waves 2-3 keep the next chunk in
// LDS and the one after it in registers.
template <bool kOutF32>
__global__ void __launch_bounds__(256)
gdn_spine_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const float* __restrict__ log_g,
                 const float* __restrict__ beta, const float* h0, void* __restrict__ out,
                 float* h_final, const uint16_t* __restrict__ slots, int T, int Hk, int Hv,
                 const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_base,
                 int nc_dense, long n_slots)
{
    __shared__ SpineBuf buf[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    // Workgroup i runs on XCD i % 8.  Map the grid so that the workgroups of
    // one k-head (its v-heads and column tiles) share an XCD and its L2.
    const int W = gridDim.x;
    const int lin = (W % 8 == 0) ? (blockIdx.x % 8) * (W / 8) + blockIdx.x / 8 : blockIdx.x;
    const int vh = lin / N_TILES;
    const int tile = lin % N_TILES;
    const int b = blockIdx.y;
    const int kh = vh / (Hv / Hk);
    const int col = tile * TILE_COLS + 16 * (w & 1) + n;   // compute lane's dv column

    long row0, len;
    seq_rows(cu, b, T, &row0, &len);
    const long slot0 = cu ? (long)chunk_base[b] : (long)b * nc_dense;
    int nc = (int)((len + C - 1) / C);
    // Only a decreasing cu_seqlens (a broken precondition) can make this
    // bind; it keeps every read inside the workspace.
    if (slot0 + nc > n_slots) nc = (int)max(0L, n_slots - slot0);
    auto rows_of = [&](int c) { return (int)min((long)C, len - (long)c * C); };

    f32x4 h[8];
    const size_t hoff = ((size_t)b * Hv + vh) * D * D;
    const uint16_t* slot_base = slots + ((size_t)slot0 * Hv + vh) * SLOT_ELEMS;
    const size_t slot_stride = (size_t)Hv * SLOT_ELEMS;
    const int lt = tid - 128;
    SpineRegs R;
    LoaderOffsets lo;
    if (w < 2) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[db][r] = h0 ? h0[hoff + (size_t)(16 * db + 4 * g + r) * D + col] : 0.f;
    } else if (nc > 0) {
        lo = loader_offsets(lt, Hk, Hv);
        spine_fetch_chunk(R, lo, q, k, v, log_g, beta, slot_base, slot_stride, row0, len, 0, Hk, Hv,
                          kh, vh, tile, lt);
        spine_store(buf[0], R, lt);
        if (nc > 1)
            spine_fetch_chunk(R, lo, q, k, v, log_g, beta, slot_base, slot_stride, row0, len, 1, Hk,
                              Hv, kh, vh, tile, lt);
    }
    __syncthreads();

    for (int c = 0; c < nc; ++c) {
        if (w < 2) {
            spine_step<kOutF32>(buf[c & 1], h, out, row0 + (long)c * C, rows_of(c), Hv, vh, col, w, g, n);
        } else if (c + 1 < nc) {
            spine_store(buf[(c + 1) & 1], R, lt);       // chunk c + 1, fetched last iteration
            if (c + 2 < nc)
                spine_fetch_chunk(R, lo, q, k, v, log_g, beta, slot_base, slot_stride, row0, len, c + 2,
                                  Hk, Hv, kh, vh, tile, lt);
        }
        __syncthreads();
    }

    if (w < 2 && h_final) {
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
    Geometry g{"gdn_wy_prep_kernel+gdn_spine_kernel", {(unsigned)(a.Hv * N_TILES), (unsigned)a.B, 1u}, 256u,
               (unsigned)(2 * sizeof(SpineBuf))};
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
        hipLaunchKernelGGL(gdn_wy_prep_kernel, dim3((unsigned)n_slots, a.Hk), dim3(256), 0, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, a.log_g, a.beta, slots, a.B,
                           a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense);
    }
    dim3 grid(a.Hv * N_TILES, a.B);
    if (a.out_dtype == 0)
        hipLaunchKernelGGL((gdn_spine_kernel<true>), grid, dim3(256), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, slots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense, n_slots);
    else
        hipLaunchKernelGGL((gdn_spine_kernel<false>), grid, dim3(256), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, slots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense, n_slots);
    return hipGetLastError();
}

}  // namespace gdn

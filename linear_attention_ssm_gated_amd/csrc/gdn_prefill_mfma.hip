// bf16 MFMA chunked prefill for dk = dv = 128, chunk = 64 (gfx950).
//
// Two kernels on the caller's stream:
//
// gdn_wy_prep_kernel, one workgroup per (chunk, k-head), all chunks at once:
//   the intra-chunk terms that do not depend on the state (the pages' W/U
//   producer behind the spine, ssm_gdn_tc_route.rs, doc of the pipe spine):
//     G = cumsum(log_g), Gamma_rs = exp(G_r - G_s) for s <= r
//     A = strict_lower(diag(beta) (Gamma o K K^T)),  T = (I + A)^-1   (per v-head)
//     S = lower_incl(Q K^T)                                            (per k-head)
//   K K^T and Q K^T run on bf16 MFMA with fp32 accumulation; T is solved in
//   fp32 (16x16 diagonal blocks by forward substitution on VALU, the blocks
//   below them on fp32 MFMA); T and S are stored as bf16 in the workspace,
//   their granules above the diagonal left unwritten (they are zero, and the
//   spine never reads them from memory).  The output's decay-weighted
//   P = Gamma o S is never formed: Gamma_rs = gm_r / gm_s with gm = exp(G)
//   factors out of the product (see the spine).
//
// gdn_spine_kernel, one workgroup per (sequence, v-head, 32 dv columns), two
//   waves of 16 columns each, walking the chunks in order: the state spine
//   (same page, the tensor-core spine: bf16 MFMA operands, the fp32
//   accumulators are the recurrent state, h stays f32).  Per chunk:
//     X = K h, Y = Q h                       (state as the bf16 B operand)
//     R = diag(beta) (V - diag(gamma) X)
//     Delta = T R                            (= U - W h of the WY form)
//     O = diag(gamma) Y + (Gamma o S) Delta
//       = diag(gamma / gamma_L) (gamma_L Y + S (el o Delta)),  el = exp(G_L - G)
//     h <- gamma_L h + K^T (el o Delta)
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
constexpr int TILE_COLS = 32;            // dv columns per spine workgroup
constexpr int N_TILES = D / TILE_COLS;   // 4
constexpr int SLOT_ELEMS = C * C;        // one 64 x 64 bf16 matrix: T per (chunk, v-head), S per (chunk, k-head)

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
// With at most MAX_ORDERED sequences, order[] (after base[B]) lists them by
// chunk count, longest first (ties by index): the spine walks sequence
// order[y] in workgroup row y, so the longest walks are dispatched first and
// the short ones fill in behind them.
constexpr int MAX_ORDERED = 256;
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
    if (B <= MAX_ORDERED) {   // one sequence per thread (per == 1)
        int32_t mine = 0;        // this sequence's chunk count
        if (tid < B) {
            long r0, len;
            seq_rows(cu, tid, T, &r0, &len);
            mine = (int32_t)((len + C - 1) / C);
        }
        __syncthreads();         // every read of the prefix sums is done
        part[tid] = mine;
        __syncthreads();
        if (tid < B) {
            int rank = 0;
            for (int j = 0; j < B; ++j) {
                const int32_t o = part[j];
                rank += (o > mine || (o == mine && j < tid)) ? 1 : 0;
            }
            base[B + 1 + rank] = tid;
        }
    }
}

// ---------------------------------------------------------------------------
// Buffer resources (gfx9 family): a wave-uniform base in SGPRs, 32-bit lane
// and SGPR byte offsets, and a byte range.  On gfx950 the range check covers
// both offsets: reads beyond the range return 0 and writes beyond it are
// dropped, which is how partial chunks are masked.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x8 buffer_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return __builtin_bit_cast(s16x8, v);
}

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// data (a compiler fence: the hardware keeps one wave's LDS operations in
// order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Buffer->LDS DMA, written as inline assembly: the compiler would otherwise
// make later LDS reads wait for every DMA in flight.  Completion is tracked
// by hand (wait_vmcnt).  The range check that zero-fills rows beyond a chunk
// covers the lane offset and the SGPR offset alike.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct Rsrc { u32x4 d; };
__device__ __forceinline__ Rsrc make_dma_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    Rsrc r;
    r.d = u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
    return r;
}
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}
__device__ __forceinline__ void dma16(const Rsrc& r, unsigned char* lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"((uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(lds))), "v"(voff), "s"(r.d),
                    "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const Rsrc& r, unsigned char* lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"((uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(lds))), "v"(voff), "s"(r.d) : "memory", "m0");
}
__device__ __forceinline__ s16x8 lds_read16(const unsigned char* p) {
    return *reinterpret_cast<const s16x8*>(p);
}
// ---------------------------------------------------------------------------
// WY prep: one workgroup per (chunk, k-head, group of up to four of its
// v-heads), one wave per v-head.  The workgroup stages the chunk's K and Q
// rows in LDS once; each wave then forms, for its v-head,
//   A = strict_lower(beta_r exp(G_r - G_s) (K K^T)_rs),   T = (I + A)^-1,
// and writes T as a bf16 64 x 64 row-major matrix to the (chunk, v-head)
// slot.  The k-head's S = lower_incl(Q K^T) (no decay) is written once, its
// ten 16 x 16 tiles shared out over the first group's waves.  The waves never
// wait for each other after the staging.
//
// Gram tiles are formed above the diagonal, tile (m, i) = K_m K_i^T and
// K_m Q_i^T (16-row blocks, m <= i), so that lane (g, n) register s holds
// the entry of row 16 i + n, column 16 m + 4g + s of K K^T and of Q K^T: the
// decay factor of both is the same, a P tile leaves as four consecutive bf16
// of one row, and an off-diagonal A tile is directly the A operand of an
// fp32 MFMA whose k-slot of lane group g at step s is 4g + s.
//
// T is formed on 16 x 16 fp32 blocks: T_ii = (I + A_ii)^-1 by forward
// substitution, then T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj by distance
// i - j.  Block row r is stored at slot p(r) = 4 (r/4) + ((r + r/4) % 4) and
// element c at c ^ 4 (r/4), so that the rows 4g + s that one MFMA operand or
// accumulator register spans fall in four different 16-bank windows.  The
// four diagonal blocks start at floats 272 i (four windows again), the six
// below the diagonal after them.  A diagonal block holds A_ii transposed
// until T_ii replaces it.
__host__ __device__ constexpr int prow(int r) { return 4 * (r >> 2) + ((r + (r >> 2)) & 3); }
__host__ __device__ constexpr int blk_elem(int r, int c) { return 16 * prow(r) + (c ^ (4 * (r >> 2))); }
__host__ __device__ constexpr int t_blk(int i, int j) {
    return i == j ? 272 * i : 1088 + 256 * ((i - 1) * i / 2 + j);
}
constexpr int PREP_WAVE_FLOATS = 1088 + 6 * 256;          // per wave, over the K/Q staging
constexpr int PREP_STAGE_BYTES = 2 * C * D * 2;           // K then Q, 256-byte rows
// K/Q staging: granule q of row r at q ^ (r % 8), so that a fragment read (8
// lanes, 8 consecutive rows, one granule) is free of bank conflicts.  After
// the larger of the staging area and the per-wave regions come G log2(e) and
// beta per row for each wave.
__host__ __device__ constexpr int prep_gb_base(int nw) {   // floats
    return PREP_STAGE_BYTES / 4 > nw * PREP_WAVE_FLOATS ? PREP_STAGE_BYTES / 4 : nw * PREP_WAVE_FLOATS;
}
__host__ __device__ constexpr size_t prep_lds_bytes(int nw) {
    return (size_t)(prep_gb_base(nw) + nw * 2 * C) * sizeof(float);
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP: shifts within
// rows of 16 lanes, then each row adds the last lane of the rows before it.
__device__ __forceinline__ float wave_scan_dpp(float x) {
#define GDN_DPP_ADD(ctrl, rmask) \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rmask, 0xf, false))
    GDN_DPP_ADD(0x111, 0xf);   // row_shr:1
    GDN_DPP_ADD(0x112, 0xf);   // row_shr:2
    GDN_DPP_ADD(0x114, 0xf);   // row_shr:4
    GDN_DPP_ADD(0x118, 0xf);   // row_shr:8
    GDN_DPP_ADD(0x142, 0xa);   // row_bcast:15 into rows 1 and 3
    GDN_DPP_ADD(0x143, 0xc);   // row_bcast:31 into rows 2 and 3
#undef GDN_DPP_ADD
    return x;
}

extern __shared__ __attribute__((aligned(1024))) float prep_lds[];

__global__ void __launch_bounds__(256, 3)
gdn_wy_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const float* __restrict__ log_g, const float* __restrict__ beta,
                   uint16_t* __restrict__ tslots, uint16_t* __restrict__ sslots, int B, int T,
                   int Hk, int Hv, const int32_t* __restrict__ cu,
                   const int32_t* __restrict__ chunk_base, int nc_dense)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), nw = blockDim.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int x = blockIdx.x, kh = blockIdx.y;
    const int G = Hv / Hk;
    const int h = blockIdx.z * nw + w;   // this wave's v-head within the k-head
    const int vh = kh * G + h;
    float* lds = prep_lds + w * PREP_WAVE_FLOATS;
    float* sG = prep_lds + prep_gb_base(nw) + w * 2 * C;   // G log2(e) per row
    float* sBt = sG + C;                                        // beta per row

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
    const uint32_t L = __builtin_amdgcn_readfirstlane((uint32_t)min((long)C, len - (long)c * C));
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)row0);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)row0 >> 32));
    const size_t ru = ((size_t)rhi << 32) | rlo;

    // stage the chunk's K and Q rows (rows >= L read as 0): 32 DMAs of 4 rows
    unsigned char* sKQ = reinterpret_cast<unsigned char*>(prep_lds);
    {
        const uint32_t rowK = (uint32_t)Hk * D * 2u;
        const Rsrc rk = make_dma_rsrc(k + (ru * Hk + kh) * D, L * rowK);
        const Rsrc rq = make_dma_rsrc(q + (ru * Hk + kh) * D, L * rowK);
        const int rr = lane >> 4, p = lane & 15;
        const uint32_t o0 = rr * rowK + 16u * (p ^ rr), o1 = rr * rowK + 16u * (p ^ (4 + rr));
        for (int j = w; j < 32; j += nw) {
            const int jj = j & 15;
            dma16(j < 16 ? rk : rq, sKQ + (j >> 4) * (C * D * 2) + 1024 * jj, (jj & 1) ? o1 : o0,
                  4u * jj * rowK);
        }
    }
    // this v-head's log_g and beta (an empty range for a wave past the last
    // v-head: it reads nothing); G = cumsum of log_g, kept as G log2(e) so
    // that exp(G_r - G_s) is one exp2
    {
        const uint32_t gb_bytes = h < G ? L * Hv * 4u : 0u;
        const rsrc_t rg = make_rsrc(log_g + ru * Hv + vh, gb_bytes);
        const rsrc_t rb_ = make_rsrc(beta + ru * Hv + vh, gb_bytes);
        const float gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)lane * Hv * 4u, 0, 0));
        const float bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb_, (uint32_t)lane * Hv * 4u, 0, 0));
        sG[lane] = wave_scan_dpp(gv) * 1.4426950408889634f;
        sBt[lane] = bv;
    }
    // the DMA is inline assembly the compiler does not track: wait for it
    // explicitly, then let every wave see every wave's rows
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    __syncthreads();

    // decay factors of this lane's entries: row 16 i + n, column 16 m + 4g + s
    float Gr[4], Bt[4];
    f32x4 Gc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        Gr[i] = sG[16 * i + n];
        Bt[i] = sBt[16 * i + n];
        const float4 t4 = *reinterpret_cast<const float4*>(sG + 16 * i + 4 * g);
        Gc[i] = f32x4{t4.x, t4.y, t4.z, t4.w};
    }

    // Gram tiles by block column i: S tiles leave at once, A stays in
    // registers.  S tile number i (i + 1) / 2 + m belongs to wave (that
    // number) % nw of the first group.
    uint16_t* dstT = tslots + ((size_t)x * Hv + vh) * SLOT_ELEMS;
    uint16_t* dstS = sslots + ((size_t)x * Hk + kh) * SLOT_ELEMS;
    const bool live = h < G;
    const bool s_group = blockIdx.z == 0;
    s16x8 kf[4][4];
    f32x4 Aoff[6];   // A_im, m < i, index (i - 1) i / 2 + m
    f32x4 Adg[4];    // A_ii: register s = A_ii[n][4g + s]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s16x8 qf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const unsigned char* fr = sKQ + (16 * i + n) * 256 + 16 * ((4 * kk + g) ^ (n & 7));
            kf[i][kk] = lds_read16(fr);
            qf[kk] = lds_read16(fr + C * D * 2);
        }
#pragma unroll
        for (int m = 0; m <= i; ++m) {
            const bool mine = s_group && ((i * (i + 1) / 2 + m) % nw) == w;   // wave-uniform
            f32x4 kk_acc = zero4(), kq_acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kk_acc = mfma_bf16(kf[m][kk], kf[i][kk], kk_acc);
            if (mine) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kq_acc = mfma_bf16(kf[m][kk], qf[kk], kq_acc);
            }
            f32x4 av, sv;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const float e = __builtin_amdgcn_exp2f(Gr[i] - Gc[m][s2]);
                av[s2] = Bt[i] * e * kk_acc[s2];
                sv[s2] = kq_acc[s2];
                if (m == i) {   // A strictly lower, S lower with the diagonal
                    av[s2] = (n > 4 * g + s2) ? av[s2] : 0.f;
                    sv[s2] = (n >= 4 * g + s2) ? sv[s2] : 0.f;
                }
            }
            if (m == i) Adg[i] = av;
            else Aoff[(i - 1) * i / 2 + m] = av;
            if (mine) {
                const s16x4 sb = s16x4{bf16_bits(sv[0]), bf16_bits(sv[1]), bf16_bits(sv[2]), bf16_bits(sv[3])};
                *reinterpret_cast<s16x4*>(dstS + (16 * i + n) * C + 16 * m + 4 * g) = sb;
            }
        }
    }
    __syncthreads();      // the staging area becomes the waves' own regions
    if (!live) return;    // a partial last group of v-heads

    // A_ii transposed into the diagonal blocks: element (4g + s, n) = A_ii[n][4g + s]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) lds[t_blk(i, i) + blk_elem(4 * g + s2, n)] = Adg[i][s2];
    wave_lds_sync();

    // T_ii = (I + A_ii)^-1 for the four diagonal blocks: lane (g, n) solves
    // column n of block g, column-oriented: once x_m is final it is removed
    // from every later row (a dependency chain of 15 steps).  All reads of
    // A_gg^T come before the writes of T_gg over it.
    {
        float* blk = lds + 272 * g;
        float colm[15][16];
#pragma unroll
        for (int m = 0; m < 15; ++m)
#pragma unroll
            for (int qd = (m + 1) >> 2; qd < 4; ++qd) {
                const float4 a4 = *reinterpret_cast<const float4*>(blk + 16 * prow(m) + 4 * (qd ^ (m >> 2)));
                colm[m][4 * qd] = a4.x; colm[m][4 * qd + 1] = a4.y;
                colm[m][4 * qd + 2] = a4.z; colm[m][4 * qd + 3] = a4.w;
            }
        float xc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xc[r] = (r == n) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m)
#pragma unroll
            for (int r = m + 1; r < 16; ++r) xc[r] = fmaf(-colm[m][r], xc[m], xc[r]);
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[blk_elem(r, n)] = xc[r];
    }
    wave_lds_sync();

    // blocks below the diagonal, by distance: M = sum_m A_im T_mj with A_im
    // from registers (k-slot 4g + s at step s), one accumulator per m; then
    // T_ij = -T_ii M with M's registers as the B operand.
    int boff[4], toff[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        boff[s2] = blk_elem(4 * g + s2, n);   // Y[4g + s][n]
        toff[s2] = blk_elem(n, 4 * g + s2);   // T_ii[n][4g + s]
    }
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        f32x4 R[3];
#pragma unroll
        for (int j = 0; j + d < 4; ++j) {
            const int i = j + d;
            f32x4 Mp[3];
#pragma unroll
            for (int m = j; m < i; ++m) {
                const float* Y = lds + t_blk(m, j);
                f32x4 acc = zero4();
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) acc = mfma_f32(Aoff[(i - 1) * i / 2 + m][s2], Y[boff[s2]], acc);
                Mp[m - j] = acc;
            }
            f32x4 M = Mp[0];
#pragma unroll
            for (int m = 1; m < d; ++m) M = M + Mp[m];
            const float* Ti = lds + t_blk(i, i);
            f32x4 t = zero4();
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) t = mfma_f32(Ti[toff[s2]], M[s2], t);
            R[j] = t;
        }
#pragma unroll
        for (int j = 0; j + d < 4; ++j)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) lds[t_blk(j + d, j) + boff[s2]] = -R[j][s2];
        wave_lds_sync();
    }

    // T rows -> workspace as bf16: the 8-column granules that reach the
    // diagonal (8 cg <= r); those wholly above it are zero and not written
    const int cg = lane & 7, jb = cg >> 1;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int r = (lane >> 3) + 8 * p, ib = p >> 1, rr = r & 15;
        if (8 * cg <= r) {
            const float* blk = lds + (jb == ib ? 272 * ib : 1088 + 256 * ((ib - 1) * ib / 2 + jb));
            const int c0 = 2 * (cg & 1);   // first 4-column granule
            const float* row = blk + 16 * prow(rr);
            const float4 a = *reinterpret_cast<const float4*>(row + 4 * (c0 ^ (rr >> 2)));
            const float4 e = *reinterpret_cast<const float4*>(row + 4 * ((c0 + 1) ^ (rr >> 2)));
            *reinterpret_cast<s16x8*>(dstT + r * C + 8 * cg) =
                s16x8{bf16_bits(a.x), bf16_bits(a.y), bf16_bits(a.z), bf16_bits(a.w),
                      bf16_bits(e.x), bf16_bits(e.y), bf16_bits(e.z), bf16_bits(e.w)};
        }
    }
}

// ---------------------------------------------------------------------------
// The state spine.  One workgroup per (sequence, v-head, 32 dv columns), six
// waves in three roles:
//   recurrence waves (2, 3): each owns 16 columns of the state h in MFMA
//     accumulators and walks the chunks in order: X = K h,
//     R = beta (V - gm X), Delta = T R, h <- gamma_L h + K^T (el Delta).
//     It hands the chunk's bf16 state (before the update) and el Delta to
//     its output wave through a double-buffered LDS exchange.
//   output waves (0, 1): one chunk behind, O = (gm / gm_L) (gm_L (Q h) +
//     S (el Delta)) for the same 16 columns, which is gm (Q h) + (Gamma o S)
//     Delta because Gamma_rs = gm_r / gm_s and el_s = gm_L / gm_s.  The
//     output path does not feed back into the state, so it leaves the
//     recurrence waves' critical path.
//   loader waves (4, 5): fill the recurrence waves' three-stage LDS ring two
//     chunks ahead, and the output waves' two-slot ring of Q and S one
//     chunk ahead, by buffer->LDS DMA (a 64-lane DMA writes lane l's 16 bytes
//     at base + 16 l; lanes beyond the buffer's range write zeros, which pads
//     a partial chunk and fills the granules of T and S above the diagonal,
//     which are not in memory), and prepare the chunk's decay factors.
// All six waves meet at one barrier per chunk.
//
// MFMA k-slots.  Lane group g (lanes 16g .. 16g+15) supplies k-values
// 8g .. 8g+7 of each 32-wide k-step, so every A fragment is one 16-byte read.
// An accumulator tile holds rows 4g .. 4g+3 in lane group g; tiles 2j and
// 2j+1 form the B operand of k-step j without any exchange when row m of
// tile t stands for index
//     sig(t, m) = 32 (t/2) + 8 (m/4) + 4 (t%2) + m%4.
// The state tiles h[db] (state rows) and the chunk-row tiles X, Y, Delta and
// O all use this map.
//
// Stage layout.  Rows are dense; the 16-byte granules of a row are permuted
// so that every fragment read is free of bank conflicts (64 banks of 4
// bytes; a 16-byte read serves 8 lanes per pass, an 8-byte read 16):
//   K (64 rows x 256 B): granule q of row r at q ^ fK(r), fK(r) = 4 (r%4) + (r/8)%2
//   T (64 rows x 128 B): granule q of row r at q ^ fT(r), fT(r) = (r/2)%2 + 2 ((r/8)%2)
//   V (64 rows x  64 B: the workgroup's 32 columns)
//   log_g, beta as loaded (64 fp32 each), then the prepared decay factors
//   gm_r = exp(G_r) and el_r = exp(G_L - G_r), and gamma_L = exp(G_L).
constexpr int ST_K = 0;
constexpr int ST_T = 16384;
constexpr int ST_V = 24576;
constexpr int ST_G = 28672;
constexpr int ST_B = 28928;
constexpr int ST_GM = 29184;
constexpr int ST_EL = 29440;
constexpr int ST_SO = 29696;
constexpr int ST_BYTES = 29712;
constexpr int N_STAGES = 3;
constexpr int DMA_K_WAVE = 17;    // loader 0: 16 K + 1 log_g (then 8 S for the output ring)
constexpr int DMA_TV_WAVE = 13;   // loader 1: 8 T + 4 V + 1 beta (then 16 Q for the output ring)
// The exchange: per output/recurrence pair and parity of the chunk, the
// bf16 state fragments (4 x 1 KB) and the bf16 el Delta fragments (2 x 1 KB),
// each stored lane-major (lane l's 16 bytes at 16 l).  Then 256 bytes of
// decay factors per output wave.
// The output ring: per slot Q (64 rows x 256 B, laid out as K) and S (64
// rows x 128 B, laid out as T).
constexpr int EX_BASE = 89344;                 // N_STAGES * ST_BYTES rounded up to 1 KB
constexpr int EX_SLOT = 6144;
constexpr int OR_BASE = EX_BASE + 4 * EX_SLOT;
constexpr int OR_Q = 0;
constexpr int OR_S = 16384;
constexpr int OR_SLOT = 24576;
constexpr int OUT_SCR = OR_BASE + 2 * OR_SLOT;
constexpr int SPINE_LDS = OUT_SCR + 2 * 256;
static_assert(SPINE_LDS <= 160 * 1024, "the spine's LDS");
static_assert(EX_BASE >= N_STAGES * ST_BYTES, "exchange after the ring");

// Batches of buffer->LDS DMAs into consecutive 1 KB pieces of LDS starting
// at the LDS byte address `lds`: M0 is set once and advanced by one scalar
// add per piece, and every lane and SGPR offset is precomputed.
__device__ __forceinline__ void dma_x4(const Rsrc& r, uint32_t lds, uint32_t v0, uint32_t v1,
                                       uint32_t v2, uint32_t v3, uint32_t s0, uint32_t s1,
                                       uint32_t s2, uint32_t s3) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %2, %1, %6 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %7 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %4, %1, %8 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %5, %1, %9 offen lds"
                 :: "s"(lds), "s"(r.d), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(s0), "s"(s1), "s"(s2), "s"(s3)
                 : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma_x8(const Rsrc& r, uint32_t lds, const uint32_t (&v)[8], const uint32_t (&so)[8]) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %2, %1, %10 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %11 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %4, %1, %12 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %5, %1, %13 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %6, %1, %14 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %7, %1, %15 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %8, %1, %16 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %9, %1, %17 offen lds"
                 :: "s"(lds), "s"(r.d), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
                    "v"(v[6]), "v"(v[7]), "s"(so[0]), "s"(so[1]), "s"(so[2]), "s"(so[3]), "s"(so[4]),
                    "s"(so[5]), "s"(so[6]), "s"(so[7])
                 : "memory", "m0", "scc");
}
__device__ __forceinline__ uint32_t lds_u32(const unsigned char* p) {
    return __builtin_amdgcn_readfirstlane(lds_addr(p));
}

// A workgroup barrier without the fences of __syncthreads, whose vmcnt(0)
// would wait for the DMA of later chunks too.  Producers wait for their own
// writes (wait_vmcnt, wait_lgkm0) before they arrive.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt vmcnt(n) for the DMA counts used here, other counters free (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define GDN_VMCNT(N) (((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n == DMA_K_WAVE) __builtin_amdgcn_s_waitcnt(GDN_VMCNT(DMA_K_WAVE));
    else if (n == DMA_TV_WAVE) __builtin_amdgcn_s_waitcnt(GDN_VMCNT(DMA_TV_WAVE));
    else __builtin_amdgcn_s_waitcnt(GDN_VMCNT(0));
}
#undef GDN_VMCNT
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ s16x8 join(s16x4 a, s16x4 b) {
    return s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// first index of tile t under sig(t, .), and of lane group g within it
__device__ __forceinline__ constexpr int sig_tile(int t) { return 32 * (t >> 1) + 4 * (t & 1); }

// Per-lane DMA byte offsets of a loader wave (chunk-independent).
struct LoadOffsets {
    uint32_t k[2];    // K rows, by (j/2)%2 of the 4-row block j
    uint32_t t[2];    // T rows, by j%2 of the 8-row block j
    uint32_t v;       // V
    uint32_t gb;      // log_g / beta
    // per 1 KB piece j: lane offsets and (uniform) SGPR offsets
    uint32_t kv[8], ks[16];   // K and Q pieces 0..15 (lane offsets repeat every 8)
    uint32_t tv[8], ts[8];    // T and S pieces 0..7 (lanes above the diagonal out of range)
    uint32_t vs[4];           // V pieces 0..3
};

__device__ __forceinline__ LoadOffsets load_offsets(int lane, int Hk, int Hv) {
    LoadOffsets o;
    const uint32_t k_row = (uint32_t)Hk * D * 2u, v_row = (uint32_t)Hv * D * 2u;
    const int rr = lane >> 4, p = lane & 15, p8 = lane & 7, hb = (lane >> 4) & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        o.k[s] = rr * k_row + (uint32_t)((p ^ (4 * rr + s)) * 16);
        o.t[s] = (uint32_t)((lane >> 3) * 128 + ((p8 ^ (hb | (s << 1))) * 16));
    }
    o.v = (uint32_t)(lane >> 2) * v_row + (uint32_t)((lane & 3) * 16);
    o.gb = (uint32_t)lane * Hv * 4u;
#pragma unroll
    for (int j = 0; j < 16; ++j) o.ks[j] = __builtin_amdgcn_readfirstlane((uint32_t)(4 * j) * k_row);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        o.kv[j] = o.k[(j >> 1) & 1];
        // piece j, lane l: row 8 j + l / 8, memory granule (columns 8 q ..
        // 8 q + 7) q = (l % 8) ^ fT(row); a granule wholly above the
        // diagonal (8 q > row) is not in memory and reads as zero
        const int row = 8 * j + (lane >> 3);
        const int qg = p8 ^ (hb | ((j & 1) << 1));
        o.tv[j] = 8 * qg <= row ? o.t[j & 1] : 0x80000000u;
        o.ts[j] = 1024u * j;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) o.vs[j] = __builtin_amdgcn_readfirstlane((uint32_t)(16 * j) * v_row);
    return o;
}

// Loader wave wl's share of chunk c's DMA into `stage`: K and log_g
// (wl = 0, DMA_K_WAVE operations) or T, V and beta (wl = 1, DMA_TV_WAVE).
// Rows beyond the chunk read as zero.
__device__ __forceinline__ void spine_load(unsigned char* stage, const LoadOffsets& o,
                                           const uint16_t* k, const uint16_t* v,
                                           const float* log_g, const float* beta,
                                           const uint16_t* slot, long row0, long len, int c, int Hk,
                                           int Hv, int kh, int vh, int tile, int wl)
{
    const long r = row0 + (long)c * C;
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)r);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r >> 32));
    const size_t ru = ((size_t)rhi << 32) | rlo;
    const uint32_t L = __builtin_amdgcn_readfirstlane((uint32_t)min((long)C, len - (long)c * C));
    const uint32_t base = lds_u32(stage);
    if (wl == 0) {
        const uint32_t k_row = (uint32_t)Hk * D * 2u;
        const Rsrc rk = make_dma_rsrc(k + (ru * Hk + kh) * D, L * k_row);
        dma_x8(rk, base + ST_K, o.kv, *reinterpret_cast<const uint32_t(*)[8]>(&o.ks[0]));
        dma_x8(rk, base + ST_K + 8192, o.kv, *reinterpret_cast<const uint32_t(*)[8]>(&o.ks[8]));
        const Rsrc rg = make_dma_rsrc(log_g + ru * Hv + vh, L * Hv * 4u);
        dma4(rg, stage + ST_G, o.gb);
    } else {
        const uint32_t v_row = (uint32_t)Hv * D * 2u;
        const Rsrc rt = make_dma_rsrc(slot, C * C * 2u);
        dma_x8(rt, base + ST_T, o.tv, o.ts);
        const Rsrc rv = make_dma_rsrc(v + (ru * Hv + vh) * D + tile * TILE_COLS, L * v_row);
        dma_x4(rv, base + ST_V, o.v, o.v, o.v, o.v, o.vs[0], o.vs[1], o.vs[2], o.vs[3]);
        const Rsrc rb = make_dma_rsrc(beta + ru * Hv + vh, L * Hv * 4u);
        dma4(rb, stage + ST_B, o.gb);
    }
}

// Loader wave wl's share of chunk c's output-ring DMA into `slot_lds`: S
// (wl = 0, 8 operations) or Q (wl = 1, 16 operations).
__device__ __forceinline__ void spine_load_out(unsigned char* slot_lds, const LoadOffsets& o,
                                               const uint16_t* q, const uint16_t* sslot, long row0,
                                               long len, int c, int Hk, int kh, int wl)
{
    const uint32_t base = lds_u32(slot_lds);
    if (wl == 0) {
        const Rsrc rs = make_dma_rsrc(sslot, C * C * 2u);
        dma_x8(rs, base + OR_S, o.tv, o.ts);
    } else {
        const long r = row0 + (long)c * C;
        const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)r);
        const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r >> 32));
        const size_t ru = ((size_t)rhi << 32) | rlo;
        const uint32_t L = __builtin_amdgcn_readfirstlane((uint32_t)min((long)C, len - (long)c * C));
        const uint32_t q_row = (uint32_t)Hk * D * 2u;
        const Rsrc rq = make_dma_rsrc(q + (ru * Hk + kh) * D, L * q_row);
        (void)q_row;   // the Q rows share K's precomputed offsets (same k-head layout)
        dma_x8(rq, base + OR_Q, o.kv, *reinterpret_cast<const uint32_t(*)[8]>(&o.ks[0]));
        dma_x8(rq, base + OR_Q + 8192, o.kv, *reinterpret_cast<const uint32_t(*)[8]>(&o.ks[8]));
    }
}

// Decay factors of the chunk in `stage` (its log_g has landed): G = cumsum
// of log_g within the chunk.  One wave, lane = row.
__device__ __forceinline__ void spine_scan(unsigned char* stage, int lane) {
    const float gv = reinterpret_cast<const float*>(stage + ST_G)[lane];
    const float G = wave_scan_dpp(gv);
    const float GL = __shfl(G, 63, 64);
    reinterpret_cast<float*>(stage + ST_GM)[lane] = __expf(G);
    reinterpret_cast<float*>(stage + ST_EL)[lane] = __expf(GL - G);
    if (lane == 0) *reinterpret_cast<float*>(stage + ST_SO) = __expf(GL);
}

// Per-lane byte offsets of a recurrence wave's operand reads inside a stage
// (chunk- and stage-independent).  Each chunk then needs a few base
// additions; the tile and k-step parts of every address are immediates.
struct FragOffsets {
    uint32_t k[4];    // K fragments, by k-step
    uint32_t t;       // T fragments
    uint32_t kt[4];   // K^T (transposing) fragments, by db / 2
    uint32_t v;       // V (transposing)
};

__device__ __forceinline__ FragOffsets frag_offsets(int g, int n, int w) {
    FragOffsets o;
    const int sig0 = 8 * (n >> 2) + (n & 3);                 // sig(0, n)
    const int fKn = 4 * (n & 3) + ((n >> 2) & 1);            // fK(sig(t, n)), any t
    const int fTn = ((n >> 1) & 1) | (((n >> 2) & 1) << 1);  // fT(sig(t, n)), any t
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o.k[kk] = (uint32_t)(sig0 * 256 + 16 * ((4 * kk + g) ^ fKn));
    o.t = (uint32_t)(sig0 * 128 + 16 * (g ^ fTn));
    // transposing reads: this lane sources row 8g + kr (+ 32 kk + 4 half) and
    // the 4 columns of quarter qq of the 8-column group
    const int kr = n >> 2, qq = n & 3;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o.kt[d] = (uint32_t)((8 * g + kr) * 256 + 16 * (4 * (d ^ kr) + (qq ^ (g & 1))));
    o.v = (uint32_t)((8 * g + kr) * 64 + 32 * w + 8 * qq);
    return o;
}

// One recurrence wave, one chunk, 16 columns (column half w of the
// workgroup) from stage S; hands its bf16 state and Delta fragments to the
// output wave through exchange slot E.
__device__ __forceinline__ void spine_step(const unsigned char* S, unsigned char* E, f32x4 (&h)[8],
                                           int g, int lane, const FragOffsets& fo)
{
    const float* gmv = reinterpret_cast<const float*>(S + ST_GM);
    const float* elv = reinterpret_cast<const float*>(S + ST_EL);
    const float* btv = reinterpret_cast<const float*>(S + ST_B);
    const unsigned char* pk[4];
    const unsigned char* pz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { pk[i] = S + fo.k[i]; pz[i] = S + fo.kt[i]; }
    const unsigned char* pt = S + fo.t;
    const unsigned char* pv = S + fo.v;
#define KF(cb, kk) lds_read16(pk[kk] + ST_K + 256 * sig_tile(cb))
#define TF(cb, kk) lds_read16(pt + ST_T + 128 * sig_tile(cb) + 64 * (kk))
#define KTF(db, kk) join(lds_read_tr(pz[(db) >> 1] + ST_K + 8192 * (kk) + 8 * ((db) & 1)), \
                         lds_read_tr(pz[(db) >> 1] + ST_K + 8192 * (kk) + 1024 + 8 * ((db) & 1)))

    // every read of the chunk's K fragments, scalars, V and T comes before
    // the exchange writes (which the compiler cannot prove disjoint from
    // them), so all are in flight while X is formed; the K fragments go
    // first, all four k-steps at once
    s16x8 kf[4][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) kf[kk][cb] = KF(cb, kk);
    float4 gm4[4], bt4[4], el4[4];
    s16x4 vv[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int row = sig_tile(cb) + 8 * g;
        gm4[cb] = *reinterpret_cast<const float4*>(gmv + row);
        bt4[cb] = *reinterpret_cast<const float4*>(btv + row);
        el4[cb] = *reinterpret_cast<const float4*>(elv + row);
        vv[cb] = lds_read_tr(pv + ST_V + 64 * sig_tile(cb));
    }
    s16x8 ft[6];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) ft[cb] = TF(cb, 0);
    ft[4] = TF(2, 1);
    ft[5] = TF(3, 1);
    const float gamL = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
        __builtin_bit_cast(int, *reinterpret_cast<const float*>(S + ST_SO))));

    s16x8 hb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        hb[kk] = frag_b(h[2 * kk], h[2 * kk + 1]);
        *reinterpret_cast<s16x8*>(E + 1024 * kk + 16 * lane) = hb[kk];
    }

    // X = K h, k-step by k-step as the fragments land
    f32x4 X[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) X[cb] = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) X[cb] = mfma_bf16(kf[kk][cb], hb[kk], X[cb]);

    // R = beta (V - gm X) for this lane's rows
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float gmr[4] = {gm4[cb].x, gm4[cb].y, gm4[cb].z, gm4[cb].w};
        const float btr[4] = {bt4[cb].x, bt4[cb].y, bt4[cb].z, bt4[cb].w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            X[cb][r] = btr[r] * (bf16_bits_to_f32((uint16_t)vv[cb][r]) - gmr[r] * X[cb][r]);
    }
    const s16x8 rb0 = frag_b(X[0], X[1]), rb1 = frag_b(X[2], X[3]);

    // Delta = T R (T lower triangular: its first 32 rows need only k < 32)
    s16x8 fk1[4];
#pragma unroll
    for (int db = 0; db < 2; ++db) { fk1[2 * db] = KTF(db, 0); fk1[2 * db + 1] = KTF(db, 1); }
    sched_fence();
    f32x4 Dl[4];
    Dl[0] = mfma_bf16(ft[0], rb0, zero4());
    Dl[1] = mfma_bf16(ft[1], rb0, zero4());
    Dl[2] = mfma_bf16(ft[2], rb0, zero4());
    Dl[3] = mfma_bf16(ft[3], rb0, zero4());
    Dl[2] = mfma_bf16(ft[4], rb1, Dl[2]);
    Dl[3] = mfma_bf16(ft[5], rb1, Dl[3]);
    sched_fence();
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        Dl[cb][0] *= el4[cb].x; Dl[cb][1] *= el4[cb].y; Dl[cb][2] *= el4[cb].z; Dl[cb][3] *= el4[cb].w;
    }
    const s16x8 ds0 = frag_b(Dl[0], Dl[1]), ds1 = frag_b(Dl[2], Dl[3]);
    *reinterpret_cast<s16x8*>(E + 4096 + 16 * lane) = ds0;
    *reinterpret_cast<s16x8*>(E + 5120 + 16 * lane) = ds1;

    // h <- gamma_L h + K^T (el Delta): 8 row blocks, two blocks ahead
#pragma unroll
    for (int db = 0; db < 8; ++db) h[db] = h[db] * gamL;
#pragma unroll
    for (int db = 0; db < 8; db += 2) {
        s16x8 fk2[4];
        if (db + 2 < 8) {
            fk2[0] = KTF(db + 2, 0); fk2[1] = KTF(db + 2, 1);
            fk2[2] = KTF(db + 3, 0); fk2[3] = KTF(db + 3, 1);
        }
        sched_fence();
        h[db] = mfma_bf16(fk1[1], ds1, mfma_bf16(fk1[0], ds0, h[db]));
        h[db + 1] = mfma_bf16(fk1[3], ds1, mfma_bf16(fk1[2], ds0, h[db + 1]));
        sched_fence();
        if (db + 2 < 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fk1[i] = fk2[i];
        }
    }
#undef KF
#undef TF
#undef KTF
    wait_lgkm0();   // the exchange writes are complete before the barrier
}

// One output wave, one chunk: O = (gm / gm_L) (gm_L (Q h) + S (el Delta))
// for its 16 columns, with Q and S from output-ring slot Sq, the bf16 state
// and el Delta from the exchange slot E the recurrence wave filled, and lg
// this lane's log_g (lane = row).  The products are formed transposed: a
// B-operand fragment of h or el Delta is the A operand of its transpose and
// an A-operand fragment of Q or S the B operand of its transpose, so the
// same fragments serve, and lane (g, n) register r of tile cb ends up
// holding O[sig(cb, n)][4g + r]: four consecutive columns of one row, stored
// at once.  `ro` covers exactly the chunk's output rows;
// `lane_off` is the lane's byte offset for row sig(0, n) and column 4g, and
// soff[cb] the uniform offset of tile cb's rows.
template <bool kOutF32>
__device__ __forceinline__ void out_step(const unsigned char* Sq, const unsigned char* E, float* scr,
                                         float lg, const FragOffsets& fo, rsrc_t ro,
                                         uint32_t lane_off, const uint32_t (&soff)[4], int n,
                                         int lane)
{
    const float G = wave_scan_dpp(lg);
    const float GL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
    scr[lane] = __expf(G - GL);   // gm_r / gm_L
    const float gmL = __expf(GL);
    s16x8 hb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) hb[kk] = lds_read16(E + 1024 * kk + 16 * lane);
    const s16x8 db0 = lds_read16(E + 4096 + 16 * lane), db1 = lds_read16(E + 5120 + 16 * lane);
    f32x4 Y[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) Y[cb] = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        s16x8 qf[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) qf[cb] = lds_read16(Sq + fo.k[kk] + OR_Q + 256 * sig_tile(cb));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) Y[cb] = mfma_bf16(hb[kk], qf[cb], Y[cb]);
    }
    s16x8 sf[6];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) sf[cb] = lds_read16(Sq + fo.t + OR_S + 128 * sig_tile(cb));
    sf[4] = lds_read16(Sq + fo.t + OR_S + 128 * sig_tile(2) + 64);
    sf[5] = lds_read16(Sq + fo.t + OR_S + 128 * sig_tile(3) + 64);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) Y[cb] = Y[cb] * gmL;
    f32x4 O[4];
    O[0] = mfma_bf16(db0, sf[0], Y[0]);
    O[1] = mfma_bf16(db0, sf[1], Y[1]);
    O[2] = mfma_bf16(db0, sf[2], Y[2]);
    O[3] = mfma_bf16(db0, sf[3], Y[3]);
    O[2] = mfma_bf16(db1, sf[4], O[2]);
    O[3] = mfma_bf16(db1, sf[5], O[3]);
    wave_lds_sync();
    const int sig0 = 8 * (n >> 2) + (n & 3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[cb] = O[cb] * scr[sig_tile(cb) + sig0];   // row factor of this lane's row
    // hardware RNE conversion; rows beyond a partial chunk fall outside `ro`
    // and are dropped
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const f32x4 o = O[cb];
        if (kOutF32) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4v{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                                          __float_as_uint(o[2]), __float_as_uint(o[3])},
                                                   ro, lane_off, soff[cb], 0);
        } else {
            const uint32_t lo = (uint16_t)bf16_bits(o[0]) | ((uint32_t)(uint16_t)bf16_bits(o[1]) << 16);
            const uint32_t hi = (uint16_t)bf16_bits(o[2]) | ((uint32_t)(uint16_t)bf16_bits(o[3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2v{lo, hi}, ro, lane_off, soff[cb], 0);
        }
    }
    wave_lds_sync();   // the decay scratch is rewritten by the next chunk
}

template <bool kOutF32>
__global__ void __launch_bounds__(384)
gdn_spine_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const float* __restrict__ log_g,
                 const float* __restrict__ beta, const float* h0, void* __restrict__ out,
                 float* h_final, const uint16_t* __restrict__ tslots,
                 const uint16_t* __restrict__ sslots, int T, int Hk, int Hv,
                 const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_base,
                 const int32_t* __restrict__ order, int nc_dense, long n_slots)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds[SPINE_LDS];
    unsigned char* ring = lds;

    const int tid = threadIdx.x;
    // the wave index is wave-uniform; say so, so per-wave values live in SGPRs
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    // Workgroup i runs on XCD i % 8.  Map the grid so that the workgroups of
    // one k-head (its v-heads and column tiles) share an XCD and its L2.
    const int W = gridDim.x;
    const int lin = (W % 8 == 0) ? (blockIdx.x % 8) * (W / 8) + blockIdx.x / 8 : blockIdx.x;
    const int vh = lin / N_TILES;
    const int tile = lin % N_TILES;
    const int b = order ? order[blockIdx.y] : (int)blockIdx.y;
    const int kh = vh / (Hv / Hk);

    long row0, len;
    seq_rows(cu, b, T, &row0, &len);
    const long slot0 = cu ? (long)chunk_base[b] : (long)b * nc_dense;
    int nc = (int)((len + C - 1) / C);
    // Only a decreasing cu_seqlens (a broken precondition) can make this
    // bind; it keeps every read inside the workspace.
    if (slot0 + nc > n_slots) nc = (int)max(0L, n_slots - slot0);
    const uint16_t* slot_base = tslots + ((size_t)slot0 * Hv + vh) * SLOT_ELEMS;   // T, by chunk
    const size_t slot_stride = (size_t)Hv * SLOT_ELEMS;
    const uint16_t* s_base = sslots + ((size_t)slot0 * Hk + kh) * SLOT_ELEMS;      // S, by chunk
    const size_t s_stride = (size_t)Hk * SLOT_ELEMS;

    if (w >= 4) {   // loader waves
        const int wl = w - 4;
        const int cnt = wl == 0 ? DMA_K_WAVE : DMA_TV_WAVE;
        const LoadOffsets o = load_offsets(lane, Hk, Hv);
        for (int c = 0; c < 2 && c < nc; ++c)
            spine_load(ring + c * ST_BYTES, o, k, v, log_g, beta, slot_base + (size_t)c * slot_stride,
                       row0, len, c, Hk, Hv, kh, vh, tile, wl);
        if (nc > 0) {
            wait_vmcnt(nc > 1 ? cnt : 0);
            if (wl == 0) spine_scan(ring, lane);
            wait_lgkm0();
        }
        for (int c = 0; c <= nc; ++c) {
            // chunk c is ready in the recurrence ring; stage (c+2)%3 and
            // output slot c%2 are free
            ring_barrier();
            if (c < nc)
                spine_load_out(lds + OR_BASE + (c & 1) * OR_SLOT, o, q, s_base + (size_t)c * s_stride, row0,
                               len, c, Hk, kh, wl);
            if (c + 2 < nc)
                spine_load(ring + ((c + 2) % N_STAGES) * ST_BYTES, o, k, v, log_g, beta,
                           slot_base + (size_t)(c + 2) * slot_stride, row0, len, c + 2, Hk, Hv, kh,
                           vh, tile, wl);
            if (c < nc) {
                // chunk c's output operands and chunk c+1 have landed
                wait_vmcnt(c + 2 < nc ? cnt : 0);
                if (c + 1 < nc && wl == 0) spine_scan(ring + ((c + 1) % N_STAGES) * ST_BYTES, lane);
                wait_lgkm0();
            }
        }
        return;
    }

    const int half = w & 1;   // which 16 of the workgroup's 32 columns
    const int col = tile * TILE_COLS + 16 * half + n;
    unsigned char* ex = lds + EX_BASE + half * 2 * EX_SLOT;

    if (w >= 2) {   // recurrence waves
        f32x4 h[8];
        const size_t hoff = ((size_t)b * Hv + vh) * D * D;
        // state row of h[db][r] in this lane: sig(db, 4g + r)
        if (h0) {   // one uniform branch: all 32 loads in flight together
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[db][r] = h0[hoff + (size_t)(sig_tile(db) + 8 * g + r) * D + col];
        } else {
#pragma unroll
            for (int db = 0; db < 8; ++db) h[db] = zero4();
        }
        const FragOffsets fo = frag_offsets(g, n, half);
        for (int c = 0; c <= nc; ++c) {
            ring_barrier();
            if (c < nc) spine_step(ring + (c % N_STAGES) * ST_BYTES, ex + (c & 1) * EX_SLOT, h, g, lane, fo);
        }
        if (h_final) {
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h_final[hoff + (size_t)(sig_tile(db) + 8 * g + r) * D + col] = h[db][r];
        }
        return;
    }

    // output waves: chunk c - 1 at step c
    float* scr = reinterpret_cast<float*>(lds + OUT_SCR + 256 * half);
    constexpr uint32_t es = kOutF32 ? 4u : 2u;
    const uint32_t rs = __builtin_amdgcn_readfirstlane((uint32_t)Hv * D * es);
    const uint32_t lane_off = (uint32_t)(8 * (n >> 2) + (n & 3)) * rs +
                              (uint32_t)(tile * TILE_COLS + 16 * half + 4 * g) * es;
    uint32_t soff[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) soff[cb] = (uint32_t)sig_tile(cb) * rs;
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)row0);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)row0 >> 32));
    char* obase = reinterpret_cast<char*>(out) + ((((size_t)rhi << 32) | rlo) * Hv + vh) * D * es;
    const FragOffsets fo = frag_offsets(g, n, half);
    float lg = 0.f;
    auto load_lg = [&](int c) {   // this chunk's log_g, lane = row
        const long r = row0 + (long)c * C;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)r);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r >> 32));
        const size_t ru = ((size_t)hi << 32) | lo;
        const uint32_t L = __builtin_amdgcn_readfirstlane((uint32_t)min((long)C, len - (long)c * C));
        const rsrc_t rg = make_rsrc(log_g + ru * Hv + vh, L * Hv * 4u);
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)lane * Hv * 4u, 0, 0));
    };
    if (nc > 0) lg = load_lg(0);
    for (int c = 0; c <= nc; ++c) {
        ring_barrier();
        if (c >= 1) {   // chunk c - 1
            const long rem = len - (long)(c - 1) * C;
            const rsrc_t ro = make_rsrc(obase + (size_t)(c - 1) * C * rs, (uint32_t)min((long)C, rem) * rs);
            const float lg_c = lg;
            if (c < nc) lg = load_lg(c);
            out_step<kOutF32>(lds + OR_BASE + ((c - 1) & 1) * OR_SLOT, ex + ((c - 1) & 1) * EX_SLOT,
                              scr, lg_c, fo, ro, lane_off, soff, n, lane);
        }
    }
}

// base[B + 1] then order[B]
size_t table_bytes(int B) { return ((size_t)(2 * B + 1) * sizeof(int32_t) + 255) & ~(size_t)255; }

long slot_count(int B, int T, bool packed) {
    return packed ? (long)(T + C - 1) / C + B : (long)B * ((T + C - 1) / C);
}

}  // namespace

size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv, bool packed)
{
    return table_bytes(B) + (size_t)slot_count(B, T, packed) * (Hv + Hk) * SLOT_ELEMS * sizeof(uint16_t);
}

bool prefill_mfma_accepts(const PrefillArgs& a)
{
    return a.io_dtype == 1 && a.dk == D && a.dv == D && a.chunk == C;
}

Geometry prefill_mfma_geometry(const PrefillArgs& a)
{
    Geometry g{"gdn_wy_prep_kernel+gdn_spine_kernel", {(unsigned)(a.Hv * N_TILES), (unsigned)a.B, 1u}, 384u,
               (unsigned)SPINE_LDS};
    return g;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s)
{
    const bool packed = a.cu_seqlens != nullptr;
    int32_t* base = reinterpret_cast<int32_t*>(a.workspace);
    const int nc_dense = (a.T + C - 1) / C;
    const long n_slots = slot_count(a.B, a.T, packed);
    uint16_t* tslots = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(a.workspace) + table_bytes(a.B));
    uint16_t* sslots = tslots + (size_t)n_slots * a.Hv * SLOT_ELEMS;
    const int32_t* order = packed && a.B <= MAX_ORDERED ? base + a.B + 1 : nullptr;
    if (packed) {
        hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.B, a.T, base);
    }
    if (n_slots > 0) {
        const int G = a.Hv / a.Hk, nw = G < 4 ? G : 4;
        const size_t shmem = prep_lds_bytes(nw);
        hipLaunchKernelGGL(gdn_wy_prep_kernel, dim3((unsigned)n_slots, a.Hk, (unsigned)((G + nw - 1) / nw)),
                           dim3(64 * nw), shmem, s,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, a.log_g, a.beta, tslots, sslots,
                           a.B, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense);
    }
    dim3 grid(a.Hv * N_TILES, a.B);
    if (a.out_dtype == 0)
        hipLaunchKernelGGL((gdn_spine_kernel<true>), grid, dim3(384), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, tslots, sslots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, order, nc_dense,
                           n_slots);
    else
        hipLaunchKernelGGL((gdn_spine_kernel<false>), grid, dim3(384), 0, s, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, a.log_g, a.beta, a.h0, a.out,
                           a.h_final, tslots, sslots, a.T, a.Hk, a.Hv, a.cu_seqlens, base, order, nc_dense,
                           n_slots);
    return hipGetLastError();
}

}  // namespace gdn

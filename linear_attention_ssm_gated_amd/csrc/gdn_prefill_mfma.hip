// bf16 MFMA chunked prefill for dk = dv = 128, chunk = 64 (gfx950).
//
// Two kernels on the caller's stream (the segment scan for narrow layers,
// further down, adds a second spine launch and a combine kernel):
//
// gdn_wy_prep_kernel, one workgroup per (chunk, k-head), all chunks at once:
//   the intra-chunk terms that do not depend on the state (the pages' W/U
//   producer behind the spine, ssm_gdn_tc_route.rs, doc of the pipe spine):
//     G = cumsum(log_g), Gamma_rs = exp(G_r - G_s) for s <= r
//     A = strict_lower(diag(beta) (Gamma o K K^T)),  T = (I + A)^-1   (per v-head)
//     T_e = diag(el) T diag(beta),  el = exp(G_L - G)                  (per v-head)
//     PT = (Gamma o lower_incl(Q K^T)) T diag(beta)                    (per v-head)
//   K K^T, Q K^T and PT run on bf16 MFMA with fp32 accumulation; T is solved
//   in 16x16 blocks: the diagonal ones by forward substitution in fp32 on VALU,
//   the ones below them on bf16 MFMA with fp32 accumulation; T_e and PT are
//   stored as bf16 MFMA fragments in
//   the workspace, their granules above the diagonal left unwritten (they are
//   zero, and the spine never reads them from memory), each followed by the
//   chunk's per-row factors gm = exp(G).  Every decay factor formed is exp of
//   a non-positive difference of cumulative log decays, so nothing can
//   overflow, whatever the gates.
//
// gdn_spine_kernel, one workgroup per (sequence, v-head, 32 dv columns),
//   walking the chunks in order: the state spine (same page, the tensor-core
//   spine: bf16 MFMA operands, the fp32 accumulators are the recurrent state,
//   h stays f32).  Per chunk:
//     X = K h,  R = V - gm X,  Delta_e = T_e R   (= diag(el) (U - W h) of the WY form)
//     O = gm (Q h) + PT R
//     h <- gamma_L h + K^T Delta_e,  gamma_L = exp(G_L)
//   Columns of h evolve independently (the dv split of the pages' SPLIT
//   variants), so the workgroups never exchange data.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16, 64 lanes, lane = 16 g + i):
// lane group g supplies k-values 8g .. 8g+7 of each 32-wide k-step.  A 16x16
// fp32 accumulator tile holds rows 4g .. 4g+3 of column n in lane 16g + n;
// when row m of tile t stands for index sig(t, m) = 32 (t/2) + 8 (m/4) +
// 4 (t%2) + m%4, tiles 2j and 2j+1 ARE the B operand of k-step j after
// rounding to bf16, and every A fragment is one 16-byte read of its row.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;        // chunk rows
constexpr int D = 128;       // dk = dv
constexpr int TILE_COLS = 32;            // dv columns per spine workgroup
constexpr int N_TILES = D / TILE_COLS;   // 4

// Workspace slots: T_b and P per (chunk, v-head), each the six 1 KiB MFMA
// fragments of a 64 x 64 bf16 lower-triangular matrix M; fragment f covers
// output tile cb(f) and k-step kk(f) (f = 0..3: (f, 0); f = 4: (2, 1); f = 5:
// (3, 1)), and its lane l = 16 g + n holds M[sig(cb, n)][32 kk + 8 g .. + 7] at
// byte 16 l.  Granules wholly above the diagonal are neither written nor read.
constexpr int NFRAG = 6;
constexpr int FRAG_BYTES = 1024;
constexpr int SLOT_BYTES = NFRAG * FRAG_BYTES;
// each slot also carries the chunk's per-row decay factors after the fragments
// (1 KiB for T_b's, 256 B for P's)
constexpr int SLOT_STRIDE = SLOT_BYTES + 1024;
__host__ __device__ constexpr int frag_cb(int f) { return f < 4 ? f : f - 2; }
__host__ __device__ constexpr int frag_kk(int f) { return f < 4 ? 0 : 1; }
// first index of tile t under sig(t, .), and the index of row m of tile t
__host__ __device__ constexpr int sig_tile(int t) { return 32 * (t >> 1) + 4 * (t & 1); }
__host__ __device__ constexpr int sig_row(int t, int m) { return sig_tile(t) + 8 * (m >> 2) + (m & 3); }
__host__ __device__ constexpr bool frag_live(int f, int l) {
    return 32 * frag_kk(f) + 8 * (l >> 4) <= sig_row(frag_cb(f), l & 15);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ short bf16_bits(float x) {
    return (short)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// B operand from two accumulator tiles of consecutive k-blocks.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats rounded to bf16 (RNE) in one dword, the first in the low half
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ s16x8 frag_b(f32x4 lo, f32x4 hi) {
    return s16x8{bf16_bits(lo[0]), bf16_bits(lo[1]), bf16_bits(lo[2]), bf16_bits(lo[3]),
                 bf16_bits(hi[0]), bf16_bits(hi[1]), bf16_bits(hi[2]), bf16_bits(hi[3])};
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
// the nontemporal cache-policy bit of a gfx950 buffer access
constexpr int CPOL_NT = 2;
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
// and writes T_b = T diag(beta) to the (chunk, v-head) slot as bf16 MFMA
// fragments, and P = exp(G_r - G_s) (Q K^T)_rs (lower, with the diagonal)
// into its own LDS fragments.  The waves never wait for each other after the
// staging.
//
// Gram tiles are formed above the diagonal, tile (m, i) = K_m K_i^T and
// K_m Q_i^T (16-row blocks, m <= i), so that lane (g, n) register s holds
// the entry of row 16 i + n, column 16 m + 4g + s of K K^T and of Q K^T: the
// decay factor of both is the same, a P tile leaves as four consecutive bf16
// of one row, and an off-diagonal A tile is directly the A operand of an
// fp32 MFMA whose k-slot of lane group g at step s is 4g + s.
//
// T is formed on 16 x 16 blocks: T_ii = (I + A_ii)^-1 by forward
// substitution in fp32, then T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj by
// distance i - j on bf16 products.  Block row r is stored at slot p(r) = 4 (r/4) + ((r + r/4) % 4) and
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
constexpr int P_TILE_BYTES = 64 * 8;   // a P tile in LDS: each lane's four bf16
constexpr int PREP_STAGE_BYTES = 2 * C * D * 2;           // K then Q, 256-byte rows
// K/Q staging: granule q of row r at q ^ (r % 8), so that a fragment read (8
// lanes, 8 consecutive rows, one granule) is free of bank conflicts.  After
// the larger of the staging area and the per-wave regions come G log2(e) and
// beta per row for each wave.
__host__ __device__ constexpr int prep_gb_base(int nw) {   // floats
    return PREP_STAGE_BYTES / 4 > nw * PREP_WAVE_FLOATS ? PREP_STAGE_BYTES / 4 : nw * PREP_WAVE_FLOATS;
}
// then each wave's P as bf16 MFMA fragments (the B operand of P T_b)
__host__ __device__ constexpr int prep_p_base(int nw) {   // bytes
    return (prep_gb_base(nw) + nw * 2 * C) * (int)sizeof(float);
}
__host__ __device__ constexpr size_t prep_lds_bytes(int nw) {
    return (size_t)prep_p_base(nw) + (size_t)nw * SLOT_BYTES;
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
                   unsigned char* __restrict__ tbs, unsigned char* __restrict__ pps, int B, int T,
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
    unsigned char* sPall = reinterpret_cast<unsigned char*>(prep_lds) + prep_p_base(nw);

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
        const float Gl2 = wave_scan_dpp(gv) * 1.4426950408889634f;
        sG[lane] = Gl2;
        sBt[lane] = bv;
        if (h < G) {
            // the spine's per-row decay factors gm = exp(G) of this (chunk,
            // v-head), rows past a partial chunk keeping the last row's G.
            // Row sig(t, m) is needed by recurrence lane group m / 4 in
            // accumulator register m % 4 of tile t, and by output lane m for
            // tile t: after T_e, gm by lane group ([m / 4][t][m % 4]) and
            // gamma_L = exp(G_L); after PT, gm by output lane ([m][t]).
            const float GLl2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gl2), 63));
            const float gm = __builtin_amdgcn_exp2f(Gl2);
            const int t = 2 * (lane >> 5) + ((lane >> 2) & 1), m = 4 * ((lane >> 3) & 3) + (lane & 3);
            float* te_tail = reinterpret_cast<float*>(tbs + ((size_t)x * Hv + vh) * SLOT_STRIDE + SLOT_BYTES);
            float* pt_tail = reinterpret_cast<float*>(pps + ((size_t)x * Hv + vh) * SLOT_STRIDE + SLOT_BYTES);
            te_tail[16 * (m >> 2) + 4 * t + (m & 3)] = gm;
            if (lane == 0) te_tail[64] = __builtin_amdgcn_exp2f(GLl2);
            pt_tail[4 * m + t] = gm;
        }
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

    // Gram tiles by block column i, each wave for its own v-head: the decay
    // factor of an entry is formed once and serves A and P alike; P tiles
    // leave at once (as bf16, into the wave's P fragments), A stays in
    // registers.  (Sharing the Q K^T tiles among the group's waves instead
    // saves MFMAs but forms every P factor again per v-head, which costs
    // more issue than the MFMAs.)
    unsigned char* dstT = tbs + ((size_t)x * Hv + vh) * SLOT_STRIDE;
    const bool live = h < G;
    s16x8 kf[4][4];
    f32x4 Aoff[6];   // A_im, m < i, index (i - 1) i / 2 + m
    f32x4 Adg[4];    // A_ii: register s = A_ii[n][4g + s]
    if (live) {
        unsigned char* sPw = sPall + w * SLOT_BYTES;
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
                f32x4 kk_acc = zero4(), kq_acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kk_acc = mfma_bf16(kf[m][kk], kf[i][kk], kk_acc);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kq_acc = mfma_bf16(kf[m][kk], qf[kk], kq_acc);
                f32x4 av, pv;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const float e = __builtin_amdgcn_exp2f(Gr[i] - Gc[m][s2]);
                    av[s2] = Bt[i] * e * kk_acc[s2];
                    pv[s2] = e * kq_acc[s2];
                    if (m == i) {
                        av[s2] = (n > 4 * g + s2) ? av[s2] : 0.f;    // A strictly lower
                        pv[s2] = (n >= 4 * g + s2) ? pv[s2] : 0.f;   // P lower with the diagonal
                    }
                }
                if (m == i) Adg[i] = av;
                else Aoff[(i - 1) * i / 2 + m] = av;
                // this lane's four P entries (row 16 i + n, columns 16 m + 4 g ..
                // + 3) in tile order, lane order within the tile
                *reinterpret_cast<s16x4*>(sPw + P_TILE_BYTES * (i * (i + 1) / 2 + m) + 8 * lane) =
                    s16x4{bf16_bits(pv[0]), bf16_bits(pv[1]), bf16_bits(pv[2]), bf16_bits(pv[3])};
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

    // blocks below the diagonal, by distance, on bf16 MFMA with fp32
    // accumulation: M = sum_{m=j}^{i-1} A_im T_mj takes two blocks m per
    // 32-wide k-step, k-slot 8g + t standing for column 4g + (t % 4) of the
    // first (t < 4) or the second block, so that A_im's registers (row n,
    // columns 4g .. 4g + 3) and T_mj's accumulator registers (rows 4g .. 4g + 3,
    // column n) are the two operands as they are; then T_ij = -T_ii M with T_ii's
    // row n from LDS as A and M's registers as B, the k-step's second half zero.
    // The diagonal blocks come from LDS in accumulator order, the others from
    // the registers of the distances before.  (The blocks enter T_e and PT as
    // bf16 anyway; their bf16 products cost one MFMA per pair of blocks where
    // the fp32 16x16x4 form took four per block at twice the cycles.)
    int boff[4], toff[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        boff[s2] = blk_elem(4 * g + s2, n);   // Y[4g + s][n]
        toff[s2] = blk_elem(n, 4 * g + s2);   // T_ii[n][4g + s]
    }
    // Column n of every block scaled by beta_{16 j + n}: the blocks formed are
    // those of T_b = T diag(beta) (the recursion is linear in a column
    // scaling), which T_e and PT take.
    f32x4 Tdg[4];   // T_b,jj: register s = T_jj[4g + s][n] beta_{16 j + n}
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float bj = sBt[16 * j + n];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) Tdg[j][s2] = lds[t_blk(j, j) + boff[s2]] * bj;
    }
    f32x4 Tlo[6];   // T_b,ij, i > j, index (i - 1) i / 2 + j: register s = T_b,ij[4g + s][n]
#pragma unroll
    for (int d = 1; d < 4; ++d) {
#pragma unroll
        for (int j = 0; j + d < 4; ++j) {
            const int i = j + d;
            f32x4 M = zero4();
#pragma unroll
            for (int m = j; m < i; m += 2) {
                const f32x4 t0 = m == j ? Tdg[j] : Tlo[(m - 1) * m / 2 + j];
                const f32x4 a1 = m + 1 < i ? Aoff[(i - 1) * i / 2 + m + 1] : zero4();
                const f32x4 t1 = m + 1 < i ? Tlo[m * (m + 1) / 2 + j] : zero4();
                M = mfma_bf16(frag_b(Aoff[(i - 1) * i / 2 + m], a1), frag_b(t0, t1), M);
            }
            f32x4 ti;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) ti[s2] = lds[t_blk(i, i) + toff[s2]];
            const f32x4 t = mfma_bf16(frag_b(ti, zero4()), frag_b(M, zero4()), zero4());
            Tlo[(i - 1) * i / 2 + j] = -t;
        }
    }
    // every read of the unscaled diagonal blocks is done: T_b into LDS
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                lds[t_blk(i, j) + boff[s2]] = i == j ? Tdg[i][s2] : Tlo[(i - 1) * i / 2 + j][s2];
    wave_lds_sync();

    // T_e = diag(el) T_b, el = exp(G_L - G) per row -> workspace as
    // bf16 fragments: lane l of fragment f holds row sig(cb, l % 16), columns
    // c0 .. c0 + 7 (c0 = 32 kk + 8 (l / 16)), when that granule reaches the
    // diagonal
    const float GL2 = sG[C - 1];
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
        if (frag_live(f, lane)) {
            const int r = sig_row(frag_cb(f), n), c0 = 32 * frag_kk(f) + 8 * g;
            const int ib = r >> 4, jb = c0 >> 4, rr = r & 15;
            const float* blk = lds + (jb == ib ? 272 * ib : 1088 + 256 * ((ib - 1) * ib / 2 + jb));
            const int q4 = (c0 & 15) >> 2;   // first 4-column granule within the block
            const float* row = blk + 16 * prow(rr);
            const float4 a = *reinterpret_cast<const float4*>(row + 4 * (q4 ^ (rr >> 2)));
            const float4 e = *reinterpret_cast<const float4*>(row + 4 * ((q4 + 1) ^ (rr >> 2)));
            const float el = __builtin_amdgcn_exp2f(GL2 - sG[r]);
            *reinterpret_cast<s16x8*>(dstT + FRAG_BYTES * f + 16 * lane) =
                s16x8{bf16_bits(el * a.x), bf16_bits(el * a.y), bf16_bits(el * a.z), bf16_bits(el * a.w),
                      bf16_bits(el * e.x), bf16_bits(el * e.y), bf16_bits(el * e.z), bf16_bits(el * e.w)};
        }
    }

    // PT = P T_b, formed transposed (PT^T = T_b^T P^T): output tile (a, ip)
    // covers columns 16 a .. + 15 and rows 16 ip .. + 15, and its k runs over
    // the row blocks ib = a .. ip of T_b (T_b and P are lower triangular), two
    // blocks per k-step, k-slot 8g + t standing for row 4g + (t % 4) of the
    // first (t < 4) or the second block: the A operand is then T_b's
    // accumulator registers (column 16 a + n, rows 4g .. 4g + 3) and the B
    // operand P's tile registers as the Gram phase left them (row 16 ip + n,
    // columns 4g .. 4g + 3), both as they are.  Lane (g, n) ends with
    // PT[16 ip + n][16 a + 4g .. + 3], half of a workspace granule; granules
    // wholly above the diagonal are not written.
    const unsigned char* sPw = sPall + w * SLOT_BYTES;
    unsigned char* dstP = pps + ((size_t)x * Hv + vh) * SLOT_STRIDE;
    auto tb = [&](int ib, int a) { return ib == a ? Tdg[a] : Tlo[(ib - 1) * ib / 2 + a]; };
    auto ptile = [&](int ip, int ib) {
        return *reinterpret_cast<const s16x4*>(sPw + P_TILE_BYTES * (ip * (ip + 1) / 2 + ib) + 8 * lane);
    };
    auto pt_tile = [&](int ip, int a) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ib = a; ib <= ip; ib += 2) {
            const bool two = ib + 1 <= ip;
            const s16x4 p0 = ptile(ip, ib);
            const s16x4 p1 = two ? ptile(ip, ib + 1) : s16x4{0, 0, 0, 0};
            const s16x8 pb = s16x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            acc = mfma_bf16(frag_b(tb(ib, a), two ? tb(ib + 1, a) : zero4()), pb, acc);
        }
        const s16x4 v = s16x4{bf16_bits(acc[0]), bf16_bits(acc[1]), bf16_bits(acc[2]), bf16_bits(acc[3])};
        return __builtin_bit_cast(u32x2v, v);
    };
    // the ten output tiles in pairs: lane groups 2e and 2e + 1 hold the two
    // halves of a granule, so one permlane16 swap per dword leaves the even
    // group with the first tile's whole granules and the odd group with the
    // second's, each stored as one 16-byte piece
    constexpr int TIP[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3}, TA[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    const int ge = g & ~1;   // the even group of the pair: the granule's first half
#pragma unroll
    for (int u = 0; u < 10; u += 2) {
        const u32x2v v0 = pt_tile(TIP[u], TA[u]), v1 = pt_tile(TIP[u + 1], TA[u + 1]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(v0[0], v1[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(v0[1], v1[1], false, false);
        const u32x4v granule = u32x4v{s0[0], s1[0], s0[1], s1[1]};
        const int ip = (g & 1) ? TIP[u + 1] : TIP[u], a = (g & 1) ? TA[u + 1] : TA[u];
        // row rho = sig(cb, np); columns 16 a + 4 ge .. + 7 are lane (gp, np)'s
        // granule in fragment (cb, kk)
        const int rho = 16 * ip + n, c0 = 16 * a + 4 * ge;
        const int cb = 2 * (rho >> 5) + ((rho >> 2) & 1), np = 4 * ((rho >> 3) & 3) + (rho & 3);
        const int kk2 = c0 >> 5, gp = (c0 & 31) >> 3;
        const int f = kk2 == 0 ? cb : cb + 2;
        if (c0 <= rho)   // the granule reaches the diagonal
            *reinterpret_cast<u32x4v*>(dstP + FRAG_BYTES * f + 16 * (16 * gp + np)) = granule;
    }
}

// ---------------------------------------------------------------------------
// The state spine.  One workgroup per (sequence, v-head, 32 dv columns), four
// waves, one per SIMD (wave w runs on SIMD w):
//   the loader (0): the workgroup's memory traffic into LDS, by buffer->LDS
//     DMA: in step c, chunk c + 3's ring stage and chunk c + 1's output slot,
//     each filled two steps before it is read, which covers the memory
//     latency, and chunk c's Q rows, read by the output wave in step c + 1.
//     A DMA holds the wave that issues it for as long as the compute unit's
//     memory path takes to accept its lines.  With many workgroups in flight
//     (Q_SPLIT_GRID or more) and the output stores on that path too, that
//     makes the loader's DMAs the pace of the step, and the recurrence waves
//     issue the Q rows instead (half each, at the start of step c); otherwise
//     the recurrence chain sets the pace and the loader keeps them.
//   the output wave (1): one chunk behind the recurrence, O = gm (Q h) + PT R
//     for all 32 columns (PT R = P Delta).
//   recurrence waves (2, 3): 16 columns each; the fp32 state h lives in MFMA
//     accumulators and walks the chunks in order:
//       X = K h,  R = V - gm X,  Delta_e = T_e R,  h <- gamma_L h + K^T Delta_e.
//     The chunk's bf16 state and R go to the output wave through a
//     double-buffered LDS exchange.  A recurrence wave is bound by its own
//     instruction issue: every operand of chunk c + 1 comes from LDS, read
//     while it computes chunk c (K fragments of X, transposed K fragments of
//     the update, V, T_e, gm), and its VALU work is only what the recurrence
//     needs: the state's bf16 copy, its decay, R and the two roundings to
//     bf16.  gm reaches the lanes that need it as a table in LDS: lane group g
//     reads the 16 factors of its accumulator rows with 4 broadcast reads.
//
// LDS (bytes).  Recurrence ring stage (three stages):
//   K rows (64 x 256 B), granule q of row r at q ^ fK(r), fK(r) = 4 (r%4) + (r/8)%2
//   V rows of the workgroup's 32 columns (64 x 64 B)
//   T_e fragments (6 KiB), then gm by lane group and gamma_L (1 KiB)
// Output slot (three): the six PT fragments, gm in output-lane order [n][cb].
// Q slot (two): Q rows laid out as K.
// Exchange, per recurrence wave and chunk parity: the bf16 state fragments
// (4 x 1 KiB) and the bf16 R fragments (2 x 1 KiB), lane-major.
constexpr int RS_K = 0;
constexpr int RS_V = 16384;
constexpr int RS_TE = 20480;
constexpr int RS_SC = RS_TE + SLOT_BYTES;
constexpr int RS_BYTES = RS_SC + 1024;
constexpr int N_RS = 3;
constexpr int N_OS = 3;
constexpr int OS_BASE = N_RS * RS_BYTES;
constexpr int OS_P = 0;
constexpr int OS_GM = SLOT_BYTES;
constexpr int OS_BYTES = SLOT_BYTES + 256;
constexpr int QS_BASE = OS_BASE + N_OS * OS_BYTES;
constexpr int QS_BYTES = 16384;
constexpr int EX_BASE = QS_BASE + 2 * QS_BYTES;
constexpr int EX_BYTES = 6144;
constexpr int SPINE_LDS = EX_BASE + 4 * EX_BYTES;
static_assert(SPINE_LDS <= 160 * 1024, "the spine's LDS");
static_assert(OS_GM + 256 <= OS_BYTES && OS_BYTES % 256 == 0, "output slot layout");
// DMA operations per chunk: K (16 pieces), T_e (6), the recurrence factors (1)
// and V (4) into a ring stage; PT (6) and gm (1) into an output slot.
constexpr int DMA_REC = 16 + NFRAG + 1 + 4;
constexpr int DMA_OUT = NFRAG + 1;
constexpr int DMA_Q = 16;

// Batches of buffer->LDS DMAs into consecutive 1 KiB pieces of LDS starting at
// the LDS byte address `lds`: M0 is set once and advanced by one scalar add per
// piece; lane and SGPR offsets are precomputed.
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
__device__ __forceinline__ void dma_x6(const Rsrc& r, uint32_t lds, const uint32_t (&v)[6], const uint32_t (&so)[6]) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %2, %1, %8 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %9 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %4, %1, %10 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %5, %1, %11 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %6, %1, %12 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %7, %1, %13 offen lds"
                 :: "s"(lds), "s"(r.d), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
                    "s"(so[0]), "s"(so[1]), "s"(so[2]), "s"(so[3]), "s"(so[4]), "s"(so[5])
                 : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma_x8(const Rsrc& r, uint32_t lds, const uint32_t (&v)[8], const uint32_t* so) {
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
// would wait for the DMA of later chunks too.  Each wave waits for its own
// LDS writes and DMA before it arrives.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt vmcnt(N), other counters free (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define GDN_VMCNT(N) (((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
// s_waitcnt lgkmcnt(N), other counters free
#define GDN_LGKMCNT(N) (15 | (3 << 14) | (7 << 4) | ((N) << 8))
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(GDN_LGKMCNT(0)); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ s16x8 join(s16x4 a, s16x4 b) {
    return s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Per-lane DMA byte offsets of the loader, chunk-independent.
struct LoadOffsets {
    uint32_t kv[8], ks[16];   // K pieces 0..15 (lane offsets repeat every 8)
    uint32_t v, vs[4];        // V pieces 0..3
    uint32_t fv[NFRAG], fs[NFRAG];   // T_e / PT fragments (granules above the diagonal out of range)
    uint32_t scv;             // the recurrence factors, 1 KiB
    uint32_t gmv;             // gm in output-lane order, 64 lanes x 4 bytes
};

__device__ __forceinline__ LoadOffsets load_offsets(int lane, int Hk, int Hv) {
    LoadOffsets o;
    const uint32_t k_row = (uint32_t)Hk * D * 2u, v_row = (uint32_t)Hv * D * 2u;
    const int rr = lane >> 4, p = lane & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j)   // piece j: rows 4 j + rr, fK = 4 rr + (j/2)%2
        o.kv[j] = rr * k_row + (uint32_t)((p ^ (4 * rr + ((j >> 1) & 1))) * 16);
#pragma unroll
    for (int j = 0; j < 16; ++j) o.ks[j] = __builtin_amdgcn_readfirstlane((uint32_t)(4 * j) * k_row);
    o.v = (uint32_t)(lane >> 2) * v_row + (uint32_t)((lane & 3) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.vs[j] = __builtin_amdgcn_readfirstlane((uint32_t)(16 * j) * v_row);
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
        o.fv[f] = frag_live(f, lane) ? 16u * lane : 0x80000000u;
        o.fs[f] = 1024u * f;
    }
    o.scv = (uint32_t)SLOT_BYTES + 16u * lane;
    o.gmv = (uint32_t)SLOT_BYTES + 4u * lane;
    return o;
}

// Where chunk cc of this workgroup's sequence starts, and its length.
struct ChunkRows {
    size_t r0;      // first token row (wave-uniform)
    uint32_t L;     // rows in the chunk, 0 past the last chunk
};
__device__ __forceinline__ ChunkRows chunk_rows(long row0, long len, int cc) {
    const long r = row0 + (long)cc * C;
    const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)r);
    const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)r >> 32));
    const long rem = len - (long)cc * C;
    ChunkRows cr;
    cr.r0 = ((size_t)rhi << 32) | rlo;
    cr.L = __builtin_amdgcn_readfirstlane((uint32_t)(rem <= 0 ? 0 : (rem < C ? rem : C)));
    return cr;
}

// Per-workgroup walk options (the segment scan's walks): V rows read as
// zero; no outputs written; the initial state is the identity; the final
// state is written as two bf16 planes (hi = bf16(x), then lo = bf16(x - hi)).
constexpr int SPINE_V_ZERO = 1, SPINE_NO_OUT = 2, SPINE_H0_EYE = 4, SPINE_SPLIT_OUT = 8;

// The segment scan's cut and buffers, passed to the spine and the combine.
// Each dense sequence b is cut into S segments of L chunks (the last one
// shorter); segment j covers tokens [j L C, min((j + 1) L C, T)).  maps
// holds, per (b S + j, v-head), the matrix N_j (fp32) and from map_m on the
// matrix M_j (bf16 hi and lo planes in the combine's A-fragment order);
// starts holds the start state of segment j >= 2, and for j = 0 the map
// walk's copy of h0 (the output walks never read h0 itself, so that h_final
// may alias it).
struct SegWalk {
    int S, L;
    int phase;             // 0: not a segment walk; 1: the map walks; 2: the output walks
    float* maps;
    long map_m;            // floats from maps to the M matrices: B S Hv D D
    float* starts;
};

struct SpineArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const unsigned char* tes;   // T_e slots (fragments, then gm by lane group and gamma_L)
    const unsigned char* pts;   // PT slots (fragments, then gm by output lane)
    long row0, len;
    long slot0;
    int nc, Hk, Hv, kh, vh, tile;
    int flags;
};

// Chunk cc's ring stage: K, T_e, the recurrence factors and V; rows past the
// chunk read as zero.
__device__ __forceinline__ void issue_rec(unsigned char* ring, const LoadOffsets& o, const SpineArgs& a, int cc) {
    const ChunkRows cr = chunk_rows(a.row0, a.len, cc);
    unsigned char* S = ring + (cc % N_RS) * RS_BYTES;
    const uint32_t base = lds_u32(S);
    const uint32_t k_row = (uint32_t)a.Hk * D * 2u;
    const Rsrc rk = make_dma_rsrc(a.k + (cr.r0 * a.Hk + a.kh) * D, cr.L * k_row);
    dma_x8(rk, base + RS_K, o.kv, &o.ks[0]);
    dma_x8(rk, base + RS_K + 8192, o.kv, &o.ks[8]);
    const Rsrc rt = make_dma_rsrc(a.tes + ((size_t)(a.slot0 + cc) * a.Hv + a.vh) * SLOT_STRIDE, SLOT_STRIDE);
    dma_x6(rt, base + RS_TE, o.fv, o.fs);
    dma16(rt, S + RS_SC, o.scv, 0);
    const uint32_t v_row = (uint32_t)a.Hv * D * 2u;
    const Rsrc rv = make_dma_rsrc(a.v + (cr.r0 * a.Hv + a.vh) * D + a.tile * TILE_COLS,
                                  (a.flags & SPINE_V_ZERO) ? 0u : cr.L * v_row);
    dma_x4(rv, base + RS_V, o.v, o.v, o.v, o.v, o.vs[0], o.vs[1], o.vs[2], o.vs[3]);
}

// Chunk cc's output slot: PT and gm.
__device__ __forceinline__ void issue_out(unsigned char* slot, const LoadOffsets& o, const SpineArgs& a, int cc) {
    const Rsrc rp = make_dma_rsrc(a.pts + ((size_t)(a.slot0 + cc) * a.Hv + a.vh) * SLOT_STRIDE, SLOT_BYTES + 256);
    dma_x6(rp, lds_u32(slot) + OS_P, o.fv, o.fs);
    dma4(rp, slot + OS_GM, o.gmv);
}

// Workgroups in a launch from which the recurrence waves issue the Q rows.
constexpr unsigned Q_SPLIT_GRID = 192;

// Chunk cc's Q rows into a Q slot, laid out as K in the ring.
__device__ __forceinline__ void issue_q(unsigned char* slot, const LoadOffsets& o, const SpineArgs& a, int cc) {
    const ChunkRows cr = chunk_rows(a.row0, a.len, cc);
    const uint32_t q_row = (uint32_t)a.Hk * D * 2u;
    const Rsrc rq = make_dma_rsrc(a.q + (cr.r0 * a.Hk + a.kh) * D, cr.L * q_row);
    const uint32_t base = lds_u32(slot);
    dma_x8(rq, base, o.kv, &o.ks[0]);
    dma_x8(rq, base + 8192, o.kv, &o.ks[8]);
}

// Half `half` of chunk cc's Q rows (rows 32 half .. + 31) into a Q slot, laid
// out as K in the ring: the K pieces 8 half .. 8 half + 7 of load_offsets,
// whose SGPR offsets qs holds.
__device__ __forceinline__ void issue_q_half(unsigned char* slot, const uint32_t (&kv)[8], const uint32_t (&qs)[8],
                                             const SpineArgs& a, int cc, int half) {
    const ChunkRows cr = chunk_rows(a.row0, a.len, cc);
    const uint32_t q_row = (uint32_t)a.Hk * D * 2u;
    const Rsrc rq = make_dma_rsrc(a.q + (cr.r0 * a.Hk + a.kh) * D, cr.L * q_row);
    dma_x8(rq, __builtin_amdgcn_readfirstlane(lds_u32(slot) + 8192u * (uint32_t)half), kv, qs);
}

// Per-lane byte offsets of the operand reads (chunk-independent).
struct FragOffsets {
    uint32_t k[4];    // K / Q fragments in the ring layout, by k-step
    uint32_t kt[4];   // K^T (transposing) fragments, by db / 2
    uint32_t v;       // V (transposing), this wave's 16 columns
};

__device__ __forceinline__ FragOffsets frag_offsets(int g, int n, int half) {
    FragOffsets o;
    const int sig0 = 8 * (n >> 2) + (n & 3);                 // sig(0, n)
    const int fKn = 4 * (n & 3) + ((n >> 2) & 1);            // fK(sig(t, n)), any t
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o.k[kk] = (uint32_t)(sig0 * 256 + 16 * ((4 * kk + g) ^ fKn));
    // transposing reads: this lane sources row 8g + kr (+ 32 kk + 4 half) and
    // the 4 columns of quarter qq of the 8-column group
    const int kr = n >> 2, qq = n & 3;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o.kt[d] = (uint32_t)((8 * g + kr) * 256 + 16 * (4 * (d ^ kr) + (qq ^ (g & 1))));
    o.v = (uint32_t)((8 * g + kr) * 64 + 32 * half + 8 * qq);
    return o;
}

// A recurrence wave's operands of one chunk, all from its ring stage: the K
// fragments of X (by k-step and tile), the transposed K fragments of the
// update (by state block and k-step), V in accumulator layout, the T_e
// fragments, gm of this lane's accumulator rows (by tile) and gamma_L.
struct RecOps {
    s16x8 kx[4][4];
    s16x8 kt[8][2];
    s16x4 vv[4];
    s16x8 te[NFRAG];
    f32x4 gm[4];
    float gl;
};

// This lane's read addresses in one ring stage: a handful of 32-bit LDS
// bases, every read a constant offset from one of them.  The stage's base
// address passes through readfirstlane, so the compiler takes it as an opaque
// wave-uniform value and does not rebuild each address from the ring index.
typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;
__device__ __forceinline__ lds_cptr lds_at(uint32_t a) { return (lds_cptr)(uintptr_t)a; }
struct StageAddr {
    uint32_t k[4];    // K fragments of X, by k-step
    uint32_t kt[4];   // transposed K fragments, by db / 2
    uint32_t v;       // V
    uint32_t te;      // T_e fragments
    uint32_t gm;      // gm of this lane group's rows
    uint32_t gl;      // gamma_L (wave-uniform)
};
__device__ __forceinline__ StageAddr stage_addr(const unsigned char* S, const FragOffsets& fo, int g, int lane) {
    const uint32_t sb = __builtin_amdgcn_readfirstlane(lds_addr(S));
    StageAddr s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s.k[i] = sb + RS_K + fo.k[i];
        s.kt[i] = sb + RS_K + fo.kt[i];
    }
    s.v = sb + RS_V + fo.v;
    s.te = sb + RS_TE + 16 * lane;
    s.gm = sb + RS_SC + 64 * g;
    s.gl = sb + RS_SC + 256;
    return s;
}
__device__ __forceinline__ s16x8 lds_rd16(uint32_t base, int off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) s16x8*>(lds_at(base) + off);
}
__device__ __forceinline__ s16x4 lds_rdtr(uint32_t base, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_at(base) + off));
}
#define GDN_KX(A, kk, cb) lds_rd16((A).k[kk], 256 * sig_tile(cb))
#define GDN_KT(A, db, kk) join(lds_rdtr((A).kt[(db) >> 1], 8192 * (kk) + 8 * ((db) & 1)), \
                               lds_rdtr((A).kt[(db) >> 1], 8192 * (kk) + 1024 + 8 * ((db) & 1)))
#define GDN_VV(A, cb) lds_rdtr((A).v, 64 * sig_tile(cb))
#define GDN_TE(A, f) lds_rd16((A).te, FRAG_BYTES * (f))
#define GDN_GM(A, cb) (*reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lds_at((A).gm) + 16 * (cb)))
#define GDN_GL(A) (*reinterpret_cast<const __attribute__((address_space(3))) float*>(lds_at((A).gl)))

// Every ring read of one chunk at once (the first chunk, before the walk).
__device__ __forceinline__ void rec_read_lds(RecOps& l, const unsigned char* S0, const FragOffsets& fo,
                                             int g, int lane) {
    const StageAddr S = stage_addr(S0, fo, g, lane);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) l.kx[kk][cb] = GDN_KX(S, kk, cb);
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) l.kt[db][kk] = GDN_KT(S, db, kk);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) l.vv[cb] = GDN_VV(S, cb);
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) l.te[f] = GDN_TE(S, f);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) l.gm[cb] = GDN_GM(S, cb);
    l.gl = GDN_GL(S);
}

// R = V - gm X on tile cb: register r is row sig(cb, 4g + r), whose gm this
// lane holds in gm[r]
__device__ __forceinline__ void resid(f32x4& x, const s16x4 vv, const f32x4 gm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = fmaf(-gm[r], x[r], bf16_bits_to_f32((uint16_t)vv[r]));
}

// One recurrence step on chunk c (operands o), 16 columns; the next chunk's
// operands go into on, read from ring stage Sn between this step's products.
// The bf16 state and R go to exchange slot E.
__device__ __forceinline__ void rec_step(f32x4 (&h)[8], const RecOps& o, RecOps& on, const unsigned char* Sn0,
                                         unsigned char* E, const FragOffsets& fo, int g, int lane)
{
    const StageAddr Sn = stage_addr(Sn0, fo, g, lane);
    // state -> bf16 B operand (to the output partner after X is issued)
    s16x8 hb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) hb[kk] = frag_b(h[2 * kk], h[2 * kk + 1]);
    sched_fence();
    // X = K h, with the next chunk's update fragments of state blocks 0..3 read
    // in between; h scaled by gamma_L meanwhile (hb holds the state before it)
    f32x4 X[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) X[cb] = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            X[cb] = mfma_bf16(o.kx[kk][cb], hb[kk], X[cb]);
            if (cb & 1) {
                const int db = 2 * kk + (cb >> 1);   // 0..7 in order
                if (db < 4) {
                    on.kt[db][0] = GDN_KT(Sn, db, 0);
                    on.kt[db][1] = GDN_KT(Sn, db, 1);
                } else {
                    h[2 * (db - 4)] = h[2 * (db - 4)] * o.gl;
                    h[2 * (db - 4) + 1] = h[2 * (db - 4) + 1] * o.gl;
                }
            }
            sched_fence();
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) *reinterpret_cast<s16x8*>(E + 1024 * kk + 16 * lane) = hb[kk];
    sched_fence();
    // the next chunk's T_e and decay factors, and K fragments of X into the
    // registers X just read
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) on.te[f] = GDN_TE(Sn, f);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) on.gm[cb] = GDN_GM(Sn, cb);
    on.gl = GDN_GL(Sn);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) on.kx[kk][cb] = GDN_KX(Sn, kk, cb);
    sched_fence();
    // R = V - gm X, rounded to the B operand of Delta_e = T_e R (and to the
    // output partner once Delta_e is issued)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) resid(X[cb], o.vv[cb], o.gm[cb]);
    const s16x8 rb0 = frag_b(X[0], X[1]), rb1 = frag_b(X[2], X[3]);
    sched_fence();
    f32x4 Dl[4];
    Dl[0] = mfma_bf16(o.te[0], rb0, zero4());
    on.kx[2][0] = GDN_KX(Sn, 2, 0);
    sched_fence();
    Dl[1] = mfma_bf16(o.te[1], rb0, zero4());
    on.kx[2][1] = GDN_KX(Sn, 2, 1);
    sched_fence();
    Dl[2] = mfma_bf16(o.te[2], rb0, zero4());
    on.kx[2][2] = GDN_KX(Sn, 2, 2);
    sched_fence();
    Dl[3] = mfma_bf16(o.te[3], rb0, zero4());
    on.kx[2][3] = GDN_KX(Sn, 2, 3);
    sched_fence();
    Dl[2] = mfma_bf16(o.te[4], rb1, Dl[2]);
    Dl[3] = mfma_bf16(o.te[5], rb1, Dl[3]);
    sched_fence();
    *reinterpret_cast<s16x8*>(E + 4096 + 16 * lane) = rb0;
    *reinterpret_cast<s16x8*>(E + 5120 + 16 * lane) = rb1;
    sched_fence();
    const s16x8 ds0 = frag_b(Dl[0], Dl[1]), ds1 = frag_b(Dl[2], Dl[3]);
    sched_fence();
    // h <- gamma_L h + K^T Delta_e, with the rest of the next chunk's ring reads
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        h[db] = mfma_bf16(o.kt[db][0], ds0, h[db]);
        if (db < 4) on.kx[3][db] = GDN_KX(Sn, 3, db);
        if (db == 4) on.kt[4][0] = GDN_KT(Sn, 4, 0);
        if (db == 5) on.kt[4][1] = GDN_KT(Sn, 4, 1);
        if (db == 6) on.kt[5][0] = GDN_KT(Sn, 5, 0);
        if (db == 7) on.kt[5][1] = GDN_KT(Sn, 5, 1);
        sched_fence();
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        h[db] = mfma_bf16(o.kt[db][1], ds1, h[db]);
        if (db == 0) on.kt[6][0] = GDN_KT(Sn, 6, 0);
        if (db == 1) on.kt[6][1] = GDN_KT(Sn, 6, 1);
        if (db == 2) on.kt[7][0] = GDN_KT(Sn, 7, 0);
        if (db == 3) on.kt[7][1] = GDN_KT(Sn, 7, 1);
        if (db == 4) { on.vv[0] = GDN_VV(Sn, 0); on.vv[1] = GDN_VV(Sn, 1); }
        if (db == 5) { on.vv[2] = GDN_VV(Sn, 2); on.vv[3] = GDN_VV(Sn, 3); }
        sched_fence();
    }
}
#undef GDN_KX
#undef GDN_KT
#undef GDN_VV
#undef GDN_TE
#undef GDN_GM
#undef GDN_GL
// ring reads a recurrence step issues after its last exchange write (R, after
// Delta_e): K fragments of k-step 3 (4), transposed fragments of state blocks
// 4..7 (16 transposing reads) and V (4)
constexpr int REC_READS_AFTER_EX = 24;
static_assert(REC_READS_AFTER_EX >= 15, "the wait below then allows at most 15 outstanding");

// The output wave, chunk c: O = gm (Q h) + PT R for the workgroup's 32
// columns, with Q from Q slot Qs, PT and gm from output slot Os, and the bf16
// state and R of column half u from exchange slot E[u].  The products are
// formed transposed: a B-operand fragment of h or R is the A operand of its
// transpose and an A-operand fragment of Q or PT the B operand of its
// transpose, so lane (g, n) register r of tile cb ends up holding
// O[sig(cb, n)][4g + r] of its column half, four consecutive columns of one
// row.  Each Q fragment serves both halves; the next k-step's fragments are
// read while this one's products run.  `ro` covers exactly the chunk's rows;
// lane_off[u] is this lane's byte offset within a row: for fp32 outputs that
// of its four columns of half u, for bf16 that of the eight columns it
// stores after the lane swaps (both entries).
template <bool kOutF32>
__device__ __forceinline__ void out_step(const unsigned char* Qs, const unsigned char* Os, const unsigned char* E0,
                                         const unsigned char* E1, const FragOffsets& fo, rsrc_t ro,
                                         const uint32_t (&lane_off)[2], const uint32_t (&soff)[4], int n, int lane)
{
    s16x8 qf[2][4], hf[2][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) qf[0][cb] = lds_read16(Qs + fo.k[0] + 256 * sig_tile(cb));
    hf[0][0] = lds_read16(E0 + 16 * lane);
    hf[0][1] = lds_read16(E1 + 16 * lane);
    f32x4 Y[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) Y[u][cb] = zero4();
    s16x8 rb[2][2], pf[NFRAG];
    float4 g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int p = kk & 1;
        if (kk < 3) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) qf[p ^ 1][cb] = lds_read16(Qs + fo.k[kk + 1] + 256 * sig_tile(cb));
            hf[p ^ 1][0] = lds_read16(E0 + 1024 * (kk + 1) + 16 * lane);
            hf[p ^ 1][1] = lds_read16(E1 + 1024 * (kk + 1) + 16 * lane);
        }
        if (kk == 2) {
            g4 = *reinterpret_cast<const float4*>(Os + OS_GM + 16 * n);
            rb[0][0] = lds_read16(E0 + 4096 + 16 * lane);
            rb[1][0] = lds_read16(E1 + 4096 + 16 * lane);
            rb[0][1] = lds_read16(E0 + 5120 + 16 * lane);
            rb[1][1] = lds_read16(E1 + 5120 + 16 * lane);
        }
        if (kk == 3) {
#pragma unroll
            for (int f = 0; f < NFRAG; ++f) pf[f] = lds_read16(Os + OS_P + 1024 * f + 16 * lane);
        }
        sched_fence();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            Y[0][cb] = mfma_bf16(hf[p][0], qf[p][cb], Y[0][cb]);
            Y[1][cb] = mfma_bf16(hf[p][1], qf[p][cb], Y[1][cb]);
        }
        sched_fence();
    }
    // O = gm (Q h) + PT R by pairs of tiles (2p, 2p + 1), both column halves;
    // rows past a partial chunk fall outside `ro`.  Nothing here reads the
    // outputs back: the stores are nontemporal.
    const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        f32x4 O[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int cb = 2 * p + e;
                O[u][e] = mfma_bf16(rb[u][0], pf[cb], Y[u][cb] * gs[cb]);
                if (p == 1) O[u][e] = mfma_bf16(rb[u][1], pf[cb + 2], O[u][e]);
            }
        if constexpr (kOutF32) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const f32x4 v = O[u][e];
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4v{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                                  __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                           ro, lane_off[u], soff[2 * p + e], CPOL_NT);
                }
        } else {
            // bf16 (hardware RNE conversion): a lane holds 8 bytes of its
            // row's 64 (the workgroup's 32 columns).  Two rounds of permlane16
            // swaps put each row's 64 bytes into the lanes n, 16 + n, 32 + n,
            // 48 + n: first between the pair's tiles within one column half
            // (the even lane group then holds 8 columns of tile 2p's row, the
            // odd group the same columns of tile 2p + 1's), then between the
            // halves, after which lane group g holds columns 8 (g / 2) +
            // 16 (g % 2) .. + 7 of one row, of tile 2p in the first register
            // and of tile 2p + 1 in the second.  Each store then writes 16 rows
            // as 64-byte pieces: half the instructions, and half the pieces,
            // of one 8-byte store per tile and half.
            u32x4v half_rows[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const f32x4 a = O[u][0], b = O[u][1];
                const auto s0 = __builtin_amdgcn_permlane16_swap(bf16x2_bits(a[0], a[1]), bf16x2_bits(b[0], b[1]),
                                                                 false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(bf16x2_bits(a[2], a[3]), bf16x2_bits(b[2], b[3]),
                                                                 false, false);
                half_rows[u] = u32x4v{s0[0], s1[0], s0[1], s1[1]};
            }
            u32x4v r0, r1;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const auto t = __builtin_amdgcn_permlane16_swap(half_rows[0][d], half_rows[1][d], false, false);
                r0[d] = t[0];
                r1[d] = t[1];
            }
            __builtin_amdgcn_raw_buffer_store_b128(r0, ro, lane_off[0], soff[2 * p], CPOL_NT);
            __builtin_amdgcn_raw_buffer_store_b128(r1, ro, lane_off[0], soff[2 * p + 1], CPOL_NT);
        }
    }
}

template <bool kOutF32>
__global__ void __launch_bounds__(256, 1)
gdn_spine_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const float* h0, void* __restrict__ out, float* h_final,
                 const unsigned char* __restrict__ tes, const unsigned char* __restrict__ pts,
                 int T, int Hk, int Hv, const int32_t* __restrict__ cu,
                 const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ order,
                 int nc_dense, long n_slots, SegWalk sw)
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
    SpineArgs a;
    a.vh = lin / N_TILES;
    a.tile = lin % N_TILES;
    a.kh = a.vh / (Hv / Hk);
    a.q = q; a.k = k; a.v = v; a.tes = tes; a.pts = pts; a.Hk = Hk; a.Hv = Hv;
    const size_t DD = (size_t)D * D;
    // the start state read, the final state written (per v-head matrices)
    const float* hin;
    float* hout;
    float* hcopy = nullptr;   // where the start state is also written (segment 0's copy of h0)
    int flags = 0;
    if (sw.phase == 0) {
        const int b = order ? order[blockIdx.y] : (int)blockIdx.y;
        seq_rows(cu, b, T, &a.row0, &a.len);
        a.slot0 = cu ? (long)chunk_base[b] : (long)b * nc_dense;
        hin = h0 ? h0 + ((size_t)b * Hv + a.vh) * DD : nullptr;
        hout = h_final ? h_final + ((size_t)b * Hv + a.vh) * DD : nullptr;
    } else {
        // phase 1, per sequence: N_0 .. N_{S-2} (N_0 walked from h0), then
        // M_1 .. M_{S-2}; phase 2: segment j from its start state, the last
        // one writing the final state
        int b, j;
        if (sw.phase == 1) {
            const int per_seq = 2 * sw.S - 3, r = (int)blockIdx.y % per_seq;
            b = (int)blockIdx.y / per_seq;
            const bool m = r >= sw.S - 1;
            j = m ? r - sw.S + 2 : r;
            const size_t mat = ((size_t)b * sw.S + j) * Hv + a.vh;
            hin = !m && j == 0 && h0 ? h0 + ((size_t)b * Hv + a.vh) * DD : nullptr;
            // segment 0's walk also copies h0 for the output walks, which
            // never read h0 itself (h_final may alias it)
            if (hin) hcopy = sw.starts + mat * DD;
            hout = m ? sw.maps + sw.map_m + mat * DD : sw.maps + mat * DD;
            flags = m ? SPINE_V_ZERO | SPINE_NO_OUT | SPINE_H0_EYE | SPINE_SPLIT_OUT : SPINE_NO_OUT;
        } else {
            b = (int)blockIdx.y / sw.S;
            j = (int)blockIdx.y % sw.S;
            const size_t mat = ((size_t)b * sw.S + j) * Hv + a.vh;
            // segment 0 starts from the map walk's copy of h0: h_final, which
            // the last segment writes in this same launch, may alias h0
            hin = j == 0 ? (h0 ? sw.starts + mat * DD : nullptr)
                         : j == 1 ? sw.maps + (mat - Hv) * DD : sw.starts + mat * DD;
            hout = j == sw.S - 1 && h_final ? h_final + ((size_t)b * Hv + a.vh) * DD : nullptr;
        }
        const long t0 = (long)j * sw.L * C;
        a.row0 = (long)b * T + t0;
        a.len = min((long)sw.L * C, (long)T - t0);
        a.slot0 = (long)b * nc_dense + (long)j * sw.L;
    }
    int nc = (int)((a.len + C - 1) / C);
    // Only a decreasing cu_seqlens (a broken precondition) can make this
    // bind; it keeps every read inside the workspace.
    if (a.slot0 + nc > n_slots) nc = (int)max(0L, n_slots - a.slot0);
    a.nc = nc;
    a.flags = flags;
    const int half = w & 1;   // which 16 of the workgroup's 32 columns
    const FragOffsets fo = frag_offsets(g, n, half);
    unsigned char* ex = lds + EX_BASE + 2 * half * EX_BYTES;   // this column half's exchange, parity 0

    // uniform over the workgroup
    const bool q_split = gridDim.x * gridDim.y >= Q_SPLIT_GRID && !(flags & SPINE_NO_OUT);
    if (w == 0) {   // the loader: in step c, chunk c's Q, chunk c + 3's ring stage and chunk c + 1's output slot
        const LoadOffsets o = load_offsets(lane, Hk, Hv);
        for (int cc = 0; cc < 2 && cc < nc; ++cc) issue_rec(ring, o, a, cc);
        __builtin_amdgcn_s_waitcnt(GDN_VMCNT(0));
        ring_barrier();   // chunks 0 and 1 are in the ring
        if (2 < nc) issue_rec(ring, o, a, 2);
        if (0 < nc) issue_out(lds + OS_BASE, o, a, 0);
        for (int c = 0; c <= nc; ++c) {
            ring_barrier();
            // stage c % 3 held chunk c, whose ring reads ended in step c - 1 (in
            // the prologue for chunk 0); slot (c + 1) % 3 held chunk c - 2, read
            // in step c - 1
            // Q slot c % 2 held chunk c - 2, read in step c - 1
            if (!q_split && c < nc) issue_q(lds + QS_BASE + (c & 1) * QS_BYTES, o, a, c);
            const bool rr = c + 3 < nc, oo = c + 1 < nc;
            if (rr) issue_rec(ring, o, a, c + 3);
            if (oo) issue_out(lds + OS_BASE + ((c + 1) % N_OS) * OS_BYTES, o, a, c + 1);
            // chunk c's Q and what was issued before this step (chunk c + 2's
            // stage, chunk c's slot) land before the next barrier
            if (rr && oo) __builtin_amdgcn_s_waitcnt(GDN_VMCNT(DMA_REC + DMA_OUT));
            else if (rr) __builtin_amdgcn_s_waitcnt(GDN_VMCNT(DMA_REC));
            else if (oo) __builtin_amdgcn_s_waitcnt(GDN_VMCNT(DMA_OUT));
            else __builtin_amdgcn_s_waitcnt(GDN_VMCNT(0));
        }
        return;
    }
    if (w == 1) {   // the output wave: chunk c - 1 in step c
        constexpr uint32_t es = kOutF32 ? 4u : 2u;
        const uint32_t rs = __builtin_amdgcn_readfirstlane((uint32_t)Hv * D * es);
        uint32_t lane_off[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            lane_off[u] = (uint32_t)(8 * (n >> 2) + (n & 3)) * rs +
                          (uint32_t)(a.tile * TILE_COLS + (kOutF32 ? 16 * u + 4 * g : 8 * (g >> 1) + 16 * (g & 1))) * es;
        uint32_t soff[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) soff[cb] = (uint32_t)sig_tile(cb) * rs;
        const uint32_t rlo = __builtin_amdgcn_readfirstlane((uint32_t)a.row0);
        const uint32_t rhi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)a.row0 >> 32));
        char* obase = reinterpret_cast<char*>(out) + ((((size_t)rhi << 32) | rlo) * Hv + a.vh) * D * es;
        const FragOffsets fq = frag_offsets(g, n, 0);
        ring_barrier();   // the prologue
        for (int c = 0; c <= nc; ++c) {
            ring_barrier();
            if (c >= 1) {
                const long rem = a.len - (long)(c - 1) * C;
                const rsrc_t ro = make_rsrc(obase + (size_t)(c - 1) * C * rs,
                                            (flags & SPINE_NO_OUT) ? 0u : (uint32_t)min((long)C, rem) * rs);
                const int par = (c - 1) & 1;
                out_step<kOutF32>(lds + QS_BASE + par * QS_BYTES, lds + OS_BASE + ((c + 2) % N_OS) * OS_BYTES,
                                  lds + EX_BASE + par * EX_BYTES, lds + EX_BASE + (2 + par) * EX_BYTES, fq, ro,
                                  lane_off, soff, n, lane);
            }
            // every read of this step's slots and exchange is done before the barrier
            wait_lgkm0();
        }
        return;
    }

    // recurrence waves
    f32x4 h[8];
    const int col = a.tile * TILE_COLS + 16 * half + n;
    // state row of h[db][r] in this lane: sig(db, 4g + r)
    if (hin) {   // one uniform branch: all 32 loads in flight together
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[db][r] = hin[(size_t)(sig_tile(db) + 8 * g + r) * D + col];
        if (hcopy) {
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) hcopy[(size_t)(sig_tile(db) + 8 * g + r) * D + col] = h[db][r];
        }
    } else if (flags & SPINE_H0_EYE) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[db][r] = sig_tile(db) + 8 * g + r == col ? 1.f : 0.f;
    } else {
#pragma unroll
        for (int db = 0; db < 8; ++db) h[db] = zero4();
    }
    RecOps oA, oB;
    // one barrier per step after the prologue's, nc + 1 steps as the other
    // waves; the exchange
    // writes are complete before each barrier (the LDS operations of one wave
    // complete in order, and more ring reads than can be in flight follow the
    // last write).  Written so that the second step of a pair is reachable only
    // through the first, which keeps the compiler's waits on the prefetched
    // reads where they are used.
    ring_barrier();   // the prologue: chunks 0 and 1 are in the ring
    if (nc > 0) rec_read_lds(oA, ring, fo, g, lane);
    // everything loaded before the walk has arrived (chunk 0's stage is free
    // for the loader from step 0 on): the loop's waits then account only for
    // the walk's own reads
    __builtin_amdgcn_s_waitcnt(0);
    ring_barrier();   // step 0
    // With q_split, step c starts with this wave's half of chunk c's Q rows
    // into Q slot c % 2 (chunk c - 2's, read by the output wave in step
    // c - 1); the wave has no other vector-memory operation in the walk, so
    // vmcnt(0) before the barrier that ends the step is exactly those pieces.
    const LoadOffsets lq = load_offsets(lane, Hk, Hv);
    uint32_t qs[8];   // the SGPR offsets of K pieces 8 half .. 8 half + 7
#pragma unroll
    for (int j = 0; j < 8; ++j)
        qs[j] = __builtin_amdgcn_readfirstlane((uint32_t)(4 * (8 * half + j)) * (uint32_t)Hk * D * 2u);
    for (int c = 0; c < nc; c += 2) {
        if (q_split) issue_q_half(lds + QS_BASE, lq.kv, qs, a, c, half);
        rec_step(h, oA, oB, ring + ((c + 1) % N_RS) * RS_BYTES, ex, fo, g, lane);
        __builtin_amdgcn_s_waitcnt(GDN_LGKMCNT(15) & GDN_VMCNT(0));
        ring_barrier();
        if (c + 1 >= nc) break;
        if (q_split) issue_q_half(lds + QS_BASE + QS_BYTES, lq.kv, qs, a, c + 1, half);
        rec_step(h, oB, oA, ring + ((c + 2) % N_RS) * RS_BYTES, ex + EX_BYTES, fo, g, lane);
        __builtin_amdgcn_s_waitcnt(GDN_LGKMCNT(15) & GDN_VMCNT(0));
        ring_barrier();
    }
    if (hout && (flags & SPINE_SPLIT_OUT)) {
        // the combine's A-fragment order: element (row, col) in fragment
        // (row / 16, col / 32), plane p, lane 16 ((col % 32) / 8) + row % 16,
        // element col % 8, each fragment 1 KiB
        uint16_t* m16 = reinterpret_cast<uint16_t*>(hout);
        const int kk = col >> 5, gc = (col & 31) >> 3, ec = col & 7;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = sig_tile(db) + 8 * g + r;
                const size_t e = ((size_t)(((row >> 4) * 4 + kk) * 2) * 64 + 16 * gc + (row & 15)) * 8 + ec;
                const short x = bf16_bits(h[db][r]);
                m16[e] = (uint16_t)x;
                m16[e + 512] = (uint16_t)bf16_bits(h[db][r] - bf16_bits_to_f32((uint16_t)x));
            }
    } else if (hout) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                hout[(size_t)(sig_tile(db) + 8 * g + r) * D + col] = h[db][r];
    }
}

// ---------------------------------------------------------------------------
// The segment scan (ssm_gdn_tc_route.rs, the spine entries: the spine walks
// the chunk states S_c in order; the map of one chunk, h -> M_c h + N_c, is
// affine in h).  When the spine's workgroups fill only a small part of the
// chip (few sequences and v-heads), each dense sequence is cut into S
// segments of whole chunks and:
//   1. one spine launch walks, all at once, segment 0 from h0 (its end state
//      N_0), segments 1 .. S-2 from h = 0 (N_j) and segments 1 .. S-2 from
//      h = I with V read as zero (the linear part M_j, written as bf16 hi/lo
//      planes); no outputs are written;
//   2. gdn_segment_combine_kernel runs the maps in order per (sequence,
//      v-head, 32 columns): start(1) = N_0, start(j) = M_{j-1} start(j-1) +
//      N_{j-1};
//   3. a second spine launch walks every segment from its start state,
//      writing the outputs, and the last segment writes the final state
//      (segment 0 starts from a copy of h0 that its map walk wrote, so
//      h_final may alias h0 as in the plain route).
// The WY prep runs once; every walk reads the same workspace slots.  The
// products in 2. are formed from bf16 splits of both fp32 operands
// (x = hi + lo; A B ~ Ahi Bhi + Ahi Blo + Alo Bhi), about 16 bits of each.

// One workgroup per (sequence, v-head, 32 columns); wave w of 8 forms rows
// 16 w .. 16 w + 15 of each product.  The start state lives in LDS as bf16 hi
// and lo planes, column-major ([32 columns][128 rows + 8]) so that an MFMA B
// fragment (8 consecutive rows of one column) is one 16-byte read.  The
// operands of step j + 2 are loaded while step j runs.
constexpr int CMB_LD = D + 8;
constexpr int CMB_WAVES = 8;
constexpr int CMB_RING = 4;
constexpr int CMB_MAX_STEPS = 8;   // S - 2 <= 8: at most 10 segments per sequence

struct CombineOps {
    s16x8 a[4][2];       // M_j rows 16 w + n, k = 32 kk + 8 g .. + 7; hi, lo
    float nv[2][4];      // N_j rows 16 w + 4 g + r, column 16 ct + n
};
// M_j as the map walk writes it: per 16-row block w and 32-column step kk,
// the hi then the lo plane of the A fragment, 64 lanes x 16 bytes each, so
// that every fragment load is one contiguous 1 KiB.

__global__ void __launch_bounds__(64 * CMB_WAVES)
gdn_segment_combine_kernel(SegWalk sw, int Hv)
{
    __shared__ __attribute__((aligned(16))) uint16_t sh[2][TILE_COLS][CMB_LD];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int vh = blockIdx.x / N_TILES, tile = blockIdx.x % N_TILES, b = blockIdx.y;
    const int c0 = tile * TILE_COLS;
    const size_t DD = (size_t)D * D;
    const int row = 16 * w + 4 * g;   // this lane's first accumulator row
    auto mat = [&](int j) { return ((size_t)b * sw.S + j) * Hv + vh; };
    auto load = [&](CombineOps& o, int j) {
        const uint16_t* m = reinterpret_cast<const uint16_t*>(sw.maps + sw.map_m + mat(j) * DD);
        const float* nj = sw.maps + mat(j) * DD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                o.a[kk][p] = *reinterpret_cast<const s16x8*>(m + ((size_t)((w * 4 + kk) * 2 + p) * 64 + lane) * 8);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) o.nv[ct][r] = nj[(size_t)(row + r) * D + c0 + 16 * ct + n];
    };
    // x (rows row .. row + 3 of column c) into the planes
    auto put = [&](const float (&x)[4], int c) {
        s16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi[r] = bf16_bits(x[r]);
            lo[r] = bf16_bits(x[r] - bf16_bits_to_f32((uint16_t)hi[r]));
        }
        *reinterpret_cast<s16x4*>(&sh[0][c][row]) = hi;
        *reinterpret_cast<s16x4*>(&sh[1][c][row]) = lo;
    };
    // step j: start(j) = M_{j-1} start(j-1) + N_{j-1}, with o = (M_{j-1}, N_{j-1})
    auto step = [&](const CombineOps& o, int j) {
        f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const s16x8 bh = *reinterpret_cast<const s16x8*>(&sh[0][16 * ct + n][32 * kk + 8 * g]);
                const s16x8 bl = *reinterpret_cast<const s16x8*>(&sh[1][16 * ct + n][32 * kk + 8 * g]);
                acc[ct] = mfma_bf16(o.a[kk][0], bh, acc[ct]);
                acc[ct] = mfma_bf16(o.a[kk][0], bl, acc[ct]);
                acc[ct] = mfma_bf16(o.a[kk][1], bh, acc[ct]);
            }
        // every wave has read start(j - 1); a plain barrier, which leaves the
        // operand loads of later steps in flight
        wait_lgkm0();
        ring_barrier();
        float* st = sw.starts + mat(j) * DD;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = acc[ct][r] + o.nv[ct][r];
                st[(size_t)(row + r) * D + c0 + 16 * ct + n] = x[r];
            }
            put(x, 16 * ct + n);
        }
        wait_lgkm0();
        ring_barrier();
    };
    // the operands of up to CMB_RING steps in flight; the walk is unrolled
    // in full, so that each step waits only for its own operands
    const int last = sw.S - 2;
    CombineOps o[CMB_RING];
    float x[2][4];
    {   // start(1) = N_0
        const float* n0 = sw.maps + mat(0) * DD;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[ct][r] = n0[(size_t)(row + r) * D + c0 + 16 * ct + n];
    }
    // the first step's operands ahead of the barrier, the others after it:
    // every wave's N_0 rows then reach the compute unit ahead of the bulk of
    // the fragment loads
    load(o[0], 1);
    put(x[0], n);
    put(x[1], 16 + n);
    wait_lgkm0();
    ring_barrier();
#pragma unroll
    for (int i = 1; i < CMB_RING; ++i) load(o[i], min(1 + i, last));   // past the last map: read it again
#pragma unroll
    for (int t = 0; t < CMB_MAX_STEPS; ++t) {
        if (2 + t >= sw.S) break;
        step(o[t % CMB_RING], 2 + t);
        if (t + CMB_RING < CMB_MAX_STEPS) load(o[t % CMB_RING], min(1 + t + CMB_RING, last));
    }
}

// base[B + 1] then order[B]
size_t table_bytes(int B) { return ((size_t)(2 * B + 1) * sizeof(int32_t) + 255) & ~(size_t)255; }

long slot_count(int B, int T, bool packed) {
    return packed ? (long)(T + C - 1) / C + B : (long)B * ((T + C - 1) / C);
}

// The segment scan's cut of dense sequences: segments per sequence (0: the
// plain spine) and chunks per segment.  It is taken when the spine's
// workgroups (B Hv 4) fill at most a third of the 256 compute units; S is
// the largest count whose map walks (2 S - 3 per sequence and v-head tile)
// still fit on the chip in one pass, at least 3 and at most 10 (the combine's
// unrolled steps).
struct SegmentCut { int S, L; };
SegmentCut segment_cut(int B, int T, int Hv, bool packed) {
    SegmentCut sc{0, 0};
    if (packed || T <= 0) return sc;
    const int nc = (T + C - 1) / C;
    const long wgs = (long)B * Hv * N_TILES;
    const long s0 = min(min((long)nc, (256L / max(wgs, 1L) + 3) / 2), (long)CMB_MAX_STEPS + 2);
    if (s0 < 3) return sc;
    const int L = (int)((nc + s0 - 1) / s0);
    const int S = (nc + L - 1) / L;
    if (S < 3) return sc;
    sc.S = S;
    sc.L = L;
    return sc;
}

}  // namespace

size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv, bool packed, bool segmented)
{
    (void)Hk;
    const size_t slots = (size_t)slot_count(B, T, packed) * Hv * 2 * SLOT_STRIDE;
    const SegmentCut sc = segmented ? segment_cut(B, T, Hv, packed) : SegmentCut{0, 0};
    const size_t plain = table_bytes(B) + slots;
    if (sc.S == 0) return plain;
    // the segment scan's: the slots, then N_j, M_j and start(j) per (segment,
    // v-head); the size covers both routes
    const size_t seg = slots + 3 * (size_t)B * sc.S * Hv * D * D * sizeof(float);
    return seg > plain ? seg : plain;
}

bool prefill_mfma_accepts(const PrefillArgs& a)
{
    return a.io_dtype == 1 && a.dk == D && a.dv == D && a.chunk == C;
}

size_t prefill_workspace_need(int B, int T, int Hk, int Hv, int dk, int dv, int chunk, int io_dtype,
                              bool packed, bool segmented)
{
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1) return 0;
    PrefillArgs a{};
    a.io_dtype = io_dtype; a.dk = dk; a.dv = dv; a.chunk = chunk;
    if (!prefill_mfma_accepts(a)) return 0;  // the generic kernel keeps everything in LDS
    return prefill_mfma_workspace_bytes(B, T, Hk, Hv, packed, segmented);
}

Geometry prefill_mfma_geometry(const PrefillArgs& a)
{
    const SegmentCut sc = a.segmented ? segment_cut(a.B, a.T, a.Hv, a.cu_seqlens != nullptr) : SegmentCut{0, 0};
    if (sc.S > 0) {
        Geometry g{"gdn_wy_prep_kernel+gdn_spine_kernel(segment maps)+gdn_segment_combine_kernel"
                   "+gdn_spine_kernel(segment outputs)",
                   {(unsigned)(a.Hv * N_TILES), (unsigned)(a.B * sc.S), 1u}, 256u, (unsigned)SPINE_LDS};
        return g;
    }
    Geometry g{"gdn_wy_prep_kernel+gdn_spine_kernel", {(unsigned)(a.Hv * N_TILES), (unsigned)a.B, 1u}, 256u,
               (unsigned)SPINE_LDS};
    return g;
}

int prefill_mfma_segments(const PrefillArgs& a)
{
    return a.segmented ? segment_cut(a.B, a.T, a.Hv, a.cu_seqlens != nullptr).S : 0;
}

namespace {
template <bool kOutF32>
void launch_spine(const PrefillArgs& a, dim3 grid, const float* h0, float* h_final, const unsigned char* tbs,
                  const unsigned char* pps, const int32_t* base, const int32_t* order, int nc_dense, long n_slots,
                  SegWalk sw, hipStream_t s)
{
    hipLaunchKernelGGL((gdn_spine_kernel<kOutF32>), grid, dim3(256), 0, s, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, h0, a.out, h_final, tbs, pps, a.T, a.Hk,
                       a.Hv, a.cu_seqlens, base, order, nc_dense, n_slots, sw);
}

void launch_spine(const PrefillArgs& a, dim3 grid, const float* h0, float* h_final, const unsigned char* tbs,
                  const unsigned char* pps, const int32_t* base, const int32_t* order, int nc_dense, long n_slots,
                  SegWalk sw, hipStream_t s)
{
    if (a.out_dtype == 0)
        launch_spine<true>(a, grid, h0, h_final, tbs, pps, base, order, nc_dense, n_slots, sw, s);
    else
        launch_spine<false>(a, grid, h0, h_final, tbs, pps, base, order, nc_dense, n_slots, sw, s);
}

void launch_prep(const PrefillArgs& a, unsigned char* tbs, unsigned char* pps, const int32_t* base,
                 int nc_dense, long n_slots, hipStream_t s)
{
    const int G = a.Hv / a.Hk, nw = G < 4 ? G : 4;
    hipLaunchKernelGGL(gdn_wy_prep_kernel, dim3((unsigned)n_slots, a.Hk, (unsigned)((G + nw - 1) / nw)),
                       dim3(64 * nw), prep_lds_bytes(nw), s,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, a.log_g, a.beta, tbs, pps,
                       a.B, a.T, a.Hk, a.Hv, a.cu_seqlens, base, nc_dense);
}

hipError_t launch_prefill_segmented(const PrefillArgs& a, SegmentCut sc, hipStream_t s)
{
    const int nc = (a.T + C - 1) / C;
    const long n_slots = (long)a.B * nc;
    unsigned char* tbs = reinterpret_cast<unsigned char*>(a.workspace);
    unsigned char* pps = tbs + (size_t)n_slots * a.Hv * SLOT_STRIDE;
    SegWalk sw{};
    sw.S = sc.S;
    sw.L = sc.L;
    sw.maps = reinterpret_cast<float*>(pps + (size_t)n_slots * a.Hv * SLOT_STRIDE);
    sw.map_m = (long)a.B * sc.S * a.Hv * D * D;
    sw.starts = sw.maps + 2 * sw.map_m;
    launch_prep(a, tbs, pps, nullptr, nc, n_slots, s);
    sw.phase = 1;
    launch_spine(a, dim3(a.Hv * N_TILES, a.B * (2 * sc.S - 3)), a.h0, nullptr, tbs, pps, nullptr, nullptr, nc,
                 n_slots, sw, s);
    hipLaunchKernelGGL(gdn_segment_combine_kernel, dim3(a.Hv * N_TILES, a.B), dim3(64 * CMB_WAVES), 0, s, sw,
                       a.Hv);
    sw.phase = 2;
    launch_spine(a, dim3(a.Hv * N_TILES, a.B * sc.S), a.h0, a.h_final, tbs, pps, nullptr, nullptr, nc, n_slots,
                 sw, s);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s)
{
    const bool packed = a.cu_seqlens != nullptr;
    const SegmentCut sc = a.segmented ? segment_cut(a.B, a.T, a.Hv, packed) : SegmentCut{0, 0};
    if (sc.S > 0) return launch_prefill_segmented(a, sc, s);
    int32_t* base = reinterpret_cast<int32_t*>(a.workspace);
    const int nc_dense = (a.T + C - 1) / C;
    const long n_slots = slot_count(a.B, a.T, packed);
    unsigned char* tbs = reinterpret_cast<unsigned char*>(a.workspace) + table_bytes(a.B);   // T_e slots
    unsigned char* pps = tbs + (size_t)n_slots * a.Hv * SLOT_STRIDE;                       // PT slots
    const int32_t* order = packed && a.B <= MAX_ORDERED ? base + a.B + 1 : nullptr;
    if (packed) {
        hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.B, a.T, base);
    }
    if (n_slots > 0) launch_prep(a, tbs, pps, base, nc_dense, n_slots, s);
    launch_spine(a, dim3(a.Hv * N_TILES, a.B), a.h0, a.h_final, tbs, pps, base, order, nc_dense, n_slots,
                 SegWalk{}, s);
    return hipGetLastError();
}

}  // namespace gdn

// The gate/beta producer ahead of the recurrence (the BA projection), gfx950.
//
// For each token t the activation row x_t (k bf16 values) is multiplied by
// the n = 2 nv weight rows w_o (bf16), and output o is placed by the pages'
// index model (ssm_ba_gates_hopper.rs, "the index model", ba_gates_slot) into
// the token's fp32 output row [gate(nv) | beta(nv)]: with G v-heads per
// group, group = o / 2G, w = o % 2G; w < G is beta of v-head group G + w, else
// the gate of v-head group G + w - G.  The gating (not printed on the pages;
// read from the names of the launcher's a_log and dt_bias arguments):
//     gate = -exp(a_log) softplus(y + dt_bias),   beta = sigmoid(y).
//
// The product is m x k by k x n with n small (96 at the pages' geometry) and
// k large (5120): it is bound by reading x once from HBM.  Two kernels:
//
// gdn_ba_partial_kernel, grid (token tiles of 128, k splits), one loader wave
//   plus one compute wave per 32 outputs.  The loader streams the tile's x
//   through a three-stage LDS ring by buffer->LDS DMA, 64 k per stage (16 KiB,
//   rows beyond m read as zero); each compute wave reads the eight 16-token A
//   fragments of a k-step from LDS and the fragments of its own 32 weight
//   rows straight from memory (the weight is small and stays in L2; those
//   loads run five blocks ahead in registers to cover its latency), on
//   v_mfma_f32_16x16x32_bf16, and writes its fp32 partial sums.  The number
//   of k splits is chosen so that the grid fills the 256 compute units once
//   (36 token tiles x 7 splits at the pages' 4576 tokens): a second round of a
//   few workgroups would cost a whole workgroup's time.  Each workgroup reads
//   128 tokens' worth of x per weight fragment it fetches.
// gdn_ba_gate_kernel, one thread per (token, output): sums the splits' partial
//   sums, applies the gating and writes the output row.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int TM = 128;           // tokens per workgroup
constexpr int RT = TM / 16;       // 16-token MFMA tiles per workgroup
constexpr int KB = 64;            // k values per ring stage
constexpr int NSTAGE = 3;         // ring stages: deeper rings measured slower (each workgroup
                                  // asks for NSTAGE - 1 stages at once at its start)
constexpr int STAGE_BYTES = TM * KB * 2;   // 16 KiB
constexpr int PIECES = STAGE_BYTES / 1024; // 1 KiB DMAs per stage (8 token rows each)
constexpr int WAHEAD = 5;         // blocks the weight loads run ahead
constexpr int OTW = 2;            // 16-output tiles per compute wave
constexpr int CU_COUNT = 256;     // compute units the split count is sized for
constexpr int MAX_SPLITS = 32;

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Buffer resource for the DMA: wave-uniform base and byte range in SGPRs.  On
// gfx950 the range check covers the lane and the SGPR offsets, so reads past
// the range (rows beyond m) return zero.
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
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p);
}
// Eight 1 KiB buffer->LDS DMAs into consecutive LDS kilobytes from `lds`:
// piece j reads lane offset v0 (even j) or v1 (odd j) plus SGPR offset
// so[j].  Written as inline assembly so that the compiler does not make every
// LDS read wait for the DMA; completion is tracked with vmcnt by the loader
// wave, the only wave that issues vector memory operations in the loop.
__device__ __forceinline__ void dma_x8(const Rsrc& r, uint32_t lds, uint32_t v0, uint32_t v1,
                                       const uint32_t* so) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %2, %1, %4 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %5 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %6 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %7 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %8 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %9 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %10 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %3, %1, %11 offen lds"
                 :: "s"(lds), "s"(r.d), "v"(v0), "v"(v1), "s"(so[0]), "s"(so[1]), "s"(so[2]),
                    "s"(so[3]), "s"(so[4]), "s"(so[5]), "s"(so[6]), "s"(so[7])
                 : "memory", "m0", "scc");
}
// s_waitcnt vmcnt(N) for the ring depths used here (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left free).
#define GDN_BA_VMCNT(N) (((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Stage layout: token row r (0..127) holds 64 k values as 8 granules of 16
// bytes; granule q of row r sits at position q ^ (r % 8), so that the eight
// lanes a 16-byte fragment read serves per pass (eight rows, one granule) hit
// distinct banks.
__device__ __forceinline__ uint32_t stage_off(int r, int q) { return (uint32_t)(r * 128 + 16 * (q ^ (r & 7))); }

__global__ void __launch_bounds__(320)
gdn_ba_partial_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                      float* __restrict__ partial, int m, int n, int k, int x_stride,
                      int blocks_per_split)
{
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NSTAGE * STAGE_BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_cw = (int)(blockDim.x >> 6) - 1;     // compute waves
    const int t0 = blockIdx.x * TM;
    const int split = blockIdx.y;
    const int nb_total = k / KB;
    const int b0 = split * blocks_per_split;
    const int nb = max(0, min(nb_total, b0 + blocks_per_split) - b0);

    if (wave == n_cw) {   // the loader wave
        const uint32_t row_bytes = (uint32_t)x_stride * 2u;
        const Rsrc rx = make_dma_rsrc(x + (size_t)t0 * x_stride, (uint32_t)(m - t0) * row_bytes);
        // lane l of piece j writes LDS row 8 j + l / 8, position l % 8; it reads
        // that row's granule (l % 8) ^ (row % 8) = (l % 8) ^ (l / 8)
        const int r8 = lane >> 3, p = lane & 7;
        const uint32_t voff = (uint32_t)r8 * row_bytes + 16u * (uint32_t)(p ^ r8);
        auto issue = [&](int b) {   // block b of this split into its stage
            uint32_t so[PIECES];
#pragma unroll
            for (int j = 0; j < PIECES; ++j)
                so[j] = __builtin_amdgcn_readfirstlane((uint32_t)(b0 + b) * KB * 2u + (uint32_t)(8 * j) * row_bytes);
            const uint32_t base = lds_addr(ring + (b % NSTAGE) * STAGE_BYTES);
            dma_x8(rx, base, voff, voff, so);
            dma_x8(rx, base + 8192u, voff, voff, so + 8);
        };
        for (int b = 0; b < NSTAGE - 1 && b < nb; ++b) issue(b);
        // block 0 has landed once at most NSTAGE - 2 blocks are outstanding
        if (nb >= NSTAGE - 1) __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(PIECES * (NSTAGE - 2)));
        else __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(0));
        for (int b = 0; b < nb; ++b) {
            ring_barrier();   // block b is ready; the stage of block b - 1 is free
            if (b + NSTAGE - 1 < nb) {
                issue(b + NSTAGE - 1);
                __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(PIECES * (NSTAGE - 2)));   // block b + 1 landed
            } else {
                __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(0));
            }
        }
        return;
    }

    // compute wave: output tiles OTW wave .. OTW wave + OTW - 1 of tokens t0 .. t0 + TM - 1
    const int g = lane >> 4, i = lane & 15;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(w), (short)0, n * k * 2, 0x00020000);
    int o_row[OTW];          // this lane's weight row (B operand column) of each tile
    uint32_t w_lane[OTW];
#pragma unroll
    for (int j = 0; j < OTW; ++j) {
        o_row[j] = 16 * (OTW * wave + j) + i;
        w_lane[j] = (uint32_t)o_row[j] * (uint32_t)k * 2u + 16u * (uint32_t)g;   // rows >= n: out of range, 0
    }
    constexpr int KS = KB / 32;   // k-steps per block
    auto load_w = [&](int b, int s, int j) {   // B fragment: tile j, k-step s of block b
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            rw, w_lane[j], (uint32_t)((b0 + b) * KB + 32 * s) * 2u, 0);
        return __builtin_bit_cast(s16x8, v);
    };
    f32x4 acc[RT][OTW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < OTW; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the weight fragments run WAHEAD blocks ahead of the MFMAs, in a ring of
    // registers indexed by the block number mod WAHEAD (the loop is unrolled
    // by WAHEAD so that every index is static)
    s16x8 wb[WAHEAD][KS][OTW];
#pragma unroll
    for (int d = 0; d < WAHEAD; ++d)
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int j = 0; j < OTW; ++j) wb[d][s][j] = d < nb ? load_w(d, s, j) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    for (int bu = 0; bu < nb; bu += WAHEAD) {
#pragma unroll
        for (int u = 0; u < WAHEAD; ++u) {
            const int b = bu + u;
            if (b < nb) {   // uniform: every wave meets the same barriers
                ring_barrier();
                const unsigned char* st = ring + (b % NSTAGE) * STAGE_BYTES;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    s16x8 af[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        af[rt] = *reinterpret_cast<const s16x8*>(st + stage_off(16 * rt + i, 4 * s + g));
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int j = 0; j < OTW; ++j) acc[rt][j] = mfma_bf16(wb[u][s][j], af[rt], acc[rt][j]);
                }
                if (b + WAHEAD < nb) {
#pragma unroll
                    for (int s = 0; s < KS; ++s)
#pragma unroll
                        for (int j = 0; j < OTW; ++j) wb[u][s][j] = load_w(b + WAHEAD, s, j);
                }
            }
        }
    }
    // partial[split][t][o].  The products are formed transposed (the weight
    // fragment as the A operand, the activations as B), so lane (g, i) of
    // tile (rt, j) holds outputs 16 (OTW wave + j) + 4 g .. + 3 of token
    // 16 rt + i: one 16-byte store each, a token's 16 outputs of the tile in
    // four neighbouring lanes.
    float* dst = partial + (size_t)split * m * n;
    // rows of whole, aligned 16-byte granules
    const bool vec = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(partial) & 15) == 0;
#pragma unroll
    for (int j = 0; j < OTW; ++j) {
        const int o4 = 16 * (OTW * wave + j) + 4 * g;
        if (o4 >= n) continue;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int t = t0 + 16 * rt + i;
            if (t >= m) continue;
            float* p = dst + (size_t)t * n + o4;
            const f32x4 v = acc[rt][j];
            if (vec) {
                *reinterpret_cast<f32x4*>(p) = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (o4 + r < n) p[r] = v[r];
            }
        }
    }
}

// The gating on the hardware's exp2, log2 and reciprocal (the IEEE division
// and the library log1p take about 150 instructions a value, and a wave whose
// lanes mix gates and betas runs both).  softplus(z) = max(z, 0) +
// log1p(exp(-|z|)), with log1p(e) = log(1 + e) e / ((1 + e) - 1) (e itself
// where 1 + e rounds to 1), which keeps its relative accuracy for small e.
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
__device__ __forceinline__ float sigmoid(float y) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-y * LOG2E));
}
__device__ __forceinline__ float softplus(float z) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(z) * LOG2E);
    const float u = 1.f + e;
    const float l1p = u == 1.f ? e : __builtin_amdgcn_logf(u) * LN2 * (e * __builtin_amdgcn_rcpf(u - 1.f));
    return fmaxf(z, 0.f) + l1p;
}

__global__ void __launch_bounds__(256)
gdn_ba_gate_kernel(const float* __restrict__ partial, const float* __restrict__ a_log,
                   const float* __restrict__ dt_bias, float* __restrict__ out, int m, int n,
                   int splits, int gate_stride, int nv, int G)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)m * n) return;
    const int t = (int)(idx / n), o = (int)(idx % n);
    // up to eight splits' loads in flight before the first add (a plain loop
    // over a run-time count waits out each load in turn); the sum still runs
    // over s = 0, 1, ... in order
    float y = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 8) {
        float p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            p[u] = s0 + u < splits ? partial[(size_t)(s0 + u) * m * n + idx] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < splits) y += p[u];
    }
    const int group = o / (2 * G), within = o % (2 * G);
    float* row = out + (size_t)t * gate_stride;
    if (within < G) {
        row[nv + group * G + within] = sigmoid(y);
    } else {
        const int vh = group * G + (within - G);
        row[vh] = -__expf(a_log[vh]) * softplus(y + dt_bias[vh]);
    }
}

// k splits of a call: as many as fill the compute units once with the token
// tiles, at most one per 64-wide k block, then evened out so that no split is
// empty.  A pure function of (m, k): the workspace size and the launch agree.
int splits_for(int m, int k) {
    const int tiles = (m + TM - 1) / TM;
    const int nb = k / KB;
    int s = tiles > 0 ? CU_COUNT / tiles : 1;
    s = s < 1 ? 1 : s > MAX_SPLITS ? MAX_SPLITS : s;
    s = s > nb ? nb : s;
    if (s < 1) return 1;
    const int bps = (nb + s - 1) / s;
    return (nb + bps - 1) / bps;
}

int compute_waves(int n) { return ((n + 15) / 16 + OTW - 1) / OTW; }

}  // namespace

size_t ba_gates_workspace_bytes(int m, int n, int k)
{
    return (size_t)splits_for(m, k) * m * n * sizeof(float);
}

Geometry ba_gates_geometry(const BaArgs& a)
{
    Geometry g{"gdn_ba_partial_kernel+gdn_ba_gate_kernel",
               {(unsigned)((a.m + TM - 1) / TM), (unsigned)splits_for(a.m, a.k), 1u},
               (unsigned)(64 * (compute_waves(a.n) + 1)), (unsigned)(NSTAGE * STAGE_BYTES)};
    return g;
}

hipError_t launch_ba_gates(const BaArgs& a, hipStream_t s)
{
    if (a.m == 0) return hipSuccess;
    const int S = splits_for(a.m, a.k);
    const int nb_total = a.k / KB;
    const int bps = (nb_total + S - 1) / S;
    float* partial = reinterpret_cast<float*>(a.workspace);
    hipLaunchKernelGGL(gdn_ba_partial_kernel, dim3((unsigned)((a.m + TM - 1) / TM), (unsigned)S),
                       dim3((unsigned)(64 * (compute_waves(a.n) + 1))), 0, s, (const uint16_t*)a.input,
                       (const uint16_t*)a.ba_weight, partial, a.m, a.n, a.k, a.k_stride, bps);
    const long total = (long)a.m * a.n;
    hipLaunchKernelGGL(gdn_ba_gate_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       partial, a.a_log, a.dt_bias, a.gate_out, a.m, a.n, S, a.gate_stride, a.nv,
                       a.vheads_per_group);
    return hipGetLastError();
}

}  // namespace gdn

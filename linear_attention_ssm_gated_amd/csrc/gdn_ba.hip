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
// gdn_ba_partial_kernel, grid (token tiles of 64, K splits), one loader wave
//   plus one compute wave per 16 outputs.  The loader streams the tile's x
//   through an eight-stage LDS ring by buffer->LDS DMA, 64 k per stage (8 KiB,
//   rows beyond m read as zero); each compute wave reads the four 16-token A
//   fragments of a k-step from LDS and its own 16 weight rows straight from
//   memory (the weight is small and stays in L2), on v_mfma_f32_16x16x32_bf16,
//   and writes its fp32 partial sums.  Splitting k over workgroups keeps each
//   compute unit's weight traffic to a quarter of the weight and puts ~290
//   workgroups on the chip.
// gdn_ba_gate_kernel, one thread per (token, output): sums the splits' partial
//   sums, applies the gating and writes the output row.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int TM = 64;            // tokens per workgroup
constexpr int KB = 64;            // k values per ring stage
constexpr int NSTAGE = 8;         // ring stages
constexpr int STAGE_BYTES = TM * KB * 2;   // 8 KiB
constexpr int MAX_SPLITS = 4;

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
// piece j reads lane offset `voff` plus SGPR offset so[j].  Written as inline
// assembly so that the compiler does not make every LDS read wait for the
// DMA; completion is tracked with vmcnt by the loader wave, the only wave
// that issues vector memory operations in the loop.
__device__ __forceinline__ void dma_x8(const Rsrc& r, uint32_t lds, uint32_t voff, const uint32_t (&so)[8]) {
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "buffer_load_dwordx4 %2, %1, %3 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %4 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %5 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %6 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %7 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %8 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %9 offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"
                 "buffer_load_dwordx4 %2, %1, %10 offen lds"
                 :: "s"(lds), "s"(r.d), "v"(voff), "s"(so[0]), "s"(so[1]), "s"(so[2]), "s"(so[3]),
                    "s"(so[4]), "s"(so[5]), "s"(so[6]), "s"(so[7])
                 : "memory", "m0", "scc");
}
// s_waitcnt vmcnt(N) for the ring depths used here (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left free).
#define GDN_BA_VMCNT(N) (((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Stage layout: token row r (0..63) holds 64 k values as 8 granules of 16
// bytes; granule q of row r sits at position q ^ (r % 8), so that the eight
// lanes a 16-byte fragment read serves per pass (eight rows, one granule)
// hit distinct banks.
__device__ __forceinline__ uint32_t stage_off(int r, int q) { return (uint32_t)(r * 128 + 16 * (q ^ (r & 7))); }

__global__ void __launch_bounds__(576)
gdn_ba_partial_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                      float* __restrict__ partial, int m, int n, int k, int x_stride,
                      int blocks_per_split)
{
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NSTAGE * STAGE_BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_tiles = (int)(blockDim.x >> 6) - 1;     // compute waves
    const int t0 = blockIdx.x * TM;
    const int split = blockIdx.y;
    const int nb_total = k / KB;
    const int b0 = split * blocks_per_split;
    const int nb = max(0, min(nb_total, b0 + blocks_per_split) - b0);

    if (wave == n_tiles) {   // the loader wave
        const uint32_t row_bytes = (uint32_t)x_stride * 2u;
        const Rsrc rx = make_dma_rsrc(x + (size_t)t0 * x_stride, (uint32_t)(m - t0) * row_bytes);
        // lane l of piece j writes LDS row 8 j + l / 8, position l % 8; it reads
        // that row's granule (l % 8) ^ (row % 8) = (l % 8) ^ (l / 8)
        const int r8 = lane >> 3, p = lane & 7;
        const uint32_t voff = (uint32_t)r8 * row_bytes + 16u * (uint32_t)(p ^ r8);
        auto issue = [&](int b) {   // block b of this split into its stage
            uint32_t so[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                so[j] = __builtin_amdgcn_readfirstlane((uint32_t)(b0 + b) * KB * 2u + (uint32_t)(8 * j) * row_bytes);
            dma_x8(rx, lds_addr(ring + (b % NSTAGE) * STAGE_BYTES), voff, so);
        };
        for (int b = 0; b < NSTAGE - 1 && b < nb; ++b) issue(b);
        // block 0 has landed once at most NSTAGE - 2 blocks are outstanding
        if (nb >= NSTAGE - 1) __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(8 * (NSTAGE - 2)));
        else __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(0));
        for (int b = 0; b < nb; ++b) {
            ring_barrier();   // block b is ready; the stage of block b - 1 is free
            if (b + NSTAGE - 1 < nb) {
                issue(b + NSTAGE - 1);
                __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(8 * (NSTAGE - 2)));   // block b + 1 landed
            } else {
                __builtin_amdgcn_s_waitcnt(GDN_BA_VMCNT(0));
            }
        }
        return;
    }

    // compute wave: outputs 16 wave .. 16 wave + 15 of tokens t0 .. t0 + 63
    const int g = lane >> 4, i = lane & 15;
    const int o_row = 16 * wave + i;   // this lane's weight row (B operand column)
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(w), (short)0, n * k * 2, 0x00020000);
    const uint32_t w_lane = (uint32_t)o_row * (uint32_t)k * 2u + 16u * (uint32_t)g;
    auto load_w = [&](int b, int s) {   // B fragment: rows o, k-step s of block b
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            rw, w_lane, (uint32_t)((b0 + b) * KB + 32 * s) * 2u, 0);
        return __builtin_bit_cast(s16x8, v);
    };
    f32x4 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the weight fragments run two blocks ahead of the MFMAs
    s16x8 wb[3][2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int s = 0; s < 2; ++s) wb[d][s] = d < nb ? load_w(d, s) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    for (int b = 0; b < nb; ++b) {
        ring_barrier();
        const unsigned char* st = ring + (b % NSTAGE) * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < 2; ++s) wb[2][s] = b + 2 < nb ? load_w(b + 2, s) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        s16x8 af[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                af[s][rt] = *reinterpret_cast<const s16x8*>(st + stage_off(16 * rt + i, 4 * s + g));
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma_bf16(af[s][rt], wb[0][s], acc[rt]);
#pragma unroll
        for (int s = 0; s < 2; ++s) { wb[0][s] = wb[1][s]; wb[1][s] = wb[2][s]; }
    }
    // partial[split][t][o]: lane (g, i) of tile rt holds tokens 16 rt + 4 g + r
    // of output column o_row
    if (o_row < n) {
        float* dst = partial + (size_t)split * m * n;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 16 * rt + 4 * g + r;
                if (t < m) dst[(size_t)t * n + o_row] = acc[rt][r];
            }
    }
}

__global__ void __launch_bounds__(256)
gdn_ba_gate_kernel(const float* __restrict__ partial, const float* __restrict__ a_log,
                   const float* __restrict__ dt_bias, float* __restrict__ out, int m, int n,
                   int splits, int gate_stride, int nv, int G)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)m * n) return;
    const int t = (int)(idx / n), o = (int)(idx % n);
    float y = 0.f;
    for (int s = 0; s < splits; ++s) y += partial[(size_t)s * m * n + idx];
    const int group = o / (2 * G), within = o % (2 * G);
    float* row = out + (size_t)t * gate_stride;
    if (within < G) {
        row[nv + group * G + within] = 1.f / (1.f + __expf(-y));
    } else {
        const int vh = group * G + (within - G);
        const float z = y + dt_bias[vh];
        const float sp = fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
        row[vh] = -__expf(a_log[vh]) * sp;
    }
}

int splits_for(int k) {
    const int nb = k / KB;
    return nb < MAX_SPLITS ? (nb > 0 ? nb : 1) : MAX_SPLITS;
}

}  // namespace

size_t ba_gates_workspace_bytes(int m, int n, int k)
{
    return (size_t)splits_for(k) * m * n * sizeof(float);
}

Geometry ba_gates_geometry(const BaArgs& a)
{
    const int tiles = (a.n + 15) / 16;
    Geometry g{"gdn_ba_partial_kernel+gdn_ba_gate_kernel",
               {(unsigned)((a.m + TM - 1) / TM), (unsigned)splits_for(a.k), 1u}, (unsigned)(64 * (tiles + 1)),
               (unsigned)(NSTAGE * STAGE_BYTES)};
    return g;
}

hipError_t launch_ba_gates(const BaArgs& a, hipStream_t s)
{
    if (a.m == 0) return hipSuccess;
    const int S = splits_for(a.k);
    const int nb_total = a.k / KB;
    const int bps = (nb_total + S - 1) / S;
    const int tiles = (a.n + 15) / 16;
    float* partial = reinterpret_cast<float*>(a.workspace);
    hipLaunchKernelGGL(gdn_ba_partial_kernel, dim3((unsigned)((a.m + TM - 1) / TM), (unsigned)S),
                       dim3((unsigned)(64 * (tiles + 1))), 0, s, (const uint16_t*)a.input,
                       (const uint16_t*)a.ba_weight, partial, a.m, a.n, a.k, a.k_stride, bps);
    const long total = (long)a.m * a.n;
    hipLaunchKernelGGL(gdn_ba_gate_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       partial, a.a_log, a.dt_bias, a.gate_out, a.m, a.n, S, a.gate_stride, a.nv,
                       a.vheads_per_group);
    return hipGetLastError();
}

}  // namespace gdn

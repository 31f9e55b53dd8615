// Full decoder-layer decode step for gfx950: RMSNorm, QKV projection, RoPE
// and KV append, paged GQA attention, o_proj with residual, RMSNorm, SwiGLU
// MLP with residual (course project section 2.1: the components of a
// Qwen-style decoder layer assembled with residual connections and two
// norms; pre-norm order).
//
// The projections are skinny (M = batch <= 32 rows) and stream their
// weights once on bf16 MFMA 16x16x32 tiles. One workgroup owns a few 16-column
// output tiles over the whole K range: its waves split K, stream their share
// of the weight rows, and the workgroup sums the per-wave accumulators through
// LDS in a fixed order (deterministic). Because a workgroup ends with finished
// output columns, each projection applies its own epilogue and no partial
// sums leave the chip:
//   QKV     -- 1 / rms(x) (from the activation stream itself), RoPE, K/V
//              append into the paged cache, q_rot;
//   o_proj  -- x2 = x + o W_o^T (fp32);
//   gate|up -- 1 / rms(x2) (from its activation stream), silu(g) * u;
//   down    -- out = bf16(x2 + a W_d^T).
// RMSNorm is x / rms(x) * w with a per-row scalar 1 / rms(x), so the GEMM runs
// on x * w and the epilogue multiplies by 1 / rms(x). The activations x * w,
// o, x2 * w2 and silu(g) * u enter the MFMAs as bf16 hi + lo pairs (about 16
// significant bits); inside the layer the rotated query also reaches the
// attention's score MFMAs as a bf16 pair (q_rot and its remainder q_lo) and
// the attention output o is kept in float32.
//
// Launch sequence: proj(qkv) -> attention (2 kernels) -> proj(o) ->
// proj(gate|up) -> proj(down).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "e4m3.h"
#include "internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BS = 16;
constexpr int kKStep = 32;               // K per MFMA

// Projection grids: waves per projection (upper bound), LDS bytes per
// workgroup (upper bound).
constexpr int kProjTargetWaves = 3072;
constexpr int kProjLdsCap = 65536;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
// float64 -> bf16 with one nearest-even rounding: float32 rounded to odd (the
// nearest-even float32, stepped one unit toward zero when it lies farther
// from zero than x, with the last bit set when inexact), then to bf16.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    if (x != x) return 0x7fc0;
    const float f = static_cast<float>(x);
    const double back = static_cast<double>(f);
    uint32_t u = __float_as_uint(f);
    if (back != x) {
        if (fabs(back) > fabs(x)) u -= 1u;
        u |= 1u;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------- skinny GEMM
// Y[m][n] = sum over k of A[m][k] * W[n][k], m < M. MFMA operand layout
// (16x16x32 bf16): lane l holds A[l % 16][8 (l / 16) .. +8) and
// B[8 (l / 16) .. +8)[l % 16]; the fp32 result D[4 (l / 16) + i][l % 16],
// i < 4. A is the activation rows (M padded to 16 per row tile), B the
// weight rows (W^T). Lanes of padding rows (m >= M) take an out-of-range
// offset, so their loads return zeros without touching memory; their output
// rows are discarded.
//
// Activation modes: kActBf16 -- A is bf16; kActGainSplit -- A is bf16 x[m][k]
// times a bf16 gain[k], formed in fp32; kActF32Split -- A is fp32;
// kActF32GainSplit -- A is fp32 x[m][k] times a bf16 gain[k]. In the split
// modes the fp32 value a is fed as a_hi = bf16(a) plus a_lo = bf16(a - a_hi),
// two MFMAs per step, so the activation keeps ~16 significant bits instead
// of 8 (the weight stream is unchanged). The gain modes also accumulate the
// sum of x^2 over the lane's K elements (the RMSNorm statistic of x).
constexpr int kActBf16 = 0;
constexpr int kActGainSplit = 1;
constexpr int kActF32Split = 2;
constexpr int kActF32GainSplit = 3;

// Epilogues of the fused projection kernel.
constexpr int kEpiQkv = 0;        // RMSNorm scale, RoPE, K/V append, q_rot
constexpr int kEpiResidual = 1;   // x2 = x + y (fp32)
constexpr int kEpiSwiglu = 2;     // a = silu(r g) * (r u), r = 1 / rms(x2) (fp32)
constexpr int kEpiOut = 3;        // out = bf16(x2 + y)

// hi = bf16(v), lo = bf16(v - hi), both round-to-nearest-even, through the
// packed hardware conversion (one instruction per pair of values).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2_t hp = {static_cast<__bf16>(v[2 * e]), static_cast<__bf16>(v[2 * e + 1])};
        h[e] = __builtin_bit_cast(uint32_t, hp);
        const float r0 = v[2 * e] - __uint_as_float(h[e] << 16);
        const float r1 = v[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u);
        const bf16x2_t lp = {static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
        l[e] = __builtin_bit_cast(uint32_t, lp);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Buffer-resource loads: the per-lane byte offset (VGPR) stays fixed for the
// whole K loop and only the scalar offset moves, so the loop carries no VGPR
// address arithmetic (which would otherwise reuse registers of loads still in
// flight and force full waits). Out-of-range offsets read zeros.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;     // raw 32-bit buffer access (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;  // lane offset beyond any buffer here: reads 0
constexpr int kAuxStream = 2;                 // non-temporal: weights are read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), kBufferDword3);
}
template <int AUX>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Loads and MFMAs of one batch of KB K-steps for NW column tiles and MT row
// tiles. load() only issues memory reads (activations, gain, then weights);
// the activation's conversion to bf16 (hi, lo) happens in mma(), so
// prefetching the next batch never waits on its own loads.
//
// Each column tile has its own buffer resource based at its first weight
// row, so a workgroup's tiles need not be adjacent (RoPE pairs, gate with
// up). The weights are loaded transposed: 4 KB lanes share a row, so one
// instruction reads 64 / (4 KB) whole row segments of 64 KB bytes (full
// 128-byte lines at KB = 2); mma() writes the batch to the wave's LDS tile and
// reads it back in the MFMA layout (rows padded by 16 bytes).
template <int MT, int NW, int ACT, int KB, bool HALF = false>
struct GemmBatch {
    static constexpr bool GAIN = ACT == kActGainSplit || ACT == kActF32GainSplit;
    static constexpr bool F32 = ACT == kActF32Split || ACT == kActF32GainSplit;
    // HALF (fp32 modes, at most 8 rows): one load per K step fills all 64
    // lanes -- lane 16 q + c loads elements 4 (c / 8) .. + 4 of the lane's
    // 8-element segment of row c % 8 -- and the two halves of a segment are
    // joined by a lane rotation by 8 within each row of 16 lanes. Lanes c >= 8
    // then feed copies of rows 0..7 as MFMA rows 8..15, whose outputs are
    // never read.
    static constexpr bool F32H = F32 && HALF;
    static_assert(!HALF || (F32 && MT == 1), "HALF: fp32 activations, one row tile");
    static constexpr int AE = F32 ? 4 : 2;                     // activation element bytes
    static constexpr int LPR = 4 * KB;                         // lanes per row
    static constexpr int RPI = 64 / LPR;                       // rows per load
    static constexpr int ROWB = 64 * KB + 16;                  // LDS bytes per row (padded)
    static constexpr int LDS_BYTES = 16 * NW * ROWB;           // per wave
    uint4 w[KB * NW];                      // load i: tile i / KB, rows (i % KB) RPI ..
    uint4 a0[KB][MT];                      // bf16 activations, or fp32 elements 0..3
    uint4 a1[F32 && !HALF ? KB : 1][F32 && !HALF ? MT : 1];  // fp32 elements 4..7
    uint4 gn[GAIN ? KB : 1];               // gain

    // kbyte: byte offset of the batch's first K column in a bf16 row. woff:
    // the lane's row segment in load 0 of a tile; rowstep: bytes between the
    // row groups of consecutive loads of a tile (RPI rows).
    __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t (&rw)[NW], uint32_t woff,
                                         uint32_t rowstep, __amdgpu_buffer_rsrc_t ra,
                                         const uint32_t (&aoff)[MT], __amdgpu_buffer_rsrc_t rg,
                                         uint32_t goff, uint32_t kbyte) {
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t ak = (kbyte + u * kKStep * 2) / 2 * AE;
                a0[u][mt] = bload<0>(ra, aoff[mt], ak);
                if constexpr (F32 && !HALF) a1[u][mt] = bload<0>(ra, aoff[mt] + 16, ak);
            }
        if constexpr (GAIN) {
#pragma unroll
            for (int u = 0; u < KB; ++u) gn[u] = bload<0>(rg, goff, kbyte + u * kKStep * 2);
        }
#pragma unroll
        for (int i = 0; i < KB * NW; ++i) w[i] = bload<kAuxStream>(rw[i / KB], woff, kbyte + (i % KB) * rowstep);
    }

    // lds: the wave's tile; wr = lane's write offset of load 0 (bytes),
    // rd = lane's read offset for step 0 of tile 0. ssq[mt] accumulates x^2
    // of the lane's activation elements (gain modes).
    __device__ __forceinline__ void mma(f32x4_t (&acc)[NW][MT], float (&ssq)[MT], char* lds, uint32_t wr,
                                        uint32_t rd) const {
#pragma unroll
        for (int i = 0; i < KB * NW; ++i) *reinterpret_cast<uint4*>(lds + wr + i * RPI * ROWB) = w[i];
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint4 hi = a0[u][mt], lo = make_uint4(0, 0, 0, 0);
                if constexpr (ACT != kActBf16) {
                    float x[8];
                    if constexpr (F32H) {
                        // own 4 elements, then the partner lane's (c xor 8) 4
                        const uint4 p0 = a0[u][mt];
                        constexpr int kRowRor8 = 0x128;      // DPP: rotate right by 8 within 16 lanes
                        const uint32_t q0 = __builtin_amdgcn_mov_dpp(static_cast<int>(p0.x), kRowRor8, 0xf, 0xf, false);
                        const uint32_t q1 = __builtin_amdgcn_mov_dpp(static_cast<int>(p0.y), kRowRor8, 0xf, 0xf, false);
                        const uint32_t q2 = __builtin_amdgcn_mov_dpp(static_cast<int>(p0.z), kRowRor8, 0xf, 0xf, false);
                        const uint32_t q3 = __builtin_amdgcn_mov_dpp(static_cast<int>(p0.w), kRowRor8, 0xf, 0xf, false);
                        x[0] = __uint_as_float(p0.x); x[1] = __uint_as_float(p0.y);
                        x[2] = __uint_as_float(p0.z); x[3] = __uint_as_float(p0.w);
                        x[4] = __uint_as_float(q0); x[5] = __uint_as_float(q1);
                        x[6] = __uint_as_float(q2); x[7] = __uint_as_float(q3);
                    } else if constexpr (F32) {
                        const uint4 p0 = a0[u][mt], p1 = a1[u][mt];
                        x[0] = __uint_as_float(p0.x); x[1] = __uint_as_float(p0.y);
                        x[2] = __uint_as_float(p0.z); x[3] = __uint_as_float(p0.w);
                        x[4] = __uint_as_float(p1.x); x[5] = __uint_as_float(p1.y);
                        x[6] = __uint_as_float(p1.z); x[7] = __uint_as_float(p1.w);
                    } else {
                        const uint32_t aw[4] = {a0[u][mt].x, a0[u][mt].y, a0[u][mt].z, a0[u][mt].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[2 * e] = bf16_to_f32(static_cast<uint16_t>(aw[e]));
                            x[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(aw[e] >> 16));
                        }
                    }
                    float v[8];
                    if constexpr (GAIN) {
                        const uint32_t gw[4] = {gn[u].x, gn[u].y, gn[u].z, gn[u].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[2 * e] = x[2 * e] * bf16_to_f32(static_cast<uint16_t>(gw[e]));
                            v[2 * e + 1] = x[2 * e + 1] * bf16_to_f32(static_cast<uint16_t>(gw[e] >> 16));
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) ssq[mt] = fmaf(x[e], x[e], ssq[mt]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = x[e];
                    }
                    split8(v, hi, lo);
                }
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    const uint4 wv = *reinterpret_cast<const uint4*>(lds + rd + j * 16 * ROWB + u * 64);
                    acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, hi), __builtin_bit_cast(bf16x8_t, wv), acc[j][mt], 0, 0, 0);
                    if constexpr (ACT != kActBf16)
                        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, lo), __builtin_bit_cast(bf16x8_t, wv), acc[j][mt],
                            0, 0, 0);
                }
            }
    }
};

// ------------------------------------------------- fused projection kernel

struct ProjArgs {
    const void* A;              // activation rows [M][K]: bf16 or fp32 by mode
    const uint16_t* gain;       // [K] RMSNorm weight (gain modes)
    const uint16_t* W0;         // weight rows [*][K] bf16
    const uint16_t* W1;         // up rows (SwiGLU), else unused
    int M, K, N;                // N: row width of the outputs (hidden or intermediate)
    float eps;
    // QKV epilogue
    int hq, hkv, D;
    uint16_t* q_rot;            // bf16 of the rotated query
    uint16_t* q_lo;             // bf16 of its remainder (q_rot + q_lo: ~16 significant bits)
    void* kc;
    void* vc;
    const int32_t* table;
    int mbps;
    const int32_t* ctx;
    int num_blocks;
    const float* kv_scales;
    uint32_t* err;
    int fp8;
    // residual epilogues
    const uint16_t* x_in;       // kEpiResidual: bf16 [M][N]
    const float* x2;            // kEpiOut: fp32 [M][N]
    float* y_f32;               // kEpiResidual: x2; kEpiSwiglu: a
    uint16_t* y_bf16;           // kEpiOut
};

// Waves per workgroup at most: 16 when a wave fits in 128 VGPRs (estimate:
// two batches of weight, activation and gain registers, the accumulators and
// about 30 for addresses and temporaries; the QKV epilogue's float64 RoPE
// needs more), else 8.
constexpr int kProjQkvWaves = 8;
constexpr int kProjVgprExtra = 30;
template <int MT, int NW, int KB, int ACT, int EPI, bool HALF>
constexpr int proj_max_waves() {
    using B = GemmBatch<MT, NW, ACT, KB, HALF>;
    constexpr int batch = 4 * (KB * NW + KB * MT * (B::F32 && !HALF ? 2 : 1) + (B::GAIN ? KB : 0));
    if (EPI == kEpiQkv) return kProjQkvWaves;
    return 2 * batch + 4 * NW * MT + kProjVgprExtra <= 128 ? 16 : 8;
}

// LDS bytes per wave: the weight staging tile during the K loop, the
// accumulators and RMSNorm sums after it.
template <int MT, int NW, int KB, int ACT>
constexpr size_t proj_lds_per_wave() {
    return std::max<size_t>(GemmBatch<MT, NW, ACT, KB>::LDS_BYTES, (NW * MT * 256 + MT * 16) * sizeof(float));
}

// One workgroup of KS = blockDim / 64 waves per group of NW column tiles.
// Tiles: QKV -- NP = NW / 2 RoPE pairs (tile j, tile j + D / 32) of one head,
// so the rotation partners d and d + D / 2 land in one workgroup; SwiGLU --
// gate tiles g NP .. + NP and the same up tiles; otherwise NW adjacent tiles. Wave w streams the K
// range [w K / KS, (w + 1) K / KS) through a two-slot register ring (the next
// batch in flight while the current one is multiplied), then the waves'
// accumulators (and RMSNorm sums) are summed through LDS in wave order and
// the epilogue runs on the finished outputs.
template <int MT, int NW, int KB, int ACT, int EPI, bool HALF>
__global__ __launch_bounds__((64 * proj_max_waves<MT, NW, KB, ACT, EPI, HALF>())) void proj_kernel(
    ProjArgs a, mikv::RopeTable rope) {
    using Batch = GemmBatch<MT, NW, ACT, KB, HALF>;
    constexpr int NP = NW / 2;                 // tile pairs (QKV, SwiGLU)
    static_assert((EPI != kEpiQkv && EPI != kEpiSwiglu) || (NW % 2 == 0), "paired tiles");
    extern __shared__ __align__(16) char lds[];
    const int KS = blockDim.x >> 6;
    // wave index as a scalar: the K offsets of the buffer loads must be
    // uniform (a per-lane value there turns every load into a loop)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int g = blockIdx.x;
    const int K = a.K;
    const int M = a.M;

    int tile[NW];
    const uint16_t* wsrc[NW];
    int head = 0, j0 = 0;
    if constexpr (EPI == kEpiQkv) {
        const int hp = a.D / 32;                // pairs per head
        const int gph = hp / NP;                // workgroups per head
        head = g / gph;
        j0 = (g - head * gph) * NP;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            tile[p] = head * (a.D / 16) + j0 + p;
            tile[NP + p] = tile[p] + hp;
            wsrc[p] = wsrc[NP + p] = a.W0;
        }
    } else if constexpr (EPI == kEpiSwiglu) {
        j0 = g * NP;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            tile[p] = tile[NP + p] = j0 + p;
            wsrc[p] = a.W0;
            wsrc[NP + p] = a.W1;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            tile[j] = g * NW + j;
            wsrc[j] = a.W0;
        }
    }
    __amdgpu_buffer_rsrc_t rw[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j)
        rw[j] = make_rsrc(wsrc[j] + static_cast<size_t>(tile[j]) * 16 * K, static_cast<uint32_t>(16 * K * 2));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, static_cast<uint32_t>(static_cast<size_t>(M) * K * Batch::AE));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain, a.gain ? static_cast<uint32_t>(K) * 2 : 0u);
    const int r_in = lane / Batch::LPR, piece = lane % Batch::LPR;
    const uint32_t woff = static_cast<uint32_t>(r_in) * K * 2 + piece * 16;
    const uint32_t rowstep = static_cast<uint32_t>(Batch::RPI) * K * 2;
    const uint32_t wr = r_in * Batch::ROWB + piece * 16;
    const uint32_t rd = col * Batch::ROWB + kq * 16;
    char* stage = lds + wv * Batch::LDS_BYTES;
    uint32_t aoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if constexpr (Batch::F32H)
            aoff[mt] = (col & 7) < M ? (static_cast<uint32_t>(col & 7) * K + kq * 8 + 4 * (col >> 3)) * Batch::AE
                                     : kOutOfRange;
        else
            aoff[mt] = mt * 16 + col < M ? (static_cast<uint32_t>(mt * 16 + col) * K + kq * 8) * Batch::AE
                                         : kOutOfRange;
    }
    const uint32_t goff = kq * 8 * 2;

    f32x4_t acc[NW][MT];
    float ssq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        ssq[mt] = 0.f;
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // QKV: the thread's first epilogue item's position, block and rotation
    // (float64 sincos) are computed here, while the first weight batches are
    // in flight, rather than after the K loop.
    int pre_pos = -1;
    int32_t pre_blk = -1;
    double pre_sn = 0.0, pre_cs = 1.0;
    if constexpr (EPI == kEpiQkv) {
        const int it = threadIdx.x;
        if (it < M * NP * 16) {
            const int m = it / (NP * 16);
            const int d = (j0 + (it >> 4) % NP) * 16 + (it & 15);
            pre_pos = a.ctx[m];
            if (pre_pos >= 0 && pre_pos / BS < a.mbps) {
                pre_blk = a.table[static_cast<size_t>(m) * a.mbps + pre_pos / BS];
                if (head < a.hq + a.hkv) sincos(static_cast<double>(pre_pos) * rope.inv_freq[d], &pre_sn, &pre_cs);
            }
        }
    }

    // Residual epilogues: the thread's first output's residual input is
    // loaded here for the same reason.
    float pre_res = 0.f;
    if constexpr (EPI == kEpiResidual || EPI == kEpiOut) {
        const int it = threadIdx.x;
        if (it < M * NW * 16) {
            const size_t at = static_cast<size_t>(it / (NW * 16)) * a.N + tile[(it >> 4) % NW] * 16 + (it & 15);
            if constexpr (EPI == kEpiResidual) pre_res = bf16_to_f32(a.x_in[at]);
            else pre_res = a.x2[at];
        }
    }

    constexpr uint32_t STEP_BYTES = KB * kKStep * 2;
    const int k_chunk = K / KS;
    const int nb = k_chunk / (KB * kKStep);   // batches (>= 1)
    const uint32_t kb0 = static_cast<uint32_t>(wv) * k_chunk * 2;
    // The scheduling barriers keep each batch's loads ahead of the previous
    // batch's MFMAs: left free, the compiler sinks them below the LDS writes
    // and every batch then waits for all loads (one batch in flight).
    auto kb = [&](int t) { return kb0 + static_cast<uint32_t>(t) * STEP_BYTES; };
    Batch b0, b1;
    b0.load(rw, woff, rowstep, ra, aoff, rg, goff, kb(0));
    int i = 0;
    for (; i + 2 < nb; i += 2) {
        b1.load(rw, woff, rowstep, ra, aoff, rg, goff, kb(i + 1));
        __builtin_amdgcn_sched_barrier(0);
        b0.mma(acc, ssq, stage, wr, rd);
        __builtin_amdgcn_sched_barrier(0);
        b0.load(rw, woff, rowstep, ra, aoff, rg, goff, kb(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        b1.mma(acc, ssq, stage, wr, rd);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i + 1 < nb) {
        b1.load(rw, woff, rowstep, ra, aoff, rg, goff, kb(i + 1));
        __builtin_amdgcn_sched_barrier(0);
        b0.mma(acc, ssq, stage, wr, rd);
        b1.mma(acc, ssq, stage, wr, rd);
    } else {
        b0.mma(acc, ssq, stage, wr, rd);
    }

    // Per-wave accumulators to LDS (the staging tiles are free once every
    // wave is past its last MFMA), then sums in wave (K-slice) order.
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
    float* sred = red + KS * NW * MT * 256;
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(((wv * NW + j) * MT + mt) * 4 + r) * 64 + lane] = acc[j][mt][r];
    if constexpr (Batch::GAIN) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float s = ssq[mt];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            if (kq == 0) sred[(wv * MT + mt) * 16 + col] = s;
        }
    }
    __syncthreads();
    // Output (row m, column c of tile j): lane (m % 16 / 4) * 16 + c, element m % 4.
    auto out = [&](int j, int m, int c) {
        const int mt = m >> 4, r = m & 15;
        const int at = ((j * MT + mt) * 4 + (r & 3)) * 64 + (r >> 2) * 16 + c;
        float v = 0.f;
        for (int w = 0; w < KS; ++w) v += red[w * NW * MT * 256 + at];
        return v;
    };
    auto inv_rms = [&](int m) {
        const int mt = m >> 4, r = m & 15;
        float s = 0.f;
        for (int w = 0; w < KS; ++w) s += sred[(w * MT + mt) * 16 + r];
        return 1.0f / sqrtf(s / static_cast<float>(K) + a.eps);
    };

    if constexpr (EPI == kEpiQkv) {
        const int D = a.D, H2 = D / 2, hq = a.hq, hkv = a.hkv;
        for (int it = threadIdx.x; it < M * NP * 16; it += blockDim.x) {
            const int m = it / (NP * 16);
            const int p = (it >> 4) % NP, c = it & 15;
            const int d = (j0 + p) * 16 + c;           // < D / 2
            const bool first = it == static_cast<int>(threadIdx.x);
            const int pos = first ? pre_pos : a.ctx[m];
            const bool pos_ok = pos >= 0 && pos / BS < a.mbps;
            const int32_t blk = !pos_ok ? -1 : first ? pre_blk : a.table[static_cast<size_t>(m) * a.mbps + pos / BS];
            const bool blk_ok = pos_ok && blk >= 0 && blk < a.num_blocks;
            if (g == 0 && p == 0 && c == 0) {
                if (!pos_ok) atomicOr(a.err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
                else if (!blk_ok) atomicOr(a.err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            }
            if (!pos_ok || (head >= hq && !blk_ok)) continue;
            const float inv = inv_rms(m);
            const float y0 = inv * out(p, m, c);
            const float y1 = inv * out(NP + p, m, c);
            const int off = pos % BS;
            if (head < hq + hkv) {
                // the same float64 RoPE and single rounding as write_decode_kv
                const double x1 = static_cast<double>(y0);
                const double x2 = static_cast<double>(y1);
                double sn = pre_sn, cs = pre_cs;
                if (!first) sincos(static_cast<double>(pos) * rope.inv_freq[d], &sn, &cs);
                const uint16_t r1 = f64_to_bf16(__dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn)));
                const uint16_t r2 = f64_to_bf16(__dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn)));
                if (head < hq) {
                    const size_t at = (static_cast<size_t>(m) * hq + head) * D;
                    const double y1 = __dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn));
                    const double y2 = __dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn));
                    a.q_rot[at + d] = r1;
                    a.q_rot[at + d + H2] = r2;
                    a.q_lo[at + d] = f64_to_bf16(y1 - static_cast<double>(bf16_to_f32(r1)));
                    a.q_lo[at + d + H2] = f64_to_bf16(y2 - static_cast<double>(bf16_to_f32(r2)));
                } else {
                    const int gk = head - hq;
                    const size_t row = ((static_cast<size_t>(blk) * hkv + gk) * BS + off) * D;
                    if (a.fp8) {
                        uint8_t* dst = static_cast<uint8_t*>(a.kc) + row;
                        dst[d] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r1, a.kv_scales[gk]));
                        dst[d + H2] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r2, a.kv_scales[gk]));
                    } else {
                        uint16_t* dst = static_cast<uint16_t*>(a.kc) + row;
                        dst[d] = r1;
                        dst[d + H2] = r2;
                    }
                }
            } else {
                const int gv = head - hq - hkv;
                const size_t row = ((static_cast<size_t>(blk) * hkv + gv) * BS + off) * D;
                const uint16_t v0 = f32_to_bf16(y0), v1 = f32_to_bf16(y1);
                if (a.fp8) {
                    uint8_t* dst = static_cast<uint8_t*>(a.vc) + row;
                    dst[d] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(v0, a.kv_scales[hkv + gv]));
                    dst[d + H2] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(v1, a.kv_scales[hkv + gv]));
                } else {
                    uint16_t* dst = static_cast<uint16_t*>(a.vc) + row;
                    dst[d] = v0;
                    dst[d + H2] = v1;
                }
            }
        }
    } else if constexpr (EPI == kEpiSwiglu) {
        for (int it = threadIdx.x; it < M * NP * 16; it += blockDim.x) {
            const int m = it / (NP * 16);
            const int p = (it >> 4) % NP, c = it & 15;
            const float inv = inv_rms(m);
            const float gt = inv * out(p, m, c);
            const float up = inv * out(NP + p, m, c);
            const float silu = gt / (1.0f + expf(-gt));
            a.y_f32[static_cast<size_t>(m) * a.N + (j0 + p) * 16 + c] = silu * up;
        }
    } else {
        for (int it = threadIdx.x; it < M * NW * 16; it += blockDim.x) {
            const int m = it / (NW * 16);
            const int j = (it >> 4) % NW, c = it & 15;
            const size_t at = static_cast<size_t>(m) * a.N + tile[j] * 16 + c;
            const float y = out(j, m, c);
            const bool first = it == static_cast<int>(threadIdx.x);
            if constexpr (EPI == kEpiResidual) a.y_f32[at] = (first ? pre_res : bf16_to_f32(a.x_in[at])) + y;
            else a.y_bf16[at] = f32_to_bf16((first ? pre_res : a.x2[at]) + y);
        }
    }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Waves per workgroup of a projection: the largest divisor of the K batches
// that keeps the workgroup within its wave bound and the LDS cap, and the
// projection within the target wave count.
// down (256 workgroups at hidden 4096) may take up to 16 waves each: with
// the one-load fp32 activations a wave fits in 76 registers. At 4 K steps
// per batch the LDS cap (4352 bytes per wave) then allows 15, so it runs the
// largest divisor of its 96 batches below that, 12. On MI355X 8 waves, and
// 2 K steps per batch, measured within run-to-run spread of it; 6 waves was
// 1-2 us slower per layer.
constexpr int kProjTargetWavesDown = 4096;
template <int MT, int NW, int KB, int ACT, int EPI, bool HALF>
int proj_waves(int wgs, int K) {
    const int target = EPI == kEpiOut ? kProjTargetWavesDown : kProjTargetWaves;
    const int units = K / (KB * kKStep);
    const int max_ks = std::min<int>(proj_max_waves<MT, NW, KB, ACT, EPI, HALF>(),
                                     static_cast<int>(kProjLdsCap / proj_lds_per_wave<MT, NW, KB, ACT>()));
    int ks = 1;
    for (int d = 1; d <= std::min(units, max_ks); ++d)
        if (units % d == 0 && static_cast<int64_t>(wgs) * d <= target) ks = d;
    return ks;
}

// Tile shapes, measured on MI355X at batch 8: QKV and gate|up pair two tiles
// per workgroup (KB 2: 4 KiB of weights per wave per batch); o_proj and down
// take one tile (KB 4), which keeps 256 workgroups at hidden 4096 (groups of
// two or four tiles were slower: fewer workgroups than CUs).
constexpr int kNwQkv = 2, kNwGu = 2;
static_assert(kNwQkv == 2 || kNwQkv == 4, "QKV pairs per workgroup must divide D / 32 for D = 64 and 128");
constexpr int kNwO = 1, kNwD = 1;
// K steps per batch: NW * KB >= 4 loads (4 KiB of weights per wave).
constexpr int kb_for(int nw) { return nw >= 2 ? 2 : 4; }
constexpr int kKbD = kb_for(kNwD);
// o_proj (float32 activations as bf16 pairs, one tile): 4 K steps per batch,
// as down.
constexpr int kKbO = 4;

template <int MT, int NW, int KB, int ACT, int EPI, bool HALF = false>
void launch_proj(const ProjArgs& a, const mikv::RopeTable& rope, int wgs, hipStream_t st) {
    const int ks = proj_waves<MT, NW, KB, ACT, EPI, HALF>(wgs, a.K);
    const size_t lds = proj_lds_per_wave<MT, NW, KB, ACT>() * ks;
    hipLaunchKernelGGL((proj_kernel<MT, NW, KB, ACT, EPI, HALF>), dim3(wgs), dim3(64 * ks), lds, st, a, rope);
}

// Row tiles by batch; fp32 activations of at most 8 rows take the one-load
// form (GemmBatch HALF).
template <int NW, int KB, int ACT, int EPI>
void launch_proj_m(const ProjArgs& a, const mikv::RopeTable& rope, int wgs, hipStream_t st) {
    constexpr bool kF32 = ACT == kActF32Split || ACT == kActF32GainSplit;
    if (kF32 && a.M <= 8) launch_proj<1, NW, KB, ACT, EPI, kF32>(a, rope, wgs, st);
    else if (a.M <= 16) launch_proj<1, NW, KB, ACT, EPI>(a, rope, wgs, st);
    else launch_proj<2, NW, KB, ACT, EPI>(a, rope, wgs, st);
}

struct LayerPlan {
    int H, I, hq, hkv, D, nqkv;
    size_t off_qrot, off_qlo, off_attn, off_o, off_x2, off_a, total;
    size_t attn_bytes;
};

bool plan_layer(const mi_layer_config* c, int batch, int max_ctx, LayerPlan* pl) {
    pl->H = c->hidden;
    pl->I = c->intermediate;
    pl->hq = c->num_q_heads;
    pl->hkv = c->num_kv_heads;
    pl->D = c->head_dim;
    pl->nqkv = (pl->hq + 2 * pl->hkv) * pl->D;
    const size_t B = static_cast<size_t>(batch);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    pl->off_qrot = take(B * pl->hq * pl->D * 2);
    pl->off_qlo = take(B * pl->hq * pl->D * 2);
    pl->attn_bytes = mikv::attention_workspace_bytes(batch, pl->hq, pl->hkv, pl->D, max_ctx,
                                                     mikv::kDefaultSplitTokens);
    pl->off_attn = take(pl->attn_bytes);
    pl->off_o = take(B * pl->hq * pl->D * sizeof(float));
    pl->off_x2 = take(B * pl->H * sizeof(float));
    pl->off_a = take(B * pl->I * sizeof(float));
    pl->total = off;
    return true;
}

int check_layer(const mi_layer_config* c, const mi_kv_pool_s* p, int batch, int max_ctx) {
    if (!c || !p || batch < 0 || max_ctx < 0) return MI_ERR_INVALID_ARG;
    if (c->hidden <= 0 || c->intermediate <= 0 || !(c->rms_eps >= 0.f) || !(c->rope_theta > 0.0))
        return MI_ERR_INVALID_ARG;
    if (c->num_kv_heads != p->num_kv_heads || c->head_dim != p->head_dim) return MI_ERR_INVALID_ARG;
    if (!mikv::supported_group(c->num_q_heads, c->num_kv_heads)) return MI_ERR_UNSUPPORTED;
    if (c->hidden % mikv::kLayerDimMultiple || c->intermediate % mikv::kLayerDimMultiple ||
        (c->num_q_heads * c->head_dim) % mikv::kLayerDimMultiple)
        return MI_ERR_UNSUPPORTED;
    if (batch > mikv::kMaxLayerBatch) return MI_ERR_UNSUPPORTED;
    return MI_OK;
}

}  // namespace

extern "C" size_t mi_decoder_layer_workspace_bytes(const mi_layer_config* cfg, mi_kv_pool_t pool,
                                                   int32_t batch, int32_t max_ctx) {
    if (check_layer(cfg, pool, batch, max_ctx) != MI_OK) return 0;
    LayerPlan pl;
    plan_layer(cfg, batch, max_ctx, &pl);
    return pl.total;
}

extern "C" int mi_decoder_layer_decode(mi_kv_pool_t p, const mi_layer_config* cfg,
                                       const mi_layer_weights* w, const uint16_t* x_in,
                                       uint16_t* x_out, const int32_t* table, int32_t mbps,
                                       const int32_t* ctx, int32_t batch, int32_t max_ctx, void* ws,
                                       size_t ws_bytes, void* stream) {
    int rc = check_layer(cfg, p, batch, max_ctx);
    if (rc != MI_OK) return rc;
    if (!mikv::pool_has_device(p) || mbps <= 0) return MI_ERR_INVALID_ARG;
    if (batch == 0) return MI_OK;
    if (!w || !w->ln1_w || !w->w_qkv || !w->w_o || !w->ln2_w || !w->w_gate || !w->w_up || !w->w_down ||
        !x_in || !x_out || !table || !ctx || !ws || x_in == x_out)
        return MI_ERR_INVALID_ARG;
    LayerPlan pl;
    plan_layer(cfg, batch, max_ctx, &pl);
    if (ws_bytes < pl.total) return MI_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    uint16_t* q_rot = reinterpret_cast<uint16_t*>(base + pl.off_qrot);
    uint16_t* q_lo = reinterpret_cast<uint16_t*>(base + pl.off_qlo);
    float* o = reinterpret_cast<float*>(base + pl.off_o);
    float* x2 = reinterpret_cast<float*>(base + pl.off_x2);
    float* act = reinterpret_cast<float*>(base + pl.off_a);
    const int H = pl.H, I = pl.I, D = pl.D, hq = pl.hq, hkv = pl.hkv;
    const mikv::RopeTable rope = mikv::make_rope_table(cfg->rope_theta, D);

    // 1. [q|k|v] = (x * ln1_w) W_qkv^T / rms(x); RoPE, K/V append, q_rot
    {
        ProjArgs a{};
        a.A = x_in;
        a.gain = w->ln1_w;
        a.W0 = a.W1 = w->w_qkv;
        a.M = batch;
        a.K = H;
        a.N = pl.nqkv;
        a.eps = cfg->rms_eps;
        a.hq = hq;
        a.hkv = hkv;
        a.D = D;
        a.q_rot = q_rot;
        a.q_lo = q_lo;
        a.kc = p->k;
        a.vc = p->v;
        a.table = table;
        a.mbps = mbps;
        a.ctx = ctx;
        a.num_blocks = p->num_blocks;
        a.kv_scales = static_cast<const float*>(p->scales);
        a.err = p->err;
        a.fp8 = mikv::pool_fp8(p) ? 1 : 0;
        launch_proj_m<kNwQkv, kb_for(kNwQkv), kActGainSplit, kEpiQkv>(a, rope, pl.nqkv / 16 / kNwQkv, st);
    }
    // 2. paged GQA decode attention (query as a bf16 pair, float32 output)
    rc = mikv::launch_layer_attention(p, q_rot, q_lo, o, table, mbps, ctx, batch, hq,
                                      1.0f / sqrtf(static_cast<float>(D)), max_ctx,
                                      base + pl.off_attn, stream);
    if (rc != MI_OK) return rc;
    // 3. x2 = x + o W_o^T
    {
        ProjArgs a{};
        a.A = o;
        a.W0 = a.W1 = w->w_o;
        a.M = batch;
        a.K = hq * D;
        a.N = H;
        a.x_in = x_in;
        a.y_f32 = x2;
        launch_proj_m<kNwO, kKbO, kActF32Split, kEpiResidual>(a, rope, H / 16 / kNwO, st);
    }
    // 4. a = silu(r2 W_gate^T) * (r2 W_up^T), r2 = x2 * ln2_w / rms(x2)
    {
        ProjArgs a{};
        a.A = x2;
        a.gain = w->ln2_w;
        a.W0 = w->w_gate;
        a.W1 = w->w_up;
        a.M = batch;
        a.K = H;
        a.N = I;
        a.eps = cfg->rms_eps;
        a.y_f32 = act;
        launch_proj_m<kNwGu, kb_for(kNwGu), kActF32GainSplit, kEpiSwiglu>(a, rope, 2 * I / 16 / kNwGu, st);
    }
    // 5. out = bf16(x2 + a W_down^T)
    {
        ProjArgs a{};
        a.A = act;
        a.W0 = a.W1 = w->w_down;
        a.M = batch;
        a.K = I;
        a.N = H;
        a.x2 = x2;
        a.y_bf16 = x_out;
        launch_proj_m<kNwD, kKbD, kActF32Split, kEpiOut>(a, rope, H / 16 / kNwD, st);
    }
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

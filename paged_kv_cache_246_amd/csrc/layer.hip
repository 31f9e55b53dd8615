// Full decoder-layer decode step for gfx950: RMSNorm, QKV projection, RoPE
// and KV append, paged GQA attention, o_proj with residual, RMSNorm, SwiGLU
// MLP with residual (course project section 2.1: the components of a
// Qwen-style decoder layer assembled with residual connections and two
// norms; pre-norm order).
//
// The projections are skinny (M = batch <= 32 rows) and stream their
// weights once: bf16 MFMA 16x16x32 tiles, split over K so that enough waves
// stream in parallel; each split leaves an fp32 partial and the consumer
// kernel sums the partials in a fixed order (deterministic) and applies the
// epilogue. RMSNorm is x / rms(x) * w with a per-row scalar 1 / rms(x), so
// the GEMM runs on x * w and the consumer multiplies by 1 / rms(x). The
// activations x * w, x2 * w2 and silu(g) * u enter the MFMAs as bf16 hi + lo
// pairs (fp32-accurate); the attention output o enters as bf16.
//
// Launch sequence: gemm(qkv) -> rope_append -> attention (2 kernels) ->
// gemm(o) -> residual_norm -> gemm(gate|up) -> silu_mul -> gemm(down) ->
// residual_out.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "e4m3.h"
#include "internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BS = 16;
constexpr int kGemmTargetWaves = 3072;   // work items per projection
constexpr int kKStep = 32;               // K per MFMA
// MFMA steps per load batch for NW column tiles per wave: NW * KB >= 8
// weight loads (8 KiB per wave) per batch, at least 2 steps.
constexpr int batch_steps(int nw) { return nw >= 4 ? 2 : 8 / nw; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    if (x != x) return 0x7fc0;
    const float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if (static_cast<double>(f) != x) u |= 1u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint32_t mul_pack(uint32_t a, uint32_t g) {
    const float lo = bf16_to_f32(static_cast<uint16_t>(a)) * bf16_to_f32(static_cast<uint16_t>(g));
    const float hi = bf16_to_f32(static_cast<uint16_t>(a >> 16)) * bf16_to_f32(static_cast<uint16_t>(g >> 16));
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ------------------------------------------------------------- skinny GEMM
// P[s][m][n] = sum over k in split s of A[m][k] * W[n][k], m < M. W rows
// n < n_split come from W0, the rest from W1 (row n - n_split): this fuses
// gate and up. One wave per (16-column tile, K split). MFMA operand layout
// (16x16x32 bf16): lane l holds A[l % 16][8 (l / 16) .. +8) and
// B[8 (l / 16) .. +8)[l % 16]; the fp32 result D[4 (l / 16) + i][l % 16],
// i < 4. A is the activation rows (M padded to 16 per tile with zeros), B the
// weight rows (W^T), so each lane streams 16 contiguous bytes of one weight
// row per MFMA step. Lanes of padding rows (m >= M) load a real row again;
// their output rows are discarded.
//
// Activation modes: kActBf16 -- A is bf16; kActGainSplit -- A is bf16 x[m][k]
// times a bf16 gain[k], formed in fp32; kActF32Split -- A is fp32. In the two
// split modes the fp32 value a is fed as a_hi = bf16(a) plus a_lo =
// bf16(a - a_hi), two MFMAs per step, so the activation keeps ~16 significant
// bits instead of 8 (the weight stream is unchanged).
constexpr int kActBf16 = 0;
constexpr int kActGainSplit = 1;
constexpr int kActF32Split = 2;

__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = f32_to_bf16(v[2 * e]), h1 = f32_to_bf16(v[2 * e + 1]);
        const uint16_t l0 = f32_to_bf16(v[2 * e] - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16(v[2 * e + 1] - bf16_to_f32(h1));
        h[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        l[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
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
// tiles. load() only issues memory reads (activations, then weights); the
// activation's conversion to bf16 (hi, lo) happens in mma(), so prefetching
// the next batch never waits on its own loads.
//
// Weight loads come in one of two layouts. Direct (TR = false): each lane
// loads exactly its MFMA B-operand piece, i.e. 16 rows x 64 bytes per load
// instruction. Transposed (TR = true): 4 KB lanes share a row, so one
// instruction reads 64 / (4 KB) whole row segments of 64 KB bytes (full
// 128-byte lines at KB = 2); mma() writes the batch to the wave's LDS tile and
// reads it back in the MFMA layout (rows padded by 16 bytes).
template <int MT, int NW, int ACT, int KB, bool TR>
struct GemmBatch {
    static constexpr int AE = (ACT == kActF32Split) ? 4 : 2;   // activation element bytes
    static constexpr int LPR = 4 * KB;                         // transposed: lanes per row
    static constexpr int RPI = 64 / LPR;                       // transposed: rows per load
    static constexpr int ROWB = 64 * KB + 16;                  // LDS bytes per row (padded)
    static constexpr int LDS_BYTES = TR ? 16 * NW * ROWB : 16;
    uint4 w[KB][NW];       // direct: [step][tile]; transposed: flat [KB * NW] loads
    uint4 a0[KB][MT];      // bf16 activations, or fp32 elements 0..3
    uint4 a1[KB][MT];      // gain (kActGainSplit) or fp32 elements 4..7

    // kbyte: byte offset of the batch's first K column in a bf16 row.
    // Direct: woff[j] = lane's offset in tile j. Transposed: woff[0] = lane's
    // offset in load 0, wstep = bytes between consecutive loads (RPI rows).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rw, const uint32_t (&woff)[NW],
                                         uint32_t wstep, __amdgpu_buffer_rsrc_t ra,
                                         const uint32_t (&aoff)[MT], __amdgpu_buffer_rsrc_t rg,
                                         uint32_t goff, uint32_t kbyte) {
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t ak = (kbyte + u * kKStep * 2) / 2 * AE;
                a0[u][mt] = bload<0>(ra, aoff[mt], ak);
                if constexpr (ACT == kActF32Split) a1[u][mt] = bload<0>(ra, aoff[mt] + 16, ak);
                else if constexpr (ACT == kActGainSplit) a1[u][mt] = bload<0>(rg, goff, kbyte + u * kKStep * 2);
                else a1[u][mt] = make_uint4(0, 0, 0, 0);
            }
        if constexpr (TR) {
#pragma unroll
            for (int i = 0; i < KB * NW; ++i)
                w[i / NW][i % NW] = bload<kAuxStream>(rw, woff[0], kbyte + i * wstep);
        } else {
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int j = 0; j < NW; ++j) w[u][j] = bload<kAuxStream>(rw, woff[j], kbyte + u * kKStep * 2);
        }
    }

    // lds: the wave's tile; wr = lane's write offset of load 0 (bytes),
    // rd = lane's read offset for step 0 of tile 0
    __device__ __forceinline__ void mma(f32x4_t (&acc)[NW][MT], char* lds, uint32_t wr,
                                        uint32_t rd) const {
        if constexpr (TR) {
#pragma unroll
            for (int i = 0; i < KB * NW; ++i)
                *reinterpret_cast<uint4*>(lds + wr + i * RPI * ROWB) = w[i / NW][i % NW];
        }
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint4 hi = a0[u][mt], lo = make_uint4(0, 0, 0, 0);
                if constexpr (ACT != kActBf16) {
                    float v[8];
                    if constexpr (ACT == kActGainSplit) {
                        const uint32_t aw[4] = {a0[u][mt].x, a0[u][mt].y, a0[u][mt].z, a0[u][mt].w};
                        const uint32_t gw[4] = {a1[u][mt].x, a1[u][mt].y, a1[u][mt].z, a1[u][mt].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[2 * e] = bf16_to_f32(static_cast<uint16_t>(aw[e])) *
                                       bf16_to_f32(static_cast<uint16_t>(gw[e]));
                            v[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(aw[e] >> 16)) *
                                           bf16_to_f32(static_cast<uint16_t>(gw[e] >> 16));
                        }
                    } else {
                        const uint4 p0 = a0[u][mt], p1 = a1[u][mt];
                        v[0] = __uint_as_float(p0.x); v[1] = __uint_as_float(p0.y);
                        v[2] = __uint_as_float(p0.z); v[3] = __uint_as_float(p0.w);
                        v[4] = __uint_as_float(p1.x); v[5] = __uint_as_float(p1.y);
                        v[6] = __uint_as_float(p1.z); v[7] = __uint_as_float(p1.w);
                    }
                    split8(v, hi, lo);
                }
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    uint4 wv;
                    if constexpr (TR) wv = *reinterpret_cast<const uint4*>(lds + rd + j * 16 * ROWB + u * 64);
                    else wv = w[u][j];
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

// One wave per (group of NW 16-column tiles, K split). The split's K range is
// walked in batches of KB MFMA steps through a two-slot register ring: the
// next batch is in flight while the current one is multiplied (the loop is
// unrolled by two so the slots are fixed registers). A group never straddles
// the W0/W1 boundary (n_split is a multiple of 16 NW).
template <int MT, int NW, int ACT, bool TR>
__global__ __launch_bounds__(64) void gemm_skinny_kernel(
    const void* __restrict__ Aptr, const uint16_t* __restrict__ gain, int M, int K,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int n_split, int N,
    int k_chunk, float* __restrict__ P) {
    constexpr int KB = batch_steps(NW);        // MFMA steps per batch
    using Batch = GemmBatch<MT, NW, ACT, KB, TR>;
    __shared__ __align__(16) char lds[Batch::LDS_BYTES];
    const int grp = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int n_first = grp * NW * 16;
    const bool second = n_first >= n_split;
    const uint16_t* W = second ? W1 : W0;
    const int row0 = second ? n_first - n_split : n_first;
    const int rows = second ? N - n_split : n_split;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, static_cast<uint32_t>(static_cast<size_t>(rows) * K * 2));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Aptr, static_cast<uint32_t>(static_cast<size_t>(M) * K * Batch::AE));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gain, gain ? static_cast<uint32_t>(K) * 2 : 0u);
    uint32_t woff[NW];
    uint32_t wstep = 0, wr = 0, rd = 0;
    if constexpr (TR) {
        const int r_in = lane / Batch::LPR, piece = lane % Batch::LPR;
        woff[0] = (static_cast<uint32_t>(row0 + r_in) * K) * 2 + piece * 16;
#pragma unroll
        for (int j = 1; j < NW; ++j) woff[j] = 0;
        wstep = static_cast<uint32_t>(Batch::RPI) * K * 2;
        wr = r_in * Batch::ROWB + piece * 16;
        rd = col * Batch::ROWB + kq * 16;
    } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) woff[j] = (static_cast<uint32_t>(row0 + j * 16 + col) * K + kq * 8) * 2;
    }
    // Rows m >= M of the MFMA tile only feed output rows that are never
    // stored, so those lanes read row M - 1 again.
    uint32_t aoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        aoff[mt] = (static_cast<uint32_t>(min(mt * 16 + col, M - 1)) * K + kq * 8) * Batch::AE;
    const uint32_t goff = kq * 8 * 2;

    f32x4_t acc[NW][MT];
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr uint32_t STEP_BYTES = KB * kKStep * 2;
    const int nb = k_chunk / (KB * kKStep);   // batches (>= 1)
    const uint32_t kb0 = static_cast<uint32_t>(s) * k_chunk * 2;
    Batch b0, b1;
    b0.load(rw, woff, wstep, ra, aoff, rg, goff, kb0);
    int i = 0;
    for (; i + 2 < nb; i += 2) {
        b1.load(rw, woff, wstep, ra, aoff, rg, goff, kb0 + (i + 1) * STEP_BYTES);
        b0.mma(acc, lds, wr, rd);
        b0.load(rw, woff, wstep, ra, aoff, rg, goff, kb0 + (i + 2) * STEP_BYTES);
        b1.mma(acc, lds, wr, rd);
    }
    if (i + 1 < nb) {
        b1.load(rw, woff, wstep, ra, aoff, rg, goff, kb0 + (i + 1) * STEP_BYTES);
        b0.mma(acc, lds, wr, rd);
        b1.mma(acc, lds, wr, rd);
    } else {
        b0.mma(acc, lds, wr, rd);
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int n = n_first + j * 16 + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + kq * 4 + r;
                if (m < M) P[(static_cast<size_t>(s) * M + m) * N + n] = acc[j][mt][r];
            }
    }
}

// 1 / sqrt(mean(x^2) + eps) of a bf16 row (H a multiple of 8), by one block.
__device__ float block_inv_rms(const uint16_t* row, int H, float eps, float* red) {
    float ss = 0.f;
    for (int i = threadIdx.x * 8; i < H; i += blockDim.x * 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + i);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = bf16_to_f32(static_cast<uint16_t>(ws[e]));
            const float hi = bf16_to_f32(static_cast<uint16_t>(ws[e] >> 16));
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
        }
    }
#pragma unroll
    for (int x = 1; x < 64; x *= 2) ss += __shfl_xor(ss, x);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wv] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += red[w];
    return 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
}

// Sum of the K-split partials of one output, in split order; the loads are
// issued eight at a time so the sum costs few memory round trips.
__device__ __forceinline__ float sum_splits(const float* P, int S, size_t stride, size_t idx) {
    float v = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = (s0 + u < S) ? P[(s0 + u) * stride + idx] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) v += t[u];
    }
    return v;
}

// ------------------------------------------- RoPE + append from the QKV GEMM
// qkv[b][c] = inv_rms1(x_b) * sum_s P[s][b][c]. Then, at pos = ctx_b, the
// same float64 RoPE and single rounding as write_decode_kv: K slot gets
// bf16(RoPE(k)), V slot bf16(v), q_rot bf16(RoPE(q)); an 8-bit cache (FP8)
// stores the E4M3 codes of those bf16 K and V under the head's scales.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void rope_append_kernel(
    const float* __restrict__ P, int S, const uint16_t* __restrict__ x, int H, float eps,
    uint16_t* __restrict__ q_rot, void* __restrict__ kc, void* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens,
    int32_t batch, int32_t hq, int32_t hkv, int32_t num_blocks, mikv::RopeTable rope,
    const float* __restrict__ kv_scales, uint32_t* __restrict__ err) {
    constexpr int H2 = D / 2;
    __shared__ float red[4];
    const int b = blockIdx.x;
    const int nqkv = (hq + 2 * hkv) * D;
    const size_t stride = static_cast<size_t>(batch) * nqkv;
    const float* Pb = P + static_cast<size_t>(b) * nqkv;
    const float inv = block_inv_rms(x + static_cast<size_t>(b) * H, H, eps, red);
    const int pos = ctx_lens[b];
    const bool pos_ok = pos >= 0 && pos / BS < mbps;
    const int32_t blk = pos_ok ? table[static_cast<size_t>(b) * mbps + pos / BS] : -1;
    const bool blk_ok = pos_ok && blk >= 0 && blk < num_blocks;
    if (blockIdx.y == 0 && threadIdx.x == 0) {
        if (!pos_ok) atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        else if (!blk_ok) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
    }
    if (!pos_ok) return;
    const int off = pos % BS;
    const int n_rot = (hq + hkv) * H2;
    const int idx = blockIdx.y * blockDim.x + threadIdx.x;
    if (idx < n_rot) {
        const int h = idx / H2;
        const int i = idx - h * H2;
        if (h >= hq && !blk_ok) return;
        const double x1 = static_cast<double>(inv * sum_splits(Pb, S, stride, h * D + i));
        const double x2 = static_cast<double>(inv * sum_splits(Pb, S, stride, h * D + i + H2));
        const double a = static_cast<double>(pos) * rope.inv_freq[i];
        double sn, cs;
        sincos(a, &sn, &cs);
        const uint16_t r1 = f64_to_bf16(__dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn)));
        const uint16_t r2 = f64_to_bf16(__dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn)));
        if (h < hq) {
            uint16_t* dst = q_rot + (static_cast<size_t>(b) * hq + h) * D;
            dst[i] = r1;
            dst[i + H2] = r2;
        } else {
            const int g = h - hq;
            const size_t row = ((static_cast<size_t>(blk) * hkv + g) * BS + off) * D;
            if constexpr (FP8) {
                uint8_t* dst = static_cast<uint8_t*>(kc) + row;
                dst[i] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r1, kv_scales[g]));
                dst[i + H2] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r2, kv_scales[g]));
            } else {
                uint16_t* dst = static_cast<uint16_t*>(kc) + row;
                dst[i] = r1;
                dst[i + H2] = r2;
            }
        }
    } else if (blk_ok) {
        const int e = idx - n_rot;                 // element of the v heads
        if (e >= hkv * D) return;
        const int g = e / D;
        const int d = e - g * D;
        const float v = inv * sum_splits(Pb, S, stride, (hq + hkv) * D + e);
        const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + off) * D + d;
        if constexpr (FP8)
            static_cast<uint8_t*>(vc)[at] =
                static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(f32_to_bf16(v), kv_scales[hkv + g]));
        else
            static_cast<uint16_t*>(vc)[at] = f32_to_bf16(v);
    }
}

// x2 = x + sum_s P_o[s]; stores x2 and x2 * w2 (fp32) and, per block of 256
// columns, the partial sum of x2^2 (the 1 / rms(x2) of silu_mul).
__global__ __launch_bounds__(256) void residual_norm_kernel(
    const float* __restrict__ P, int S, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w2,
    int batch, int H, float* __restrict__ x2, float* __restrict__ xw2, float* __restrict__ ssq) {
    __shared__ float red[4];
    const int b = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    float ss = 0.f;
    if (i < H) {
        const size_t at = static_cast<size_t>(b) * H + i;
        const float v = bf16_to_f32(x[at]) + sum_splits(P, S, static_cast<size_t>(batch) * H, at);
        x2[at] = v;
        xw2[at] = v * bf16_to_f32(w2[i]);
        ss = v * v;
    }
#pragma unroll
    for (int k = 1; k < 64; k *= 2) ss += __shfl_xor(ss, k);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) ssq[static_cast<size_t>(b) * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// a = silu(r * gate) * (r * up) with r = 1 / rms(x2) from the partial sums
// of squares, gate/up summed over the K splits (fp32 output).
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ P, int S, int batch,
                                                       int I, int H, float eps, const float* __restrict__ ssq,
                                                       int nssq, float* __restrict__ a) {
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= I) return;
    const float tot = sum_splits(ssq + static_cast<size_t>(b) * nssq, nssq, 1, 0);
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
    const size_t stride = static_cast<size_t>(batch) * 2 * I;
    const size_t row = static_cast<size_t>(b) * 2 * I;
    const float g = inv * sum_splits(P, S, stride, row + i);
    const float u = inv * sum_splits(P, S, stride, row + I + i);
    const float silu = g / (1.0f + expf(-g));
    a[static_cast<size_t>(b) * I + i] = silu * u;
}

// out = bf16(x2 + sum_s P_d[s]).
__global__ __launch_bounds__(256) void residual_out_kernel(const float* __restrict__ P, int S,
                                                           int batch, int H, const float* __restrict__ x2,
                                                           uint16_t* __restrict__ out) {
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H) return;
    const size_t at = static_cast<size_t>(b) * H + i;
    out[at] = f32_to_bf16(x2[at] + sum_splits(P, S, static_cast<size_t>(batch) * H, at));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape of a projection's grid: NW column tiles per wave and S K splits.
// Measured on MI355X (8-row activations, transposed weight loads): 4 tiles
// (64 weight rows) per wave and about 1536 waves stream best; S is the
// largest divisor of the K batches that keeps the wave count within that.
struct GemmShape {
    int nw, splits;
};
GemmShape gemm_shape(int N, int K, int n_split) {
    const int tiles = N / 16;
    const int split_tiles = n_split / 16;
    int nw = 4;
    while (nw > 1 && (tiles % nw || split_tiles % nw)) nw /= 2;
    const int target = 1536;
    const int groups = tiles / nw;
    const int units = K / (kKStep * batch_steps(nw));
    int best = 1;
    for (int d = 1; d <= units; ++d)
        if (units % d == 0 && static_cast<int64_t>(groups) * d <= target) best = d;
    return {nw, best};
}

struct LayerPlan {
    int H, I, hq, hkv, D, nqkv;
    GemmShape g_qkv, g_o, g_gu, g_d;
    int s_qkv, s_o, s_gu, s_d;
    size_t off_pqkv, off_qrot, off_attn, off_o, off_po, off_x2, off_xw2, off_inv2, off_pgu, off_a,
        off_pd, total;
    size_t attn_bytes;
};

bool plan_layer(const mi_layer_config* c, int batch, int max_ctx, LayerPlan* pl) {
    pl->H = c->hidden;
    pl->I = c->intermediate;
    pl->hq = c->num_q_heads;
    pl->hkv = c->num_kv_heads;
    pl->D = c->head_dim;
    pl->nqkv = (pl->hq + 2 * pl->hkv) * pl->D;
    pl->g_qkv = gemm_shape(pl->nqkv, pl->H, pl->nqkv);
    pl->g_o = gemm_shape(pl->H, pl->hq * pl->D, pl->H);
    pl->g_gu = gemm_shape(2 * pl->I, pl->H, pl->I);
    pl->g_d = gemm_shape(pl->H, pl->I, pl->H);
    pl->s_qkv = pl->g_qkv.splits;
    pl->s_o = pl->g_o.splits;
    pl->s_gu = pl->g_gu.splits;
    pl->s_d = pl->g_d.splits;
    const size_t B = static_cast<size_t>(batch);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    pl->off_pqkv = take(pl->s_qkv * B * pl->nqkv * sizeof(float));
    pl->off_qrot = take(B * pl->hq * pl->D * 2);
    pl->attn_bytes = mikv::attention_workspace_bytes(batch, pl->hq, pl->hkv, pl->D, max_ctx,
                                                     mikv::kDefaultSplitTokens);
    pl->off_attn = take(pl->attn_bytes);
    pl->off_o = take(B * pl->hq * pl->D * 2);
    pl->off_po = take(pl->s_o * B * pl->H * sizeof(float));
    pl->off_x2 = take(B * pl->H * sizeof(float));
    pl->off_xw2 = take(B * pl->H * sizeof(float));
    pl->off_inv2 = take(B * ((pl->H + 255) / 256) * sizeof(float));
    pl->off_pgu = take(pl->s_gu * B * 2 * pl->I * sizeof(float));
    pl->off_a = take(B * pl->I * sizeof(float));
    pl->off_pd = take(pl->s_d * B * pl->H * sizeof(float));
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

#ifndef MIKV_GEMM_TRANSPOSED
#define MIKV_GEMM_TRANSPOSED true
#endif

template <int MT, int ACT>
void launch_gemm_mt(const void* A, const uint16_t* gain, int M, int K, const uint16_t* W0,
                    const uint16_t* W1, int n_split, int N, GemmShape g, float* P, hipStream_t st) {
    constexpr bool TR = MIKV_GEMM_TRANSPOSED;
    const dim3 grid(N / 16 / g.nw, g.splits);
    const int k_chunk = K / g.splits;
    if (g.nw == 8)
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, 8, ACT, TR>), grid, dim3(64), 0, st, A, gain, M, K, W0,
                           W1, n_split, N, k_chunk, P);
    else if (g.nw == 4)
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, 4, ACT, TR>), grid, dim3(64), 0, st, A, gain, M, K, W0,
                           W1, n_split, N, k_chunk, P);
    else if (g.nw == 2)
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, 2, ACT, TR>), grid, dim3(64), 0, st, A, gain, M, K, W0,
                           W1, n_split, N, k_chunk, P);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<MT, 1, ACT, TR>), grid, dim3(64), 0, st, A, gain, M, K, W0,
                           W1, n_split, N, k_chunk, P);
}

template <int ACT>
void launch_gemm_act(const void* A, const uint16_t* gain, int M, int K, const uint16_t* W0,
                     const uint16_t* W1, int n_split, int N, GemmShape g, float* P, hipStream_t st) {
    if (M <= 16) launch_gemm_mt<1, ACT>(A, gain, M, K, W0, W1, n_split, N, g, P, st);
    else launch_gemm_mt<2, ACT>(A, gain, M, K, W0, W1, n_split, N, g, P, st);
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
    float* p_qkv = reinterpret_cast<float*>(base + pl.off_pqkv);
    uint16_t* q_rot = reinterpret_cast<uint16_t*>(base + pl.off_qrot);
    uint16_t* o = reinterpret_cast<uint16_t*>(base + pl.off_o);
    float* p_o = reinterpret_cast<float*>(base + pl.off_po);
    float* x2 = reinterpret_cast<float*>(base + pl.off_x2);
    float* xw2 = reinterpret_cast<float*>(base + pl.off_xw2);
    float* inv2 = reinterpret_cast<float*>(base + pl.off_inv2);
    float* p_gu = reinterpret_cast<float*>(base + pl.off_pgu);
    float* a = reinterpret_cast<float*>(base + pl.off_a);
    float* p_d = reinterpret_cast<float*>(base + pl.off_pd);
    const int H = pl.H, I = pl.I, D = pl.D, hq = pl.hq, hkv = pl.hkv;

    // 1. [q|k|v] partials of bf16(x * ln1_w) W_qkv^T
    launch_gemm_act<kActGainSplit>(x_in, w->ln1_w, batch, H, w->w_qkv, w->w_qkv, pl.nqkv, pl.nqkv,
                                   pl.g_qkv, p_qkv, st);
    // 2. 1/rms(x), RoPE, append K/V, q_rot
    {
        const int items = (hq + hkv) * (D / 2) + hkv * D;
        const dim3 grid(batch, (items + 255) / 256);
        const mikv::RopeTable rope = mikv::make_rope_table(cfg->rope_theta, D);
        const bool f8 = mikv::pool_fp8(p);
        auto kern = D == 128 ? (f8 ? rope_append_kernel<128, true> : rope_append_kernel<128, false>)
                             : (f8 ? rope_append_kernel<64, true> : rope_append_kernel<64, false>);
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, p_qkv, pl.s_qkv, x_in, H, cfg->rms_eps, q_rot,
                           p->k, p->v, table, mbps, ctx, batch, hq, hkv, p->num_blocks, rope,
                           static_cast<const float*>(p->scales), p->err);
    }
    // 3. paged GQA decode attention
    rc = mikv::launch_paged_gqa_decode(p, q_rot, o, table, mbps, ctx, batch, hq,
                                       1.0f / sqrtf(static_cast<float>(D)), max_ctx,
                                       mikv::kDefaultSplitTokens, base + pl.off_attn, stream);
    if (rc != MI_OK) return rc;
    // 4. o_proj partials, 5. x2 = x + o W_o^T, bf16(x2 * ln2_w), 1/rms(x2)
    launch_gemm_act<kActBf16>(o, nullptr, batch, hq * D, w->w_o, w->w_o, H, H, pl.g_o, p_o, st);
    const int nssq = (H + 255) / 256;
    hipLaunchKernelGGL(residual_norm_kernel, dim3(nssq, batch), dim3(256), 0, st, p_o, pl.s_o, x_in,
                       w->ln2_w, batch, H, x2, xw2, inv2);
    // 6. gate|up partials, 7. a = silu(g) * u
    launch_gemm_act<kActF32Split>(xw2, nullptr, batch, H, w->w_gate, w->w_up, I, 2 * I, pl.g_gu, p_gu,
                                  st);
    hipLaunchKernelGGL(silu_mul_kernel, dim3((I + 255) / 256, batch), dim3(256), 0, st, p_gu, pl.s_gu,
                       batch, I, H, cfg->rms_eps, inv2, nssq, a);
    // 8. down partials, 9. out = x2 + a W_d^T
    launch_gemm_act<kActF32Split>(a, nullptr, batch, I, w->w_down, w->w_down, H, H, pl.g_d, p_d, st);
    hipLaunchKernelGGL(residual_out_kernel, dim3((H + 255) / 256, batch), dim3(256), 0, st, p_d, pl.s_d,
                       batch, H, x2, x_out);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

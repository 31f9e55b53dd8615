// Paged-KV decode kernels for gfx950 (CDNA4): write_decode_kv (RoPE, then
// append), split-K paged GQA decode attention with its combine, and the
// gather-through-the-block-table export used by tests.
//
// Pages: mini-infer README, "decode_batch key steps" (gather through the
// BlockTable, forward, write_decode_kv); course project section 2.1 (RoPE,
// GQA with KV heads shared by groups of query heads, KV-cache append);
// nxmr.cn inference-techniques article, section 5.1 (stable softmax: subtract
// the maximum, exponentiate, normalise by the sum) and section 4.1 (scores in
// FP32 or better).
//
// Data layout: K and V pools [num_blocks, Hkv, 16, D] bf16. One (block, kv
// head) tile is 16 * D * 2 bytes (4 KiB at D = 128), contiguous.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "e4m3.h"
#include "internal.h"

namespace {


constexpr int BS = 16;                // tokens per KV block
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleSlack = 8.0f; // log2 units: running max may lag by 2^8

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// float64 -> bf16, nearest-even, a single rounding: float32 rounded to odd
// (16 guard bits and a sticky bit), then rounded to bf16. Round-to-odd is the
// value truncated toward zero with its last bit set when inexact; truncation is
// the nearest-even float32 stepped one unit toward zero when that nearest
// value lies farther from zero than x (the two differ by at most one unit, and
// the hardware conversion rounds to nearest, so no emulated truncation is
// needed).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
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

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
    return static_cast<double>(__uint_as_float(static_cast<uint32_t>(h) << 16));
}

// ============================================================== write_decode_kv
// Per decode row (grid.x = sequence): rotation threads, each owning pair
// (i, i + D/2) of one head, q heads first, then the new k heads; then 16-byte
// pieces of the V copy; workgroups of 256 threads tile that index space
// (grid.y). The angle pos * theta^(-2i/D) (inverse frequencies from the host
// table), its sine and cosine and the rotation are float64 with separately
// rounded products, rounded once to bf16. An 8-bit cache (FMT = kFmtFp8)
// stores the E4M3 codes of that bf16 K and of v under the head's scales.
constexpr int kFmtBf16 = 0;
constexpr int kFmtFp8 = 1;

template <int D, int FMT>
__global__ __launch_bounds__(256) void write_decode_kv_kernel(
    const uint16_t* q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* q_rot, void* __restrict__ kc, void* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens,
    int32_t hq, int32_t hkv, int32_t num_blocks, mikv::RopeTable rope,
    const float* __restrict__ kv_scales, uint32_t* __restrict__ err) {
    constexpr int H2 = D / 2;
    const int row = blockIdx.x;               // row of q, k, v = sequence
    const int b = row;
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
    // Rotation threads: thread (h, i) owns pair i of head h (q heads, then
    // the new k heads) and computes its angle's float64 sine and cosine (a
    // decode row is latency bound: one head per thread).
    const int nh = hq + hkv;
    const int n_rot = nh * H2;
    const int idx = blockIdx.y * blockDim.x + threadIdx.x;
    if (idx < n_rot) {
        const int h = idx / H2;
        const int i = idx - h * H2;
        const uint16_t* src = h < hq ? q + (static_cast<size_t>(row) * hq + h) * D
                                     : k + (static_cast<size_t>(row) * hkv + (h - hq)) * D;
        const uint16_t in1 = src[i], in2 = src[i + H2];
        if (h >= hq && !blk_ok) return;
        double sn, cs;
        sincos(static_cast<double>(pos) * rope.inv_freq[i], &sn, &cs);
        const double x1 = bf16_to_f64(in1);
        const double x2 = bf16_to_f64(in2);
        const uint16_t r1 = f64_to_bf16_rne(__dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn)));
        const uint16_t r2 = f64_to_bf16_rne(__dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn)));
        if (h < hq) {
            uint16_t* dst = q_rot + (static_cast<size_t>(row) * hq + h) * D;
            dst[i] = r1;
            dst[i + H2] = r2;
        } else {
            const int g = h - hq;
            const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + off) * D;
            if constexpr (FMT == kFmtBf16) {
                uint16_t* dst = static_cast<uint16_t*>(kc) + at;
                dst[i] = r1;
                dst[i + H2] = r2;
            } else {
                uint8_t* dst = static_cast<uint8_t*>(kc) + at;
                const float sc = kv_scales[g];
                dst[i] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r1, sc));
                dst[i + H2] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r2, sc));
            }
        }
    } else if (blk_ok) {
        // V: 8 elements (16 input bytes) per thread
        const int piece = idx - n_rot;
        if (piece >= hkv * (D / 8)) return;
        const int g = piece / (D / 8);
        const int e = (piece - g * (D / 8)) * 8;
        const uint4 val = *reinterpret_cast<const uint4*>(v + (static_cast<size_t>(row) * hkv + g) * D + e);
        const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + off) * D + e;
        if constexpr (FMT == kFmtBf16)
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(vc) + at) = val;
        else
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(vc) + at) =
                mikv_dev::e4m3_quantize_bf16x8(val, kv_scales[hkv + g]);
    }
}

// ====================================================== prompt KV write (prefill)
// The packed rows of a prefill chunk (row i of sequence b: cu[b] <= i <
// cu[b + 1], position ctx_b + i - cu[b]) with the same arithmetic as
// write_decode_kv: the float64 angle, sine and cosine, a float64 rotation with
// separately rounded products and one rounding to bf16 (an 8-bit cache stores
// the E4M3 codes of that bf16 K and of v). Shaped for bandwidth: a workgroup
// takes kWpRows rows; every access is a 16-byte piece (8 dims of one head and
// the 8 dims D/2 further, which are their rotation partners, or 8 dims of v),
// consecutive threads take consecutive pieces of a row, and each thread
// loads all of its pieces of a pass before it rotates and stores any. The
// rows' sines and cosines (kWpRows x D/2, one per thread) sit in LDS. Rows with a bad position write nothing (fault bit); rows whose
// block id is bad write q_rot only.
constexpr int kWpRows = 1;          // prompt rows per workgroup
constexpr int kWpItems = 2;         // 16-byte pieces per thread per pass
constexpr int kWpThreads = 256;
template <int D, int FMT>
__global__ __launch_bounds__(kWpThreads) void write_prefill_kv_kernel(
    const uint16_t* q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* q_rot, void* __restrict__ kc, void* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ cu, int32_t batch, int32_t tokens, int32_t hq, int32_t hkv,
    int32_t num_blocks, mikv::RopeTable rope, const float* __restrict__ kv_scales,
    uint32_t* __restrict__ err) {
    constexpr int H2 = D / 2;
    constexpr int PC = H2 / 8;          // rotation pieces per head (each with its partner piece)
    constexpr int VC = D / 8;           // v pieces per head
    constexpr int R = kWpRows;
    constexpr int NT = kWpThreads;
    __shared__ int s_pos[R], s_blk[R];  // s_pos < 0: row not written; s_blk < 0: no K/V
    __shared__ double s_cs[R][H2], s_sn[R][H2];
    const int tid = threadIdx.x;
    const int row0 = static_cast<int>(blockIdx.x) * R;
    const int nh = hq + hkv;
    const int per_rot = nh * PC, per_v = hkv * VC;
    const int n_rot = R * per_rot;
    const int total = n_rot + R * per_v;
    // piece it: rotation pieces (row, head, j) first, then v pieces (row, kv head, e)
    struct Piece {
        uint4 lo, hi;
    };
    auto fetch = [&](int it) __attribute__((always_inline)) {
        Piece pc{make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
        if (it < n_rot) {
            const int r = it / per_rot, rem = it - r * per_rot;
            const int h = rem / PC, j = rem - h * PC;
            const int row = row0 + r;
            if (row < tokens) {
                const uint16_t* src = h < hq ? q + (static_cast<size_t>(row) * hq + h) * D
                                             : k + (static_cast<size_t>(row) * hkv + (h - hq)) * D;
                pc.lo = *reinterpret_cast<const uint4*>(src + 8 * j);
                pc.hi = *reinterpret_cast<const uint4*>(src + H2 + 8 * j);
            }
        } else if (it < total) {
            const int iv = it - n_rot;
            const int r = iv / per_v, rem = iv - r * per_v;
            const int g = rem / VC, e = (rem - g * VC) * 8;
            const int row = row0 + r;
            if (row < tokens)
                pc.lo = *reinterpret_cast<const uint4*>(v + (static_cast<size_t>(row) * hkv + g) * D + e);
        }
        return pc;
    };
    auto put = [&](int it, const Piece& pc) __attribute__((always_inline)) {
        if (it < n_rot) {
            const int r = it / per_rot, rem = it - r * per_rot;
            const int h = rem / PC, j = rem - h * PC;
            const int pos = s_pos[r], blk = s_blk[r];
            if (pos >= 0 && (h < hq || blk >= 0)) {
                const uint32_t a[4] = {pc.lo.x, pc.lo.y, pc.lo.z, pc.lo.w};
                const uint32_t c[4] = {pc.hi.x, pc.hi.y, pc.hi.z, pc.hi.w};
                uint32_t o1[4], o2[4];
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    uint32_t p1 = 0, p2 = 0;
#pragma unroll
                    for (int sh = 0; sh < 2; ++sh) {
                        const int d = 8 * j + 2 * w2 + sh;
                        const double x1 = bf16_to_f64(static_cast<uint16_t>(a[w2] >> (16 * sh)));
                        const double x2 = bf16_to_f64(static_cast<uint16_t>(c[w2] >> (16 * sh)));
                        const double cs = s_cs[r][d], sn = s_sn[r][d];
                        const uint32_t r1 = f64_to_bf16_rne(__dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn)));
                        const uint32_t r2 = f64_to_bf16_rne(__dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn)));
                        p1 |= r1 << (16 * sh);
                        p2 |= r2 << (16 * sh);
                    }
                    o1[w2] = p1;
                    o2[w2] = p2;
                }
                const uint4 v1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
                const uint4 v2 = make_uint4(o2[0], o2[1], o2[2], o2[3]);
                const int row = row0 + r;
                if (h < hq) {
                    uint16_t* dst = q_rot + (static_cast<size_t>(row) * hq + h) * D;
                    *reinterpret_cast<uint4*>(dst + 8 * j) = v1;
                    *reinterpret_cast<uint4*>(dst + H2 + 8 * j) = v2;
                } else {
                    const int g = h - hq;
                    const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + pos % BS) * D;
                    if constexpr (FMT == kFmtBf16) {
                        uint16_t* dst = static_cast<uint16_t*>(kc) + at;
                        *reinterpret_cast<uint4*>(dst + 8 * j) = v1;
                        *reinterpret_cast<uint4*>(dst + H2 + 8 * j) = v2;
                    } else {
                        uint8_t* dst = static_cast<uint8_t*>(kc) + at;
                        const float sc = kv_scales[g];
                        *reinterpret_cast<uint2*>(dst + 8 * j) = mikv_dev::e4m3_quantize_bf16x8(v1, sc);
                        *reinterpret_cast<uint2*>(dst + H2 + 8 * j) = mikv_dev::e4m3_quantize_bf16x8(v2, sc);
                    }
                }
            }
        } else if (it < total) {
            const int iv = it - n_rot;
            const int r = iv / per_v, rem = iv - r * per_v;
            const int g = rem / VC, e = (rem - g * VC) * 8;
            const int pos = s_pos[r], blk = s_blk[r];
            if (pos >= 0 && blk >= 0) {
                const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + pos % BS) * D + e;
                if constexpr (FMT == kFmtBf16)
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(vc) + at) = pc.lo;
                else
                    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(vc) + at) =
                        mikv_dev::e4m3_quantize_bf16x8(pc.lo, kv_scales[hkv + g]);
            }
        }
    };
    if (tid < R) {                      // row -> sequence, position, block (faults recorded per row)
        const int row = row0 + tid;
        int pos = -1, blk = -1;
        if (row < tokens) {
            int lo_b = 0, hi_b = batch - 1;     // last b with cu[b] <= row
            while (lo_b < hi_b) {
                const int mid = (lo_b + hi_b + 1) >> 1;
                if (cu[mid] <= row) lo_b = mid;
                else hi_b = mid - 1;
            }
            const int b = lo_b;
            pos = ctx_lens[b] + row - cu[b];
            const bool pos_ok = pos >= 0 && pos / BS < mbps;
            blk = pos_ok ? table[static_cast<size_t>(b) * mbps + pos / BS] : -1;
            const bool blk_ok = pos_ok && blk >= 0 && blk < num_blocks;
            if (!pos_ok) atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
            else if (!blk_ok) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            if (!pos_ok) pos = -1;
            if (!blk_ok) blk = -1;
        }
        s_pos[tid] = pos;
        s_blk[tid] = blk;
    }
    __syncthreads();
    for (int a2 = tid; a2 < R * H2; a2 += NT) {
        const int r = a2 / H2, i = a2 - r * H2;
        const int pos = s_pos[r];
        double sn = 0.0, cs = 1.0;
        if (pos >= 0) sincos(static_cast<double>(pos) * rope.inv_freq[i], &sn, &cs);
        s_cs[r][i] = cs;
        s_sn[r][i] = sn;
    }
    __syncthreads();
    for (int base = 0; base < total; base += NT * kWpItems) {
        Piece pc[kWpItems];
#pragma unroll
        for (int u = 0; u < kWpItems; ++u) pc[u] = fetch(base + u * NT + tid);
#pragma unroll
        for (int u = 0; u < kWpItems; ++u) put(base + u * NT + tid, pc[u]);
    }
}

// Whole-pool quantisation of bf16 caches into an 8-bit pool: 8 elements per
// thread, grid-stride over the pool (grid.y: 0 = K, 1 = V); the KV head of an
// element picks its scale.
template <int D>
__global__ __launch_bounds__(256) void quantize_pool_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, size_t pieces, int32_t hkv,
    const float* __restrict__ kv_scales) {
    const bool is_v = blockIdx.y == 1;
    const uint16_t* src = is_v ? v_src : k_src;
    uint8_t* dst = is_v ? vc : kc;
    constexpr size_t kPiecesPerTile = BS * D / 8;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < pieces;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int g = static_cast<int>((i / kPiecesPerTile) % hkv);
        const float s = kv_scales[(is_v ? hkv : 0) + g];
        const uint4 w = reinterpret_cast<const uint4*>(src)[i];
        reinterpret_cast<uint2*>(dst)[i] = mikv_dev::e4m3_quantize_bf16x8(w, s);
    }
}

// ================================================= work partition (stream-K)
// The work of one call is the list of 16-token tiles of every segment
// (sequence b, kv head g), g fastest; segment (b, g) has nt_b =
// ceil((ctx_b + 1) / 16) tiles, and a sequence whose length is out of range
// has none. W waves split the list into W equal contiguous ranges,
// [floor(w T / W), floor((w + 1) T / W)), so every wave streams the same
// number of tiles whatever the length mix. A segment cut by a range boundary
// leaves one fp32 partial per piece; a segment inside one range is finished by
// that wave. W = min(grid, ceil(T / min_tiles)): small workloads get many
// short ranges (a tile fetch costs a memory round trip), large ones are
// capped by the resident waves.
constexpr int kMaxBatch = 1024;      // sequences per call (LDS prefix table)

// TP[b] = first global tile of sequence b, TP[batch] = T. One wave; every lane
// of the wave returns T. Records a length fault in *bad.
__device__ __forceinline__ int build_tile_prefix(const int32_t* __restrict__ ctx_lens, int batch,
                                                 int mbps, int max_ctx, int hkv, int* TP,
                                                 bool* bad, int lane) {
    int carry = 0;
    bool any_bad = false;
    for (int base = 0; base < batch; base += 64) {
        const int b = base + lane;
        int v = 0;
        if (b < batch) {
            const int c = ctx_lens[b];
            const bool badb = c < 0 || c > max_ctx || c + 1 > mbps * BS;
            any_bad |= badb;
            v = badb ? 0 : (c + BS) / BS * hkv;
        }
#pragma unroll
        for (int x = 1; x < 64; x *= 2) {
            const int y = __shfl_up(v, x);
            if (lane >= x) v += y;
        }
        if (b < batch) TP[b + 1] = carry + v;
        carry += __shfl(v, 63);
    }
    if (lane == 0) TP[0] = 0;
    *bad = __ballot(any_bad) != 0;
    return carry;
}

__device__ __forceinline__ int active_waves(int T, int grid_waves, int min_tiles) {
    return max(1, min(grid_waves, (T + min_tiles - 1) / min_tiles));
}

__device__ __forceinline__ int range_start(int w, int T, int W) {
    return static_cast<int>(static_cast<int64_t>(w) * T / W);
}

// The wave whose range holds tile x (0 <= x < T): the largest w with
// floor(w T / W) <= x, i.e. floor(((x + 1) W - 1) / T).
__device__ __forceinline__ int wave_of_tile(int x, int T, int W) {
    const int w = static_cast<int>((static_cast<int64_t>(x + 1) * W - 1) / T);
    return min(max(w, 0), W - 1);
}

// Largest b with TP[b] <= x (that segment is non-empty for x < T).
__device__ __forceinline__ int find_sequence(const int* TP, int batch, int x) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (TP[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ======================================================= paged GQA decode
// One wavefront per work range (see the partition above). For each segment
// piece in its range the wave streams the piece's K/V tiles in logical order
// through a register ring (tile i in slot i % (PF + 1), the PF tiles after
// the one being consumed in flight); the G query heads of the segment share
// every tile. The piece ends either as the final bf16 output (the whole
// segment) or as an fp32 partial (m, l, acc) in slot 2w (first piece of the
// range) or 2w + 1 (last piece), merged by the combine kernel.
// Both contractions of a tile run on the matrix cores. Lane l = 16 q + n
// (n = l % 16, q = l / 16) of the wave:
//  - scores S^T = K Q^T by 16x16x32 bf16 MFMAs: rows are the 16 tokens of
//    the tile, columns the query heads (n < G; the other columns are
//    padding), the D dims split in slices of 32. The lane holds token row n
//    of K and column n of Q^T for its 8 dims of each slice and receives the
//    scores of tokens 4q .. 4q + 3 for head n;
//  - O^T += V^T P^T by 16x16x16 bf16 MFMAs: B = P^T is exactly the score
//    layout (tokens 4q .. 4q + 3 of head n, rounded to bf16), A = V^T takes
//    dim psi of tokens 4q .. 4q + 3, built by 16-bit permutes from the four
//    token rows the lane loads (D / 16 dims each). Output dims of MFMA jj
//    in row 4q + r are psi = (D / 16)(4q + r) + jj, so every lane owns D / 4
//    consecutive dims of its head.
// Softmax state is per head: the running max m is shared by the 4 lanes of
// a head, each lane keeps the sum of its own p; a tile raises m only when
// some score exceeds it by more than the slack (one wave vote), then the 4
// lanes agree on the new maximum through two lane exchanges.
// With an 8-bit cache (E4M3) the codes are widened to bf16 exactly by the
// hardware conversion; the per-head scales multiply the scores and the
// weighted V sum.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D, int FMT>
struct MfmaTile {
    static constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1;       // bytes per element
    static constexpr int ROW = D * ESZ;                         // bytes per token row
    static constexpr int NQK = D / 32;                          // score MFMAs
    static constexpr int NKL = FMT == kFmtBf16 ? NQK : NQK / 2; // 16-byte K loads per lane
    static constexpr int NPV = D / 16;                          // output MFMAs
    static constexpr int VB = D * ESZ / 16;                     // V bytes per lane per row
    static constexpr int VW = VB / 4;                           // ... in 32-bit words
    static constexpr int BW = D / 32;                           // bf16 words per lane per row
    static_assert(NKL >= 1 && VW >= 1, "head_dim");
};

// NB-byte load of words; NT: non-temporal (each tile streamed once, decode),
// else an ordinary cached load (tiles read again, prefill).
template <int NB, bool NT>
__device__ __forceinline__ void ld_words(const char* base, uint32_t off, uint32_t (&w)[NB / 4]) {
    if constexpr (NB == 16) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4* p = reinterpret_cast<const u32x4*>(base + off);
        const u32x4 t = NT ? __builtin_nontemporal_load(p) : *p;
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (NB == 8) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2* p = reinterpret_cast<const u32x2*>(base + off);
        const u32x2 t = NT ? __builtin_nontemporal_load(p) : *p;
        w[0] = t.x; w[1] = t.y;
    } else {
        const unsigned int* p = reinterpret_cast<const unsigned int*>(base + off);
        w[0] = NT ? __builtin_nontemporal_load(p) : *p;
    }
}

// Two E4M3 codes (bytes 0-1 or 2-3 of w) -> two bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                            static_cast<int>(w), 1.0f, HI));
}

struct MfmaSoftmax {
    float m;      // running max of head n (log2 units), shared by its 4 lanes
    float l;      // this lane's sum of 2^(s - m)
};

// Fixed softmax reference (prefill, shared-tile kernel): a query's reference
// m is the largest score of the first key step and is never raised, so no
// step rescales the accumulators. The weights 2^(s - m) and their sum stay
// finite while the sum stays within 2^64; a chunk in which one did not is
// repeated with the online rescaling form.
constexpr float kFixedHeadroomSum = 18446744073709551616.0f;   // 2^64

// Operand builders of one 16-token tile.
// K operand of 32-dim slice j: the lane's key row, 8 dims (bf16; E4M3 codes
// widened exactly).
template <int D, int FMT>
__device__ __forceinline__ uint4 k_operand(const uint4 (&kr)[MfmaTile<D, FMT>::NKL], int j) {
    if constexpr (FMT == kFmtBf16) {
        return kr[j];
    } else {
        const uint4 w = kr[j / 2];
        const uint32_t w0 = (j & 1) ? w.z : w.x;
        const uint32_t w1 = (j & 1) ? w.w : w.y;
        return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                          fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
    }
}

// V^T operands (one per output MFMA): dim psi of key rows 4q4 .. 4q4+3, built
// by 16-bit permutes of the four rows the lane loaded. With tail, rows >=
// valid_rows are zeroed (their bits may be NaN and 0 * NaN would reach the
// sum).
template <int D, int FMT>
__device__ __forceinline__ void v_operands(const uint32_t (&vr)[4][MfmaTile<D, FMT>::VW], int q4,
                                           int valid_rows, bool tail,
                                           s16x4_t (&vt)[MfmaTile<D, FMT>::NPV]) {
    using TL = MfmaTile<D, FMT>;
    uint32_t bw[4][TL::BW];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool ok = !tail || 4 * q4 + r < valid_rows;
#pragma unroll
        for (int e = 0; e < TL::BW; ++e) {
            uint32_t x;
            if constexpr (FMT == kFmtBf16) x = vr[r][e];
            else x = (e & 1) ? fp8x2_to_bf16x2<true>(vr[r][e / 2]) : fp8x2_to_bf16x2<false>(vr[r][e / 2]);
            bw[r][e] = ok ? x : 0u;
        }
    }
#pragma unroll
    for (int jj = 0; jj < TL::NPV; ++jj) {
        const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
        const int e = jj / 2;
        const uint32_t lo = __builtin_amdgcn_perm(bw[1][e], bw[0][e], sel);
        const uint32_t hi = __builtin_amdgcn_perm(bw[3][e], bw[2][e], sel);
        vt[jj] = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
    }
}

// Online-softmax step of one column block: scores of key rows 4q4 .. 4q4+3
// for column n, masked (column dead, or with tail a key row >= qlim), the
// running max raised only past the slack (one wave vote), the lane's sum
// updated; returns the P^T operand (weights rounded to bf16).
//
// RAW (prefill): the max is taken on the raw scores and scaled once (the
// scale is positive) and the scale folds into the exponent's FMA; without
// tail nothing is masked -- a dead column there has a zero query, finite
// scores and an output that is never stored.
// With PLO the rounding remainders of the weights, bf16(p - bf16(p)), go to
// *plo (the weighted V sum then takes p at about 16 significant bits).
template <int NPV, bool RAW = false, bool PLO = false>
__device__ __forceinline__ bf16x4_t softmax_step(f32x4_t s, float sl2, bool col_ok, int q4, int qlim,
                                                 bool tail, MfmaSoftmax& sm, f32x4_t (&o)[NPV],
                                                 bf16x4_t* plo = nullptr) {
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sc[i] = RAW ? s[i] : s[i] * sl2;
        if (!RAW || tail) {
            const bool ok = col_ok && (!tail || 4 * q4 + i < qlim);
            sc[i] = ok ? sc[i] : kNegInf;
        }
    }
    const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * (RAW ? sl2 : 1.0f);
    if (__ballot(mx > sm.m + kRescaleSlack) != 0) {
        float hm = fmaxf(mx, __shfl_xor(mx, 16));
        hm = fmaxf(hm, __shfl_xor(hm, 32));
        const float mn = fmaxf(sm.m, hm);
        const float alpha = __builtin_amdgcn_exp2f(sm.m - mn);
        sm.m = mn;
        sm.l *= alpha;
#pragma unroll
        for (int jj = 0; jj < NPV; ++jj) o[jj] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(RAW ? fmaf(sc[i], sl2, -sm.m) : sc[i] - sm.m);
        sm.l += p[i];
    }
    const bf16x4_t hi = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                         static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
    if constexpr (PLO)
        *plo = bf16x4_t{static_cast<__bf16>(p[0] - static_cast<float>(hi[0])),
                        static_cast<__bf16>(p[1] - static_cast<float>(hi[1])),
                        static_cast<__bf16>(p[2] - static_cast<float>(hi[2])),
                        static_cast<__bf16>(p[3] - static_cast<float>(hi[3]))};
    return hi;
}

// One 16-token tile for QB column blocks of 16 (query heads in decode, QB = 1;
// query tokens in prefill). The K operands and the V^T operands are built
// once and shared by every block. Column n of block c is live if col_ok[c];
// with tail, key row t counts for it only if t < qlim[c] (the rows written so
// far in decode, the causal limit in prefill), and V rows >= valid_rows are
// zeroed.
// PAIR: the query operand is a bf16 pair, qb the rounded value and ql the
// rounding remainder, and so are the softmax weights (about 16 significant
// bits each); both contractions take one MFMA per half.
template <int D, int FMT, int QB, bool RAW = false, bool PAIR = false>
__device__ __forceinline__ void mfma_consume(const uint4 (&kr)[MfmaTile<D, FMT>::NKL],
                                             const uint32_t (&vr)[4][MfmaTile<D, FMT>::VW],
                                             const uint4 (&qb)[QB][MfmaTile<D, FMT>::NQK],
                                             const uint4 (&ql)[PAIR ? QB : 1][MfmaTile<D, FMT>::NQK],
                                             float sl2, const bool (&col_ok)[QB], int q4,
                                             const int (&qlim)[QB], int valid_rows, bool tail,
                                             MfmaSoftmax (&sm)[QB],
                                             f32x4_t (&o)[QB][MfmaTile<D, FMT>::NPV]) {
    using TL = MfmaTile<D, FMT>;
    uint4 a[TL::NQK];
#pragma unroll
    for (int j = 0; j < TL::NQK; ++j) a[j] = k_operand<D, FMT>(kr, j);
    bf16x4_t pb[QB];
    bf16x4_t pl[PAIR ? QB : 1];
#pragma unroll
    for (int c = 0; c < QB; ++c) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TL::NQK; ++j) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[j]),
                                                        __builtin_bit_cast(bf16x8_t, qb[c][j]), s, 0, 0, 0);
            if constexpr (PAIR)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[j]),
                                                            __builtin_bit_cast(bf16x8_t, ql[c][j]), s, 0, 0, 0);
        }
        pb[c] = softmax_step<TL::NPV, RAW, PAIR>(s, sl2, col_ok[c], q4, qlim[c], tail, sm[c], o[c],
                                                        PAIR ? &pl[c] : nullptr);
    }
    s16x4_t vt[TL::NPV];
    v_operands<D, FMT>(vr, q4, valid_rows, tail, vt);
#pragma unroll
    for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int jj = 0; jj < TL::NPV; ++jj) {
            o[c][jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                vt[jj], __builtin_bit_cast(s16x4_t, pb[c]), o[c][jj], 0, 0, 0);
            if constexpr (PAIR)
                o[c][jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    vt[jj], __builtin_bit_cast(s16x4_t, pl[c]), o[c][jj], 0, 0, 0);
        }
}

// Per-wave state of the QB column blocks (RAW: the prefill softmax form;
// PAIR: query and weights as bf16 pairs).
template <int D, int FMT, int QB, bool RAW = false, bool PAIR = false>
struct MfmaCols {
    using TL = MfmaTile<D, FMT>;
    uint4 qb[QB][TL::NQK];
    uint4 ql[PAIR ? QB : 1][TL::NQK];
    bool col_ok[QB];
    MfmaSoftmax sm[QB];
    f32x4_t o[QB][TL::NPV];
    float sl2;
    int q4;

    __device__ __forceinline__ void consume(const uint4 (&kr)[TL::NKL], const uint32_t (&vr)[4][TL::VW],
                                            const int (&qlim)[QB], int valid_rows, bool tail) {
        mfma_consume<D, FMT, QB, RAW, PAIR>(kr, vr, qb, ql, sl2, col_ok, q4, qlim, valid_rows, tail,
                                                   sm, o);
    }
    // unmasked tile, or a tile whose rows >= valid_rows are masked for every column
    __device__ __forceinline__ void consume_rows(const uint4 (&kr)[TL::NKL], const uint32_t (&vr)[4][TL::VW],
                                                 int valid_rows, bool tail) {
        int lim[QB];
#pragma unroll
        for (int c = 0; c < QB; ++c) lim[c] = valid_rows;
        consume(kr, vr, lim, valid_rows, tail);
    }
};

// NT: non-temporal K/V loads (decode: every tile is read once per call);
// prefill re-reads tiles across query blocks and heads and keeps them cached.
template <int D, int FMT, int PF, bool NT = true>
struct MfmaRing {
    using TL = MfmaTile<D, FMT>;
    uint4 kr[PF + 1][TL::NKL];
    uint32_t vr[PF + 1][4][TL::VW];
    const char* kbase;
    const char* vbase;
    size_t blk_stride;
    uint32_t koff[TL::NKL];
    uint32_t voff[4];
    int32_t my_id;   // lane i holds the chunk's i-th block id

    template <int S>
    __device__ __forceinline__ void load(int tile) {
        const int32_t id = __builtin_amdgcn_readlane(my_id, tile);
        const char* kb = kbase + static_cast<size_t>(id) * blk_stride;
        const char* vb = vbase + static_cast<size_t>(id) * blk_stride;
#pragma unroll
        for (int j = 0; j < TL::NKL; ++j) {
            uint32_t w[4];
            ld_words<16, NT>(kb, koff[j], w);
            kr[S][j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ld_words<TL::VB, NT>(vb, voff[r], vr[S][r]);
    }
    template <int S>
    __device__ __forceinline__ void prologue(int nblk) {
        if constexpr (S < PF) {
            load<S>(min(S, nblk - 1));
            prologue<S + 1>(nblk);
        }
    }
    // PF + 1 full tiles i .. i+PF; tile i+U prefetches tile i+U+PF
    template <int U, class Cols>
    __device__ __forceinline__ void steady(int i, int nblk, Cols& cols) {
        if constexpr (U <= PF) {
            load<(U + PF) % (PF + 1)>(min(i + U + PF, nblk - 1));
            cols.consume_rows(kr[U], vr[U], BS, false);
            steady<U + 1>(i, nblk, cols);
        }
    }
    // the last nblk - i (1 .. PF+1) tiles, all already requested; the final
    // one may be partial (valid_rows < 16)
    template <int U, class Cols>
    __device__ __forceinline__ void rest(int i, int nblk, int valid_rows, Cols& cols) {
        if constexpr (U <= PF) {
            const int tile = i + U;
            if (tile < nblk - 1) {
                cols.consume_rows(kr[U], vr[U], BS, false);
            } else if (tile == nblk - 1) {
                if (valid_rows == BS) cols.consume_rows(kr[U], vr[U], BS, false);
                else cols.consume_rows(kr[U], vr[U], valid_rows, true);
            }
            rest<U + 1>(i, nblk, valid_rows, cols);
        }
    }
    // every tile of [0, nblk): the unrolled ring loop. prep() runs once the
    // first tiles are requested, before any is consumed (work whose loads
    // may then overlap the tiles' own).
    template <class Cols, class Prep>
    __device__ __forceinline__ void run(int nblk, int last_rows, Cols& cols, Prep&& prep) {
        prologue<0>(nblk);
        prep();
        int i = 0;
        for (; i + PF + 1 < nblk; i += PF + 1) steady<0>(i, nblk, cols);
        load<PF>(min(i + PF, nblk - 1));
        rest<0>(i, nblk, last_rows, cols);
    }
    template <class Cols>
    __device__ __forceinline__ void run(int nblk, int last_rows, Cols& cols) {
        run(nblk, last_rows, cols, [] {});
    }
};

// The new token of a one-launch decode step (STEP kernels): q, k and v (bf16
// [B, Hq, D], [B, Hkv, D], [B, Hkv, D]), the RoPE inverse frequencies and an
// optional q_rot output.
struct StepToken {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* q_rot;
    mikv::RopeTable rope;
};

// STEP: write_decode_kv happens inside the attention launch. The wave whose
// piece holds a segment's last tile owns the segment's write: before loading
// any tile it rotates the new k (and, if asked for, the G query heads for
// q_rot) with the float64 rotation and single rounding of write_decode_kv,
// stores k and v into the slot, and the piece waits for those stores before
// its first tile load, so the new token is read back from the cache like
// every other. Each segment's last tile belongs to exactly one piece: every
// slot is written once, and read only by its writer. Every piece also needs
// the rotated query heads as its MFMA operand; those it rotates itself in
// float32 (angle reduced to a fraction of a turn in float64, hardware sine
// and cosine), which differs from the float64 rotation by at most one bf16
// rounding. The wave loads its q elements and their rotation partners
// before its first tile load and rotates them once that load is issued, so
// the two memory round trips overlap.
template <int D, int G, int FMT>
__device__ __forceinline__ void step_owner_write(const StepToken& tok, int b, int g, int hkv, int pos,
                                                 int32_t blk, const float* kv_scales, uint8_t* kc,
                                                 uint8_t* vc, int lane) {
    constexpr int H2 = D / 2;
    const int i = lane % H2;
    double sn, cs;
    sincos(static_cast<double>(pos) * tok.rope.inv_freq[i], &sn, &cs);
    auto rot = [&](uint16_t a, uint16_t c, uint16_t& r1, uint16_t& r2) {
        const double x1 = bf16_to_f64(a), x2 = bf16_to_f64(c);
        r1 = f64_to_bf16_rne(__dsub_rn(__dmul_rn(x1, cs), __dmul_rn(x2, sn)));
        r2 = f64_to_bf16_rne(__dadd_rn(__dmul_rn(x2, cs), __dmul_rn(x1, sn)));
    };
    if (tok.q_rot) {
        const size_t qrow = (static_cast<size_t>(b) * hkv + g) * G * D;
#pragma unroll
        for (int p = lane; p < G * H2; p += 64) {
            const int h = p / H2;
            uint16_t r1, r2;
            rot(tok.q[qrow + h * D + i], tok.q[qrow + h * D + i + H2], r1, r2);
            tok.q_rot[qrow + h * D + i] = r1;
            tok.q_rot[qrow + h * D + i + H2] = r2;
        }
    }
    if (blk >= 0) {
        const size_t krow = (static_cast<size_t>(b) * hkv + g) * D;
        const size_t at = ((static_cast<size_t>(blk) * hkv + g) * BS + pos % BS) * D;
        if (lane < H2) {
            uint16_t r1, r2;
            rot(tok.k[krow + i], tok.k[krow + i + H2], r1, r2);
            if constexpr (FMT == kFmtBf16) {
                uint16_t* dst = reinterpret_cast<uint16_t*>(kc) + at;
                dst[i] = r1;
                dst[i + H2] = r2;
            } else {
                const float ks = kv_scales[g];
                kc[at + i] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r1, ks));
                kc[at + i + H2] = static_cast<uint8_t>(mikv_dev::e4m3_quantize_bf16(r2, ks));
            }
        }
        if (lane < D / 8) {
            const uint4 val = *reinterpret_cast<const uint4*>(tok.v + krow + 8 * lane);
            if constexpr (FMT == kFmtBf16)
                *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(vc) + at + 8 * lane) = val;
            else
                *reinterpret_cast<uint2*>(vc + at + 8 * lane) =
                    mikv_dev::e4m3_quantize_bf16x8(val, kv_scales[hkv + g]);
        }
    }
}

// cos and sin of the H2 RoPE angles at pos, float32, into LDS (lane i < H2:
// angle i, reduced to a fraction of a turn in float64 first).
template <int D>
__device__ __forceinline__ void step_angles(const StepToken& tok, int pos, float2* CS, int lane) {
    constexpr int H2 = D / 2;
    if (lane < H2) {
        const double turns = static_cast<double>(pos) * tok.rope.inv_freq[lane] * 0.15915494309189535;
        const float frac = static_cast<float>(turns - floor(turns));
        CS[lane] = make_float2(__builtin_amdgcn_cosf(frac), __builtin_amdgcn_sinf(frac));
    }
}

// Rotates the lane's 8-dim slices of its query head (raw bf16 in x, the
// partner dims d +- D/2 in px; slice j starts at dim dim0[j]) with the LDS
// angle table, into bf16 operand words.
template <int D, int NQ>
__device__ __forceinline__ void step_rotate_q(const uint4 (&x)[NQ], const uint4 (&px)[NQ],
                                              const int (&dim0)[NQ], const float2* CS,
                                              uint4 (&qb)[NQ]) {
    constexpr int H2 = D / 2;
    auto el = [](const uint4& u, int e) {
        const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    };
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const bool lo = dim0[j] < H2;
        const float2* cs = CS + (lo ? dim0[j] : dim0[j] - H2);
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float2 a = cs[e], c = cs[e + 1];
            const float x0 = el(x[j], e), x1 = el(x[j], e + 1);
            const float p0 = el(px[j], e), p1 = el(px[j], e + 1);
            const float r0 = lo ? fmaf(x0, a.x, -p0 * a.y) : fmaf(x0, a.x, p0 * a.y);
            const float r1 = lo ? fmaf(x1, c.x, -p1 * c.y) : fmaf(x1, c.x, p1 * c.y);
            wd[e / 2] = static_cast<uint32_t>(f32_to_bf16_rne(r0)) |
                        (static_cast<uint32_t>(f32_to_bf16_rne(r1)) << 16);
        }
        qb[j] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

// Inputs and outputs of the attention inside the decoder layer (LAYER
// kernels): the query arrives as a bf16 pair (q_rot, the rounded value, and
// q_lo, the remainder), the softmax weights enter the V product as bf16
// pairs too, and the output is stored in float32 for the o projection, which
// takes it as a bf16 pair.
struct LayerIO {
    const uint16_t* q_lo;      // [B, Hq, D] bf16
    float* out;                // [B, Hq, D] float32
};

// The cache pointers are read-only (and restrict) except in STEP kernels,
// which write the new token's slot.
template <bool STEP> struct CachePtr { typedef const uint8_t* __restrict__ type; };
template <> struct CachePtr<true> { typedef uint8_t* type; };

template <int D, int G, int FMT, int PF, bool STEP, bool LAYER = false>
__global__ __launch_bounds__(64) void paged_attn_mfma_kernel(
    const uint16_t* __restrict__ q_rot, typename CachePtr<STEP>::type kc,
    typename CachePtr<STEP>::type vc, const int32_t* __restrict__ table, int32_t mbps,
    const int32_t* __restrict__ ctx_lens, int32_t batch, int32_t hkv, int32_t num_blocks,
    int32_t max_ctx, int32_t min_tiles, float scale_log2, const float* __restrict__ kv_scales,
    float* __restrict__ part_acc, float2* __restrict__ part_ml, uint16_t* __restrict__ out,
    uint32_t* __restrict__ err, StepToken tok, LayerIO lio) {
    static_assert(!(STEP && LAYER), "the layer path runs the two-call form");
    using TL = MfmaTile<D, FMT>;
    constexpr int NPV = TL::NPV;
    constexpr size_t TILE = static_cast<size_t>(BS) * TL::ROW;   // bytes per (block, head) tile
    __shared__ int TP[kMaxBatch + 1];
    __shared__ __align__(16) float2 CS[STEP ? D / 2 : 1];       // RoPE cos, sin at pos (STEP)
    const int w = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const bool head_ok = n < G;

    bool bad_len;
    const int T = build_tile_prefix(ctx_lens, batch, mbps, max_ctx, hkv, TP, &bad_len, lane);
    __syncthreads();
    if (bad_len && w == 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
    if (T == 0) return;
    const int W = active_waves(T, gridDim.x, min_tiles);
    if (w >= W) return;
    const int start = range_start(w, T, W);
    const int end = range_start(w + 1, T, W);
    const size_t blk_stride = static_cast<size_t>(hkv) * TILE;

    int pos = start;
    int b = find_sequence(TP, batch, pos);
    bool first_piece = true;
    while (pos < end) {
        while (__builtin_amdgcn_readfirstlane(TP[b + 1]) <= pos) ++b;
        const int seg0 = __builtin_amdgcn_readfirstlane(TP[b]);
        const int nt = (__builtin_amdgcn_readfirstlane(TP[b + 1]) - seg0) / hkv;
        const int rel = pos - seg0;
        const int g = rel / nt;
        const int t0 = rel - g * nt;
        const int t1 = min(nt, t0 + (end - pos));
        const int L = ctx_lens[b] + 1;

        // Q^T operand: head n, the lane's 8 dims of each 32-dim slice (the
        // same dims its K row supplies)
        MfmaCols<D, FMT, 1, false, LAYER> cols;
        auto load_q = [&](size_t qoff) {
#pragma unroll
            for (int j = 0; j < TL::NQK; ++j) {
                const int d0 = FMT == kFmtBf16 ? 32 * j + 8 * q4 : 64 * (j / 2) + 16 * q4 + 8 * (j & 1);
                cols.qb[0][j] = head_ok ? *reinterpret_cast<const uint4*>(q_rot + qoff + d0) : make_uint4(0, 0, 0, 0);
                if constexpr (LAYER)
                    cols.ql[0][j] = head_ok ? *reinterpret_cast<const uint4*>(lio.q_lo + qoff + d0)
                                            : make_uint4(0, 0, 0, 0);
            }
        };
        // block ids of the piece's first chunk (lane i: its i-th tile)
        int32_t id0 = 0;
        if (lane < min(64, t1 - t0)) id0 = table[static_cast<size_t>(b) * mbps + t0 + lane];
        // STEP: the raw query slices and their rotation partners
        uint4 qraw[TL::NQK], qpart[TL::NQK];
        int qdim[TL::NQK];
        if constexpr (STEP) {
            const int pos = L - 1;
            if (t1 == nt) {                   // this piece holds the segment's last tile
                int32_t blk = table[static_cast<size_t>(b) * mbps + pos / BS];
                if (blk < 0 || blk >= num_blocks) blk = -1;     // recorded by the tile loop
                step_owner_write<D, G, FMT>(tok, b, g, hkv, pos, blk, kv_scales, kc, vc, lane);
            }
            const uint16_t* qh = tok.q + (static_cast<size_t>(b) * hkv * G + g * G + (head_ok ? n : 0)) * D;
#pragma unroll
            for (int j = 0; j < TL::NQK; ++j) {
                qdim[j] = FMT == kFmtBf16 ? 32 * j + 8 * q4 : 64 * (j / 2) + 16 * q4 + 8 * (j & 1);
                qraw[j] = *reinterpret_cast<const uint4*>(qh + qdim[j]);
                qpart[j] = *reinterpret_cast<const uint4*>(qh + (qdim[j] + D / 2) % D);
            }
            step_angles<D>(tok, pos, CS, lane);
            // the owner's stores complete before the piece's first tile load
            // (the barrier's fence keeps the tile loads below this point)
            if (t1 == nt) __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        } else {
            load_q((static_cast<size_t>(b) * hkv * G + g * G + (head_ok ? n : 0)) * D);
        }
        cols.sl2 = scale_log2;
        float vscale = 1.f;
        if constexpr (FMT == kFmtFp8) {
            cols.sl2 *= kv_scales[g];
            vscale = kv_scales[hkv + g];
        }
        cols.q4 = q4;
        cols.col_ok[0] = head_ok;
        cols.sm[0] = MfmaSoftmax{head_ok ? kNegInf : 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < NPV; ++jj) cols.o[0][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        MfmaSoftmax& sm = cols.sm[0];
        f32x4_t (&o)[NPV] = cols.o[0];

        MfmaRing<D, FMT, PF> ring;
        ring.kbase = reinterpret_cast<const char*>(kc) + static_cast<size_t>(g) * TILE;
        ring.vbase = reinterpret_cast<const char*>(vc) + static_cast<size_t>(g) * TILE;
        ring.blk_stride = blk_stride;
#pragma unroll
        for (int j = 0; j < TL::NKL; ++j) ring.koff[j] = n * TL::ROW + 64 * j + 16 * q4;
#pragma unroll
        for (int r = 0; r < 4; ++r) ring.voff[r] = (4 * q4 + r) * TL::ROW + TL::VB * n;

        for (int s0 = t0; s0 < t1; s0 += 64) {
            const int nblk = min(64, t1 - s0);
            int32_t id = id0;
            if (s0 != t0 && lane < nblk) id = table[static_cast<size_t>(b) * mbps + s0 + lane];
            const bool bad_id = lane < nblk && (id < 0 || id >= num_blocks);
            if (__ballot(bad_id) != 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            ring.my_id = bad_id ? 0 : id;
            // The loop is unrolled by PF + 1 so ring slots are compile-time
            // registers (no copies that would wait on in-flight loads), and
            // every prefetch in it is unconditional (clamped to the last
            // tile, a cache hit), so the wait before each tile covers exactly
            // the older loads.
            const int last_rows = (s0 + nblk == nt) ? L - (nt - 1) * BS : BS;
            ring.run(nblk, last_rows, cols, [&] {
                if constexpr (STEP) {
                    if (s0 == t0) {
                        step_rotate_q<D>(qraw, qpart, qdim, CS, cols.qb[0]);
#pragma unroll
                        for (int j = 0; j < TL::NQK; ++j)
                            if (!head_ok) cols.qb[0][j] = make_uint4(0, 0, 0, 0);
                    }
                }
            });
        }

        // head totals of the lane sums (same bits in the 4 lanes of a head)
        float lt = sm.l + __shfl_xor(sm.l, 16);
        lt += __shfl_xor(lt, 32);
        const bool whole = (t0 == 0 && t1 == nt);
        const size_t slot = 2 * static_cast<size_t>(w) + (first_piece ? 0 : 1);
        if (head_ok) {
            const int dbase = NPV * 4 * q4;     // first of the lane's D/4 dims
            if (whole && LAYER) {
                const float inv = vscale / lt;
                float* of = lio.out + (static_cast<size_t>(b) * hkv * G + g * G + n) * D + dbase;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int e = 0; e < NPV / 4; ++e)
                        reinterpret_cast<float4*>(of + NPV * r)[e] =
                            make_float4(o[4 * e][r] * inv, o[4 * e + 1][r] * inv,
                                        o[4 * e + 2][r] * inv, o[4 * e + 3][r] * inv);
            } else if (whole) {
                const float inv = vscale / lt;
                uint16_t* oh = out + (static_cast<size_t>(b) * hkv * G + g * G + n) * D + dbase;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t wd[NPV / 2];
#pragma unroll
                    for (int e = 0; e < NPV / 2; ++e)
                        wd[e] = static_cast<uint32_t>(f32_to_bf16_rne(o[2 * e][r] * inv)) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(o[2 * e + 1][r] * inv)) << 16);
                    if constexpr (NPV == 8)
                        *reinterpret_cast<uint4*>(oh + NPV * r) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                    else
                        *reinterpret_cast<uint2*>(oh + NPV * r) = make_uint2(wd[0], wd[1]);
                }
            } else {
                float* dst = part_acc + (slot * G + n) * D + dbase;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int e = 0; e < NPV / 4; ++e)
                        reinterpret_cast<float4*>(dst + NPV * r)[e] =
                            make_float4(o[4 * e][r] * vscale, o[4 * e + 1][r] * vscale,
                                        o[4 * e + 2][r] * vscale, o[4 * e + 3][r] * vscale);
                if (q4 == 0) part_ml[slot * G + n] = make_float2(sm.m, lt);
            }
        }
        pos += t1 - t0;
        first_piece = false;
    }
}

// ================================ paged GQA decode, per-segment form
// Short segments (every one at most kSegWaves x kSegMaxTilesPerWave tiles,
// few of them): one workgroup of kSegWaves waves per (KV head g,
// sequence b). Wave w streams tiles [w nt / kSegWaves, (w + 1) nt /
// kSegWaves) of the segment through the MFMA kernel's register ring and
// consume step, then the waves' (m, l, acc) are merged through LDS in wave
// order and the bf16 output is stored: the whole call is one launch, with
// no split partials in memory and no combine launch. Same tile arithmetic
// as the stream-K kernel; the results depend only on logical positions.
// A sequence whose length is out of range gets NaN outputs and a recorded
// fault, as in the stream-K path.
// Beyond three tiles per wave the waves' serial tile round trips cost more
// than the stream-K kernel's combine launch (segments of 65 tiles: 8.1
// instead of 2 tiles per wave, 17-25 against 17-21 us per step).
constexpr int kSegWaves = 8;              // waves per workgroup (two per SIMD)
constexpr int kSegMaxTilesPerWave = 3;    // longest segment: 24 tiles (384 tokens)
constexpr int kSegMaxSegments = 512;      // workgroups (batch x KV heads)

template <int D, int G, int FMT, int PF>
__global__ __launch_bounds__(64 * kSegWaves) void paged_attn_seg_kernel(
    const uint16_t* __restrict__ q_rot, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens, int32_t hkv,
    int32_t num_blocks, int32_t max_ctx, float scale_log2, const float* __restrict__ kv_scales,
    uint16_t* __restrict__ out, uint32_t* __restrict__ err) {
    using TL = MfmaTile<D, FMT>;
    constexpr int NPV = TL::NPV;
    constexpr size_t TILE = static_cast<size_t>(BS) * TL::ROW;   // bytes per (block, head) tile
    constexpr int NT = 64 * kSegWaves;
    __shared__ float s_m[kSegWaves][G], s_l[kSegWaves][G];
    __shared__ float s_o[kSegWaves][G][D];
    const int g = blockIdx.x;
    const int b = blockIdx.y;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const bool head_ok = n < G;
    uint16_t* o_seg = out + (static_cast<size_t>(b) * hkv * G + g * G) * D;

    const int c = ctx_lens[b];
    if (c < 0 || c > max_ctx || c + 1 > mbps * BS) {        // uniform over the workgroup
        if (g == 0 && threadIdx.x == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        for (int i = threadIdx.x; i < G * D; i += NT) o_seg[i] = 0x7fc0;
        return;
    }
    const int L = c + 1;
    const int nt = (L + BS - 1) / BS;
    const int t0 = wv * nt / kSegWaves;
    const int t1 = (wv + 1) * nt / kSegWaves;

    MfmaCols<D, FMT, 1> cols;
    const size_t qoff = (static_cast<size_t>(b) * hkv * G + g * G + (head_ok ? n : 0)) * D;
#pragma unroll
    for (int j = 0; j < TL::NQK; ++j) {
        const int d0 = FMT == kFmtBf16 ? 32 * j + 8 * q4 : 64 * (j / 2) + 16 * q4 + 8 * (j & 1);
        cols.qb[0][j] = head_ok ? *reinterpret_cast<const uint4*>(q_rot + qoff + d0) : make_uint4(0, 0, 0, 0);
    }
    cols.sl2 = scale_log2;
    float vscale = 1.f;
    if constexpr (FMT == kFmtFp8) {
        cols.sl2 *= kv_scales[g];
        vscale = kv_scales[hkv + g];
    }
    cols.q4 = q4;
    cols.col_ok[0] = head_ok;
    cols.sm[0] = MfmaSoftmax{head_ok ? kNegInf : 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NPV; ++jj) cols.o[0][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (t0 < t1) {
        MfmaRing<D, FMT, PF> ring;
        ring.kbase = reinterpret_cast<const char*>(kc) + static_cast<size_t>(g) * TILE;
        ring.vbase = reinterpret_cast<const char*>(vc) + static_cast<size_t>(g) * TILE;
        ring.blk_stride = static_cast<size_t>(hkv) * TILE;
#pragma unroll
        for (int j = 0; j < TL::NKL; ++j) ring.koff[j] = n * TL::ROW + 64 * j + 16 * q4;
#pragma unroll
        for (int r = 0; r < 4; ++r) ring.voff[r] = (4 * q4 + r) * TL::ROW + TL::VB * n;
        for (int s0 = t0; s0 < t1; s0 += 64) {
            const int nblk = min(64, t1 - s0);
            int32_t id = 0;
            if (lane < nblk) id = table[static_cast<size_t>(b) * mbps + s0 + lane];
            const bool bad_id = lane < nblk && (id < 0 || id >= num_blocks);
            if (__ballot(bad_id) != 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            ring.my_id = bad_id ? 0 : id;
            const int last_rows = (s0 + nblk == nt) ? L - (nt - 1) * BS : BS;
            ring.run(nblk, last_rows, cols);
        }
    }

    // the wave's partial: head totals of the lane sums, the lane's D / 4 dims
    const MfmaSoftmax& sm = cols.sm[0];
    float lt = sm.l + __shfl_xor(sm.l, 16);
    lt += __shfl_xor(lt, 32);
    if (head_ok) {
        const int dbase = NPV * 4 * q4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int jj = 0; jj < NPV; ++jj) s_o[wv][n][dbase + NPV * r + jj] = cols.o[0][jj][r];
        if (q4 == 0) {
            s_m[wv][n] = sm.m;
            s_l[wv][n] = lt;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += NT) {
        const int h = i / D;
        const int d = i - h * D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kSegWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float l = 0.f, a = 0.f;
#pragma unroll
        for (int w = 0; w < kSegWaves; ++w) {
            const float mw = s_m[w][h];
            const float f = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            l = fmaf(f, s_l[w][h], l);
            a = fmaf(f, s_o[w][h][d], a);
        }
        o_seg[i] = f32_to_bf16_rne(a * (vscale / l));
    }
}

// ===================================== paged GQA decode, dot-product form
// The decode attention with both contractions on the vector ALUs instead of
// the matrix cores: the same work partition, ring of in-flight tiles and
// partial format as the MFMA kernel above, selected for mi_paged_gqa_decode
// by the pool flag MI_POOL_DECODE_DOT (the comparison design). Lane
// l = LAM r + c of the wave holds key rows r, r + TPI, ... (TPI = 64 / LAM
// rows per load instruction) of a 16-token tile and, of each row, the
// 8-element pieces c + LAM j; q.k is a chain of packed bf16 dot products with
// fp32 accumulation, summed over the LAM lanes of a row by DPP moves. Every
// lane keeps a running max, sum and weighted V sum per query head over its
// own rows; the rows are merged at the end of a segment piece. E4M3 codes are
// widened to bf16 exactly before use; the per-head scales multiply the
// scores and the weighted V sum, as in the MFMA kernel.
template <int D, int LAM, int FMT>
struct DotTile {
    static constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1;     // bytes per element
    static constexpr int TPI = 64 / LAM;                      // key rows per load instruction
    static constexpr int NT = BS / TPI;                       // key rows per lane per tile
    static constexpr int NJ = D / (8 * LAM);                  // 8-element pieces per lane per row
    static constexpr int PB = 8 * ESZ;                        // bytes per piece
    static constexpr int ROW = D * ESZ;                       // bytes per key row
    static_assert(NJ >= 1 && NJ * 8 * LAM == D, "head_dim / lane split");
};

// Lane sums inside a DPP row of 16 lanes (row_mask and bank_mask all on).
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i within each 8
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15 - i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LAM consecutive lanes of one key row (LAM = 8 or 16); each of
// them ends with the same bits (every step adds a commutative pair).
template <int LAM>
__device__ __forceinline__ float dot_row_sum(float x) {
    x += dpp_move<kDppQuadSwap1>(x);
    x += dpp_move<kDppQuadSwap2>(x);
    x += dpp_move<kDppHalfMirror>(x);
    if constexpr (LAM == 16) x += dpp_move<kDppRowMirror>(x);
    return x;
}

// An 8-element piece as four bf16 pairs (E4M3 codes widened exactly).
template <int FMT>
__device__ __forceinline__ uint4 dot_piece(const uint32_t (&w)[FMT == kFmtBf16 ? 4 : 2]) {
    if constexpr (FMT == kFmtBf16) {
        return make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        return make_uint4(fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                          fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1]));
    }
}

__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w),
                                          acc, false);
    return acc;
}

// Per-wave state: the G heads' query pieces, running max (log2 units), sums
// and weighted V sums over the lane's key rows.
template <int D, int G, int LAM, int FMT>
struct DotCols {
    using TS = DotTile<D, LAM, FMT>;
    static constexpr int NT = TS::NT;
    static constexpr int NJ = TS::NJ;
    static constexpr int PW = TS::PB / 4;
    uint4 qv[G][NJ];
    float m[G], l[G];
    float acc[G][NJ][8];
    float sl2;
    int r;

    // One tile: with TAIL, key rows >= valid_rows are left out by selection
    // (their bits may be anything, NaN included).
    template <bool TAIL>
    __device__ __forceinline__ void consume(const uint32_t (&kw)[NT][NJ][PW], const uint32_t (&vw)[NT][NJ][PW],
                                            int valid_rows) {
        constexpr int TPI = TS::TPI;
        bool valid[NT];
        uint4 kp[NT][NJ], vp[NT][NJ];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            valid[t] = !TAIL || t * TPI + r < valid_rows;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                kp[t][j] = dot_piece<FMT>(kw[t][j]);
                vp[t][j] = valid[t] ? dot_piece<FMT>(vw[t][j]) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) a = dot8_bf16(qv[h][j], kp[t][j], a);
                s[t] = dot_row_sum<LAM>(a) * sl2;
                if (TAIL && !valid[t]) s[t] = kNegInf;
            }
            float mx = s[0];
#pragma unroll
            for (int t = 1; t < NT; ++t) mx = fmaxf(mx, s[t]);
            if (mx > m[h] + kRescaleSlack) {          // lane-local: its own rows only
                const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
                m[h] = mx;
                l[h] *= alpha;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][j][e] *= alpha;
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float p = __builtin_amdgcn_exp2f(s[t] - m[h]);
                if (TAIL) p = valid[t] ? p : 0.f;
                l[h] += p;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const uint32_t w4[4] = {vp[t][j].x, vp[t][j].y, vp[t][j].z, vp[t][j].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[h][j][2 * e] = fmaf(p, __uint_as_float(w4[e] << 16), acc[h][j][2 * e]);
                        acc[h][j][2 * e + 1] = fmaf(p, __uint_as_float(w4[e] & 0xffff0000u), acc[h][j][2 * e + 1]);
                    }
                }
            }
        }
    }
};

// Ring of PF + 1 tiles in registers (the MFMA ring's scheme: slots are
// compile-time, every prefetch is unconditional and clamped to the last tile).
template <int D, int LAM, int FMT, int PF>
struct DotRing {
    using TS = DotTile<D, LAM, FMT>;
    static constexpr int NT = TS::NT;
    static constexpr int NJ = TS::NJ;
    static constexpr int PW = TS::PB / 4;
    uint32_t kw[PF + 1][NT][NJ][PW];
    uint32_t vw[PF + 1][NT][NJ][PW];
    const char* kbase;
    const char* vbase;
    size_t blk_stride;
    uint32_t loff[NT][NJ];
    int32_t my_id;   // lane i holds the chunk's i-th block id

    template <int S>
    __device__ __forceinline__ void load(int tile) {
        const int32_t id = __builtin_amdgcn_readlane(my_id, tile);
        const char* kb = kbase + static_cast<size_t>(id) * blk_stride;
        const char* vb = vbase + static_cast<size_t>(id) * blk_stride;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < NJ; ++j) ld_words<TS::PB, true>(kb, loff[t][j], kw[S][t][j]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < NJ; ++j) ld_words<TS::PB, true>(vb, loff[t][j], vw[S][t][j]);
    }
    template <int S>
    __device__ __forceinline__ void prologue(int nblk) {
        if constexpr (S < PF) {
            load<S>(min(S, nblk - 1));
            prologue<S + 1>(nblk);
        }
    }
    template <int U, class Cols>
    __device__ __forceinline__ void steady(int i, int nblk, Cols& cols) {
        if constexpr (U <= PF) {
            load<(U + PF) % (PF + 1)>(min(i + U + PF, nblk - 1));
            cols.template consume<false>(kw[U], vw[U], BS);
            steady<U + 1>(i, nblk, cols);
        }
    }
    template <int U, class Cols>
    __device__ __forceinline__ void rest(int i, int nblk, int valid_rows, Cols& cols) {
        if constexpr (U <= PF) {
            const int tile = i + U;
            if (tile < nblk - 1 || (tile == nblk - 1 && valid_rows == BS))
                cols.template consume<false>(kw[U], vw[U], BS);
            else if (tile == nblk - 1)
                cols.template consume<true>(kw[U], vw[U], valid_rows);
            rest<U + 1>(i, nblk, valid_rows, cols);
        }
    }
    template <class Cols>
    __device__ __forceinline__ void run(int nblk, int last_rows, Cols& cols) {
        prologue<0>(nblk);
        int i = 0;
        for (; i + PF + 1 < nblk; i += PF + 1) steady<0>(i, nblk, cols);
        load<PF>(min(i + PF, nblk - 1));
        rest<0>(i, nblk, last_rows, cols);
    }
};

template <int D, int G, int LAM, int FMT, int PF>
__global__ __launch_bounds__(64) void paged_attn_dot_kernel(
    const uint16_t* __restrict__ q_rot, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens, int32_t batch,
    int32_t hkv, int32_t num_blocks, int32_t max_ctx, int32_t min_tiles, float scale_log2,
    const float* __restrict__ kv_scales, float* __restrict__ part_acc, float2* __restrict__ part_ml,
    uint16_t* __restrict__ out, uint32_t* __restrict__ err) {
    using TS = DotTile<D, LAM, FMT>;
    constexpr int NT = TS::NT;
    constexpr int NJ = TS::NJ;
    constexpr size_t TILE = static_cast<size_t>(BS) * TS::ROW;   // bytes per (block, head) tile
    __shared__ int TP[kMaxBatch + 1];
    const int w = blockIdx.x;
    const int lane = threadIdx.x;
    const int r = lane / LAM;
    const int c = lane % LAM;

    bool bad_len;
    const int T = build_tile_prefix(ctx_lens, batch, mbps, max_ctx, hkv, TP, &bad_len, lane);
    __syncthreads();
    if (bad_len && w == 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
    if (T == 0) return;
    const int W = active_waves(T, gridDim.x, min_tiles);
    if (w >= W) return;
    const int start = range_start(w, T, W);
    const int end = range_start(w + 1, T, W);

    int pos = start;
    int b = find_sequence(TP, batch, pos);
    bool first_piece = true;
    while (pos < end) {
        while (__builtin_amdgcn_readfirstlane(TP[b + 1]) <= pos) ++b;
        const int seg0 = __builtin_amdgcn_readfirstlane(TP[b]);
        const int nt = (__builtin_amdgcn_readfirstlane(TP[b + 1]) - seg0) / hkv;
        const int rel = pos - seg0;
        const int g = rel / nt;
        const int t0 = rel - g * nt;
        const int t1 = min(nt, t0 + (end - pos));
        const int L = ctx_lens[b] + 1;

        DotCols<D, G, LAM, FMT> cols;
        cols.r = r;
        cols.sl2 = scale_log2;
        float vscale = 1.f;
        if constexpr (FMT == kFmtFp8) {
            cols.sl2 *= kv_scales[g];
            vscale = kv_scales[hkv + g];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                cols.qv[h][j] = *reinterpret_cast<const uint4*>(
                    q_rot + (static_cast<size_t>(b) * hkv * G + g * G + h) * D + (c + LAM * j) * 8);
            cols.m[h] = kNegInf;
            cols.l[h] = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) cols.acc[h][j][e] = 0.f;
        }

        DotRing<D, LAM, FMT, PF> ring;
        ring.kbase = reinterpret_cast<const char*>(kc) + static_cast<size_t>(g) * TILE;
        ring.vbase = reinterpret_cast<const char*>(vc) + static_cast<size_t>(g) * TILE;
        ring.blk_stride = static_cast<size_t>(hkv) * TILE;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < NJ; ++j) ring.loff[t][j] = (t * TS::TPI + r) * TS::ROW + (c + LAM * j) * TS::PB;

        for (int s0 = t0; s0 < t1; s0 += 64) {
            const int nblk = min(64, t1 - s0);
            int32_t id = 0;
            if (lane < nblk) id = table[static_cast<size_t>(b) * mbps + s0 + lane];
            const bool bad_id = lane < nblk && (id < 0 || id >= num_blocks);
            if (__ballot(bad_id) != 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            ring.my_id = bad_id ? 0 : id;
            const int last_rows = (s0 + nblk == nt) ? L - (nt - 1) * BS : BS;
            ring.run(nblk, last_rows, cols);
        }

        // merge the TPI key-row groups (lanes c, c + LAM, ... hold the same dims)
        const bool whole = (t0 == 0 && t1 == nt);
        const size_t slot = 2 * static_cast<size_t>(w) + (first_piece ? 0 : 1);
        uint16_t* o = out + (static_cast<size_t>(b) * hkv * G + g * G) * D;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = cols.m[h];
#pragma unroll
            for (int x = LAM; x < 64; x *= 2) M = fmaxf(M, __shfl_xor(M, x));
            const float f = (cols.m[h] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(cols.m[h] - M);
            float lt = cols.l[h] * f;
#pragma unroll
            for (int x = LAM; x < 64; x *= 2) lt += __shfl_xor(lt, x);
            float red[NJ][8];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = cols.acc[h][j][e] * f;
#pragma unroll
                    for (int x = LAM; x < 64; x *= 2) a += __shfl_xor(a, x);
                    red[j][e] = a;
                }
            if (r != 0) continue;
            if (whole) {
                const float inv = vscale / lt;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    uint32_t wd[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wd[e] = static_cast<uint32_t>(f32_to_bf16_rne(red[j][2 * e] * inv)) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(red[j][2 * e + 1] * inv)) << 16);
                    *reinterpret_cast<uint4*>(o + h * D + (c + LAM * j) * 8) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
            } else {
                float* dst = part_acc + (slot * G + h) * D;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    float4* d4 = reinterpret_cast<float4*>(dst + (c + LAM * j) * 8);
                    d4[0] = make_float4(red[j][0] * vscale, red[j][1] * vscale, red[j][2] * vscale, red[j][3] * vscale);
                    d4[1] = make_float4(red[j][4] * vscale, red[j][5] * vscale, red[j][6] * vscale, red[j][7] * vscale);
                }
                if (c == 0) part_ml[slot * G + h] = make_float2(M, lt);
            }
        }
        pos += t1 - t0;
        first_piece = false;
    }
}

// Lanes per key row and prefetch depth of the dot-product kernel: the
// accumulators (G D / LAM floats per lane) and PF + 1 tiles stay in VGPRs.
template <int D, int G>
struct DotShape {
    static constexpr int LAM = (D == 128 && G > 2) ? 16 : 8;
    static constexpr int PF = (D == 128 && G > 4) ? 1 : 2;
};

// ================================================ paged prefill, rescaling form
// Causal attention of a prefill chunk (packed rows, see the prompt KV write)
// with the online rescaling softmax. One wave per (block of 16 QB new
// tokens, query head): the MFMA tile of the decode kernel with QB column
// blocks taken by the block's query tokens instead of the group's heads, so
// every K/V tile a wave loads serves 16 QB queries; the loads are ordinary
// cached loads, since the other query blocks and heads of the sequence read
// the same tiles. The wave streams its sequence's K/V tiles 0 .. last in
// logical order; tiles whose keys all lie at or before the block's first
// position are unmasked and go through the register ring, the tiles on the
// diagonal (at most QB + 1) follow with a per-column causal limit. Blocks
// are issued longest first (largest key range).
// This is the second launch of a prefill call, with the online rescaling
// softmax: it runs over every query block only if the shared-tile kernel
// (below) wrote this call's generation into the pool's redo word (a row sum
// outgrew its fixed reference), and every wave exits at once otherwise.
// Generations count the calls on a pool, so the word needs no clearing
// between calls.
template <int D, int G, int FMT, int PF, int QB>
__global__ __launch_bounds__(64, 1) void paged_prefill_rescale_kernel(
    const uint16_t* __restrict__ q_rot, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const int32_t* __restrict__ table, int32_t mbps,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu, int32_t hkv,
    int32_t num_blocks, int32_t total, int32_t max_new, float scale_log2,
    const float* __restrict__ kv_scales, uint16_t* __restrict__ out, uint32_t* __restrict__ err,
    uint32_t* __restrict__ redo_word, uint32_t gen) {
    if (__builtin_amdgcn_readfirstlane(*redo_word) != gen) return;
    using TL = MfmaTile<D, FMT>;
    constexpr int NPV = TL::NPV;
    constexpr int QT = BS * QB;                  // query tokens per wave
    constexpr size_t TILE = static_cast<size_t>(BS) * TL::ROW;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int q4 = lane >> 4;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / G;
    const int row0 = cu[b];
    const int nnew = cu[b + 1] - row0;
    const int ctx = ctx_lens[b];
    if (row0 < 0 || nnew < 0 || row0 + nnew > total || nnew > max_new || ctx < 0 ||
        ctx + nnew > mbps * BS) {
        if (blockIdx.x == 0 && h == 0 && lane == 0)
            atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        return;
    }
    const int nqb = (nnew + QT - 1) / QT;
    if (static_cast<int>(blockIdx.x) >= nqb) return;
    const int j0 = (nqb - 1 - static_cast<int>(blockIdx.x)) * QT;   // first query token
    const int p_first = ctx + j0;
    const int p_last = ctx + min(j0 + QT, nnew) - 1;
    const int nkt = p_last / BS + 1;             // tiles holding keys 0 .. p_last
    const int kt_m = (p_first + 1) / BS;         // tiles below are unmasked for every query

    int p_n[QB];
#pragma unroll
    for (int c = 0; c < QB; ++c) p_n[c] = ctx + j0 + BS * c + n;
    float sl2 = scale_log2, vscale = 1.f;
    if constexpr (FMT == kFmtFp8) {
        sl2 *= kv_scales[g];
        vscale = kv_scales[hkv + g];
    }

    // query operands and fresh softmax state of the wave's QB column blocks
    auto init_cols = [&](auto& cl) {
#pragma unroll
        for (int c = 0; c < QB; ++c) {
            const int j = j0 + BS * c + n;
            cl.col_ok[c] = j < nnew;
            const uint16_t* qh = q_rot + (static_cast<size_t>(row0 + (cl.col_ok[c] ? j : 0)) * hkv * G + h) * D;
#pragma unroll
            for (int jj = 0; jj < TL::NQK; ++jj) {
                const int d0 = FMT == kFmtBf16 ? 32 * jj + 8 * q4 : 64 * (jj / 2) + 16 * q4 + 8 * (jj & 1);
                cl.qb[c][jj] = cl.col_ok[c] ? *reinterpret_cast<const uint4*>(qh + d0) : make_uint4(0, 0, 0, 0);
            }
            cl.sm[c] = MfmaSoftmax{cl.col_ok[c] ? kNegInf : 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < NPV; ++jj) cl.o[c][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        cl.sl2 = sl2;
        cl.q4 = q4;
    };

    // every key tile of the block: [0, kt_m) unmasked through the register
    // ring, 64 per sub-chunk, then the diagonal tiles [kt_m, nkt) with a causal
    // limit per column
    auto run_pass = [&](auto& cl) {
        MfmaRing<D, FMT, PF, false> ring;
        ring.kbase = reinterpret_cast<const char*>(kc) + static_cast<size_t>(g) * TILE;
        ring.vbase = reinterpret_cast<const char*>(vc) + static_cast<size_t>(g) * TILE;
        ring.blk_stride = static_cast<size_t>(hkv) * TILE;
#pragma unroll
        for (int jj = 0; jj < TL::NKL; ++jj) ring.koff[jj] = n * TL::ROW + 64 * jj + 16 * q4;
#pragma unroll
        for (int r = 0; r < 4; ++r) ring.voff[r] = (4 * q4 + r) * TL::ROW + TL::VB * n;

        // block ids of the sub-chunk starting at tile s0 (lane i: tile s0 + i)
        auto fetch_ids = [&](int s0, int cnt) {
            int32_t id = 0;
            if (lane < cnt) id = table[static_cast<size_t>(b) * mbps + s0 + lane];
            const bool bad_id = lane < cnt && (id < 0 || id >= num_blocks);
            if (__ballot(bad_id) != 0 && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
            ring.my_id = bad_id ? 0 : id;
        };
        for (int s0 = 0; s0 < kt_m; s0 += 64) {
            const int nblk = min(64, kt_m - s0);
            fetch_ids(s0, nblk);
            ring.run(nblk, BS, cl);
        }
        fetch_ids(kt_m, nkt - kt_m);
        for (int t = 0; t < nkt - kt_m; ++t) {
            const int base = (kt_m + t) * BS;
            int qlim[QB];
#pragma unroll
            for (int c = 0; c < QB; ++c) qlim[c] = min(BS, max(0, p_n[c] + 1 - base));
            ring.template load<0>(t);
            cl.consume(ring.kr[0], ring.vr[0], qlim, min(BS, p_last + 1 - base), true);
        }
    };

    auto store = [&](auto& cl) {
#pragma unroll
        for (int c = 0; c < QB; ++c) {
            float lt = cl.sm[c].l + __shfl_xor(cl.sm[c].l, 16);
            lt += __shfl_xor(lt, 32);
            if (!cl.col_ok[c]) continue;
            const float inv = vscale / lt;
            uint16_t* oh = out + (static_cast<size_t>(row0 + j0 + BS * c + n) * hkv * G + h) * D + NPV * 4 * q4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t wd[NPV / 2];
#pragma unroll
                for (int e = 0; e < NPV / 2; ++e)
                    wd[e] = static_cast<uint32_t>(f32_to_bf16_rne(cl.o[c][2 * e][r] * inv)) |
                            (static_cast<uint32_t>(f32_to_bf16_rne(cl.o[c][2 * e + 1][r] * inv)) << 16);
                if constexpr (NPV == 8)
                    *reinterpret_cast<uint4*>(oh + NPV * r) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                else
                    *reinterpret_cast<uint2*>(oh + NPV * r) = make_uint2(wd[0], wd[1]);
            }
        }
    };

    MfmaCols<D, FMT, QB, true> cols;
    init_cols(cols);
    run_pass(cols);
    store(cols);
}

// ============================================== prefill, shared-tile form
// Causal attention of a prefill chunk with the K/V tiles shared by the query
// heads of a KV group; this register-staged form serves 8-bit caches (the
// copy widens the codes), bf16 caches take paged_prefill_dma_kernel below.
// One workgroup per (KV head g, sequence, 32-token query
// block), one wave per query head of the group (G waves); the blocks with the
// longest key ranges are dispatched first across the whole chunk
// (fa_block_of_rank). A sequence with a bad length or chunk is recorded as a
// fault by the first workgroup and gets no blocks. The key range
// 0 .. p_last of the block goes by in steps of 64 keys (four 16-token cache
// blocks): the workgroup copies a step's K and V from the paged cache into
// LDS once (double buffered, one barrier per step; the copy of step s + 1 is
// in flight while step s is computed) and every wave contracts its own
// head's 32 queries against them on 32x32x16 bf16 MFMAs:
//  - S^T = K Q^T per 32-key half t: 32 keys x 32 queries, D / 16 MFMAs (the
//    two halves are independent chains); lane l holds query l % 32 (its B
//    operand column, Q^T loaded once) and receives the scores of keys
//    32 t + 8 (i / 4) + 4 (l / 32) + i % 4, i < 16;
//  - O^T += V^T P^T: D / 32 dim tiles x 4 MFMAs of 16 keys. P^T is the score
//    layout itself (registers 8 (a % 2) .. + 7 of half a / 2 are the B
//    operand of key group a), so V is stored transposed in LDS with the keys
//    of each group in the matching order: key 16a + r sits at column 16a +
//    8 ((r / 4) % 2) + (r % 4) + 4 (r / 8), and the A operand of a lane is one
//    16-byte read.
// Rows of K and of V^T are padded (16 bytes) so the 16 lanes a 16-byte
// operand read serves per cycle fall on distinct banks. The softmax uses a fixed
// reference (the largest score of the first step, never raised) and the row
// sum adds the weights as rounded for the MFMA. A query whose row sum ends
// above kFixedHeadroomSum (which any single weight above that bound forces)
// makes the wave write the call's generation into the redo word, and the
// rescaling launch repeats the chunk. Keys after the block's last position
// are not used (zero rows, so NaN bits in the cache tail never reach an
// MFMA); keys after a query's own position are masked by selection on the
// diagonal steps.
constexpr int kFaRows = 32;         // query tokens per wave (one MFMA tile)
constexpr int kFaKeys = 64;         // keys per step

// Buffer-resource loads of one cache block: the block's base and size sit in
// scalar registers, the lane's byte offset in the block is fixed for the whole
// kernel, so a load carries no per-lane address arithmetic.
typedef unsigned int fa_u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kFaBufferDword3 = 0x00020000;    // raw 32-bit buffer access (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fa_rsrc(const uint8_t* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), kFaBufferDword3);
}
template <typename Piece>
__device__ __forceinline__ Piece fa_bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    if constexpr (sizeof(Piece) == 16) {
        const fa_u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        return Piece{t.x, t.y, t.z, t.w};
    } else {
        const fa_u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        return Piece{t.x, t.y};
    }
}

template <int D>
struct FaLayout {
    static constexpr int KROW = D * 2 + 16;             // bytes per K row
    static constexpr int VROW = kFaKeys * 2 + 16;       // bytes per V^T row
    static constexpr int KBYTES = kFaKeys * KROW;
    static constexpr int BUF = KBYTES + D * VROW;        // one stage: K, then V^T
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Column of key r (0 .. kFaKeys - 1) of a step in the V^T rows.
__device__ __forceinline__ int fa_vcol(int r) {
    const int q = r & 15;
    return (r & ~15) + 8 * ((q >> 2) & 1) + (q & 3) + 4 * (q >> 3);
}

// Longest-first order of the query blocks (ROWS tokens) of a chunk. Block y
// of sequence b (y = 0 holds the chunk's last tokens) is ranked by
// A_b - ROWS y, with A_b = ctx_b + ROWS nqb_b (its key count, rounded up to the block grid
// for y = 0), descending, ties in sequence order. The block of rank r is found
// without a sort: the largest key count T with more than r blocks at or above
// it, then the (r - count above T)-th sequence, in order, that has a block
// exactly at T. The search for T is 64-way: each lane counts the blocks at or
// above its own candidate, over all sequences (lane b holds sequence b's A_b
// and nqb_b), and the range shrinks 64 times per round.
// Wave-uniform; every lane returns the same (b, y), or b = -1 past the last
// block. When every sequence has the same key count, and beyond kFaRankBatch
// sequences (where the search would cost more than it saves), the order is
// plain block-index major instead, which for one key count is the same order.
// Sequences with a bad length (recorded by the kernel) have no blocks.
struct FaBlock {
    int b, y;
};
constexpr int kFaRankBatch = 64;
template <int ROWS>
__device__ __forceinline__ FaBlock fa_block_of_rank(int r, const int32_t* __restrict__ ctx_lens,
                                                    const int32_t* __restrict__ cu, int batch, int total,
                                                    int max_new, int mbps, int lane) {
    auto seq = [&](int bb, int& A, int& nq) {       // A_b and nqb_b of sequence bb (0 blocks if bad)
        A = 0;
        nq = 0;
        if (bb < batch) {
            const int row0 = cu[bb], n = cu[bb + 1] - row0, c = ctx_lens[bb];
            if (!(row0 < 0 || n < 0 || row0 + n > total || n > max_new || c < 0 || c + n > mbps * BS)) {
                nq = (n + ROWS - 1) / ROWS;
                A = c + ROWS * nq;
            }
        }
    };
    auto plain = [&]() {                            // block index major
        const int y = r / batch, bb = r % batch;
        int A, nq;
        seq(bb, A, nq);
        return FaBlock{y < nq ? bb : -1, y};
    };
    if (batch > kFaRankBatch) return plain();
    int A, nq;
    seq(lane, A, nq);
    int amax = 0, amin = INT_MAX, tmin = INT_MAX;   // tmin: key count of the shortest last block
    for (int bb = 0; bb < batch; ++bb) {            // scalar: lane bb's values are uniform
        const int Ab = __builtin_amdgcn_readlane(A, bb), nb = __builtin_amdgcn_readlane(nq, bb);
        if (nb > 0) {
            amax = max(amax, Ab);
            amin = min(amin, Ab);
            tmin = min(tmin, Ab - ROWS * (nb - 1));
        }
    }
    if (amax == amin) return plain();               // one key count: the plain order is longest-first
    if (amax <= 0) return FaBlock{-1, 0};
    auto count_from = [&](int T) {                  // blocks with key count >= T (T per lane)
        int c = 0;
        for (int bb = 0; bb < batch; ++bb) {
            const int Ab = __builtin_amdgcn_readlane(A, bb), nb = __builtin_amdgcn_readlane(nq, bb);
            if (nb > 0 && Ab >= T) c += min(nb, (Ab - T) / ROWS + 1);
        }
        return c;
    };
    // count(tmin) is every block; the largest T with count(T) > r is in [tmin, amax]
    int lo = tmin, hi = amax;
    if (__builtin_amdgcn_readfirstlane(count_from(tmin)) <= r) return FaBlock{-1, 0};
    while (lo < hi) {
        const int step = (hi - lo + 64) / 64;       // ceil((hi - lo + 1) / 64)
        const int t = min(lo + lane * step, hi);
        const uint64_t good = __ballot(count_from(t) > r);   // a prefix of the lanes, lane 0 in it
        const int L = __popcll(good) - 1;
        const int nlo = min(lo + L * step, hi);
        hi = min(hi, nlo + step - 1);
        lo = nlo;
    }
    const int T = lo;
    // blocks above T, then the sequences with a block exactly at T, in order
    int above = (nq > 0 && A >= T + 1) ? min(nq, (A - T - 1) / ROWS + 1) : 0;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) above += __shfl_xor(above, x);
    const int rr = r - above;
    const bool at = nq > 0 && A >= T && (A - T) % ROWS == 0 && (A - T) / ROWS < nq;
    uint64_t mm = __ballot(at);
    if (rr < 0 || rr >= __popcll(mm)) return FaBlock{-1, 0};
    for (int i = 0; i < rr; ++i) mm &= mm - 1;
    const int src = __ffsll(static_cast<unsigned long long>(mm)) - 1;
    return FaBlock{src, (__shfl(A, src) - T) / ROWS};
}

template <int D, int G, int FMT>
__global__ __launch_bounds__(64 * G, 2) void paged_prefill_fa_kernel(
    const uint16_t* __restrict__ q_rot, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const int32_t* __restrict__ table, int32_t mbps,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu, int32_t batch, int32_t hkv,
    int32_t num_blocks, int32_t total, int32_t max_new, float scale_log2,
    const float* __restrict__ kv_scales, uint16_t* __restrict__ out, uint32_t* __restrict__ err,
    uint32_t* __restrict__ redo_word, uint32_t gen) {
    using L = FaLayout<D>;
    constexpr int ROWS = kFaRows;           // query tokens per workgroup (per wave and head)
    constexpr int NT = 64 * G;              // threads
    constexpr int ESZ = FMT == kFmtBf16 ? 2 : 1;
    constexpr int CPR = D / 8;              // 8-element pieces per key row
    constexpr int KITEMS = kFaKeys * CPR;   // K pieces per step
    constexpr int KPER = (KITEMS + NT - 1) / NT;
    constexpr int NKK = D / 16;             // score MFMAs per 32-key half
    constexpr int NDT = D / 32;             // output dim tiles
    constexpr int NH = kFaKeys / 32;        // 32-key halves per step
    constexpr int BPS = kFaKeys / BS;       // cache blocks per step
    constexpr int UPB = CPR / 8;            // V units (64 lanes: 8 key pairs x 8 pieces) per cache block
    constexpr int VUNITS = BPS * UPB;       // V units per step
    constexpr int VPER = (VUNITS + G - 1) / G;
    __shared__ __align__(16) char lds[2 * L::BUF];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31;
    const int half = lane >> 5;
    // grid: KV heads x (batch x query blocks of the longest chunk); the
    // workgroups of rank r (dispatched in order) take the r-th longest block
    const int g = static_cast<int>(blockIdx.x) % hkv;
    if (blockIdx.x == 0 && tid == 0) {
        for (int bb = 0; bb < batch; ++bb) {
            const int r0 = cu[bb], n = cu[bb + 1] - r0, c = ctx_lens[bb];
            if (r0 < 0 || n < 0 || r0 + n > total || n > max_new || c < 0 || c + n > mbps * BS)
                atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        }
    }
    const FaBlock fb = fa_block_of_rank<ROWS>(static_cast<int>(blockIdx.x) / hkv, ctx_lens, cu, batch,
                                              total, max_new, mbps, lane);
    if (fb.b < 0) return;
    const int b = __builtin_amdgcn_readfirstlane(fb.b);
    const int qblk = __builtin_amdgcn_readfirstlane(fb.y);
    const int h = g * G + w;
    const int hq = hkv * G;
    const int row0 = cu[b];
    const int nnew = cu[b + 1] - row0;
    const int ctx = ctx_lens[b];
    const int nqb = (nnew + ROWS - 1) / ROWS;
    const int j0 = (nqb - 1 - qblk) * ROWS;     // longest blocks first
    const int p_first = ctx + j0;
    const int p_last = ctx + min(j0 + ROWS, nnew) - 1;
    const int nks = p_last / kFaKeys + 1;       // steps holding keys 0 .. p_last
    const int ks_m = (p_first + 1) / kFaKeys;   // steps before this are unmasked for every query
    const int jq = j0 + col;                    // this lane's query token
    const bool q_ok = jq < nnew;
    const int pq = ctx + jq;

    float sl2 = scale_log2, vscale = 1.f;
    if constexpr (FMT == kFmtFp8) {
        sl2 *= kv_scales[g];
        vscale = kv_scales[hkv + g];
    }

    // Q^T operand of the score MFMAs: dims 16 kk + 8 half .. + 8 of the query
    uint4 qop[NKK];
    {
        const uint16_t* qh = q_rot + (static_cast<size_t>(row0 + (q_ok ? jq : 0)) * hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qop[kk] = q_ok ? *reinterpret_cast<const uint4*>(qh + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0);
    }

    // Copy of one step (keys 64 s .. 64 s + 63) through registers into LDS.
    // Each load of a wave reads one cache block: K as rows of 8-element
    // pieces (item it = tid + u NT is row it / CPR, piece it % CPR), V in
    // units of 8 key pairs x 8 pieces (unit c = w + G u: block c / UPB,
    // pieces 8 (c % UPB) .. + 7; lane: pair lane & 7, piece + lane >> 3) for
    // the transposed store. Blocks past the chunk's last key are clamped to
    // its block; rows past p_last are read (they lie in an allocated block)
    // and zeroed when stored. The block ids of the next fetch are read one
    // step ahead (scalar loads, range-checked: a bad id is recorded and
    // replaced by 0).
    typedef typename std::conditional<FMT == kFmtBf16, uint4, uint2>::type Piece;
    struct Stage {
        Piece k[KPER];
        Piece v[VPER][2];
    };
    const uint32_t blk_bytes = static_cast<uint32_t>(hkv) * BS * D * ESZ;
    const uint32_t head_off = static_cast<uint32_t>(g) * BS * D * ESZ;
    const int last_blk = p_last / BS;
    const int32_t* trow = table + static_cast<size_t>(b) * mbps;
    int jbk[KPER], jbv[VPER];                   // block of the step read by load u (wave-uniform)
    uint32_t koff[KPER], voff[VPER];            // the lane's byte offset in that block
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
        const int it0 = min(w * 64 + u * NT, KITEMS - 64);     // the wave's first item
        const int it = it0 + lane;
        jbk[u] = (it0 / CPR) / BS;
        koff[u] = head_off + static_cast<uint32_t>(((it / CPR) % BS) * D + 8 * (it % CPR)) * ESZ;
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int c = min(w + G * u, VUNITS - 1);
        jbv[u] = c / UPB;
        voff[u] = head_off + static_cast<uint32_t>((2 * (lane & 7)) * D + 8 * (8 * (c % UPB) + (lane >> 3))) * ESZ;
    }
    bool bad_id = false;                        // wave-uniform; recorded once after the loop
    int32_t kid[KPER], vid[VPER];
    auto load_ids = [&](int s) {               // all scalar loads first, then the checks
        int32_t rk[KPER], rv[VPER];
#pragma unroll
        for (int u = 0; u < KPER; ++u) rk[u] = trow[min(BPS * s + jbk[u], last_blk)];
#pragma unroll
        for (int u = 0; u < VPER; ++u) rv[u] = trow[min(BPS * s + jbv[u], last_blk)];
        auto check = [&](int32_t id) {
            const bool ok = id >= 0 && id < num_blocks;
            bad_id |= !ok;
            return __builtin_amdgcn_readfirstlane(ok ? id : 0);
        };
#pragma unroll
        for (int u = 0; u < KPER; ++u) kid[u] = check(rk[u]);
#pragma unroll
        for (int u = 0; u < VPER; ++u) vid[u] = check(rv[u]);
    };
    auto fetch = [&](Stage& st) {
#pragma unroll
        for (int u = 0; u < KPER; ++u)
            st.k[u] = fa_bload<Piece>(fa_rsrc(kc + static_cast<size_t>(kid[u]) * blk_bytes, blk_bytes), koff[u]);
#pragma unroll
        for (int u = 0; u < VPER; ++u) {
            const __amdgpu_buffer_rsrc_t r = fa_rsrc(vc + static_cast<size_t>(vid[u]) * blk_bytes, blk_bytes);
            st.v[u][0] = fa_bload<Piece>(r, voff[u]);
            st.v[u][1] = fa_bload<Piece>(r, voff[u] + D * ESZ);
        }
    };
    auto widen = [&](const Piece& x) -> uint4 {       // 8 elements as bf16 (E4M3 codes widened exactly)
        if constexpr (FMT == kFmtBf16) {
            return x;
        } else {
            return make_uint4(fp8x2_to_bf16x2<false>(x.x), fp8x2_to_bf16x2<true>(x.x),
                              fp8x2_to_bf16x2<false>(x.y), fp8x2_to_bf16x2<true>(x.y));
        }
    };
    // LDS destinations (within a stage) of the lane's K pieces and V pairs
    uint32_t kdst[KPER], vdst[VPER];
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
        const int it = tid + u * NT;
        kdst[u] = static_cast<uint32_t>((it / CPR) * L::KROW + (it % CPR) * 16);
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int c = min(w + G * u, VUNITS - 1);
        const int r = BS * (c / UPB) + 2 * (lane & 7);
        const int piece = 8 * (c % UPB) + (lane >> 3);
        vdst[u] = static_cast<uint32_t>(L::KBYTES + (8 * piece) * L::VROW + fa_vcol(r) * 2);
    }
    auto stash_rows = [&](int s, const Stage& st, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        char* buf = lds + (s & 1) * L::BUF;
        const int rows = p_last + 1 - kFaKeys * s;     // valid key rows of the step (1 .. 64)
#pragma unroll
        for (int u = 0; u < KPER; ++u) {
            const int it = tid + u * NT;
            if (KITEMS % NT == 0 || it < KITEMS) {
                uint4 x = widen(st.k[u]);
                if (TAIL && (it / CPR) >= rows) x = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(buf + kdst[u]) = x;
            }
        }
#pragma unroll
        for (int u = 0; u < VPER; ++u) {
            if (VUNITS % G == 0 || w + G * u < VUNITS) {
                const int r = BS * ((w + G * u) / UPB) + 2 * (lane & 7);
                uint4 a = widen(st.v[u][0]), c = widen(st.v[u][1]);
                if (TAIL && r >= rows) a = make_uint4(0, 0, 0, 0);
                if (TAIL && r + 1 >= rows) c = make_uint4(0, 0, 0, 0);
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
                char* dst = buf + vdst[u];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    *reinterpret_cast<uint32_t*>(dst + e * L::VROW) =
                        __builtin_amdgcn_perm(cw[e / 2], aw[e / 2], sel);
                }
            }
        }
    };
    auto stash = [&](int s, const Stage& st) {
        if (p_last + 1 - kFaKeys * s >= kFaKeys) stash_rows(s, st, std::false_type{});
        else stash_rows(s, st, std::true_type{});
    };

    f32x16_t oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
    float m = kNegInf, l = 0.f;

    // One step: scores, softmax, weighted V sum from LDS buffer s % 2.
    auto compute = [&](int s) {
        const char* kb = lds + (s & 1) * L::BUF;
        const char* vb = kb + L::KBYTES;
        f32x16_t sacc[NH];
#pragma unroll
        for (int t = 0; t < NH; ++t) sacc[t] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                const uint4 a = *reinterpret_cast<const uint4*>(kb + (32 * t + col) * L::KROW + (16 * kk + 8 * half) * 2);
                sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, qop[kk]), sacc[t], 0, 0, 0);
            }
        float sc[NH][16];
        if (s >= ks_m) {            // diagonal step: key position <= the query's own
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kp = kFaKeys * s + 32 * t + 8 * (i / 4) + 4 * half + (i % 4);
                    sc[t][i] = kp <= pq ? sacc[t][i] : kNegInf;
                }
        } else {
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[t][i] = sacc[t][i];
        }
        if (s == 0) {               // the fixed reference: largest score of the first step
            float mx = sc[0][0];
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[t][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
            m = q_ok ? mx : 0.f;
        }
        // the row sum adds the weights as they enter the MFMA (bf16), so
        // numerator and denominator use the same rounded weights
        bf16x8_t pb[2 * NH];
#pragma unroll
        for (int t = 0; t < NH; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pb[2 * t + i / 8][i % 8] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[t][i], sl2, -m)));
        const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
        for (int a = 0; a < 2 * NH; ++a) {
            const bf16x8_t x = pb[a];
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones, l, false);
        }
#pragma unroll
        for (int a = 0; a < 2 * NH; ++a)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const uint4 v = *reinterpret_cast<const uint4*>(vb + (32 * dt + col) * L::VROW + (16 * a + 8 * half) * 2);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v), pb[a],
                                                                   oacc[dt], 0, 0, 0);
            }
    };

    // Step s + 1 is fetched into registers while step s is computed from
    // LDS, then stored to the other LDS buffer; one barrier per step. The
    // fetch is issued unconditionally (past the last step it reads the last
    // step again and is dropped), so every path keeps the same loads in
    // flight. The ids of step s + 2 are read while step s is computed.
    Stage st;
    load_ids(0);
    fetch(st);
    load_ids(min(1, nks - 1));
    stash(0, st);
    __syncthreads();
    for (int s = 0; s < nks; ++s) {
        fetch(st);                              // step s + 1 (the last step again past the end)
        load_ids(min(s + 2, nks - 1));
        compute(s);
        if (s + 1 < nks) stash(s + 1, st);
        __syncthreads();
    }
    if (bad_id && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));

    const float lt = l + __shfl_xor(l, 32);
    if (q_ok) {
        const float inv = vscale / lt;
        uint16_t* oh = out + (static_cast<size_t>(row0 + jq) * hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * dt + 8 * r4 + 4 * half;
                const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4] * inv)) |
                                    (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 1] * inv)) << 16);
                const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 2] * inv)) |
                                    (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 3] * inv)) << 16);
                *reinterpret_cast<uint2*>(oh + d0) = make_uint2(w0, w1);
            }
    }
    if (__ballot(q_ok && !(lt <= kFixedHeadroomSum)) != 0 && lane == 0) atomicExch(redo_word, gen);
}

// ===================================== prefill, shared-tile form, bf16 DMA
// The shared-tile kernel above for bf16 caches with the K/V copy done by
// gfx950's direct global-to-LDS loads (`buffer_load_dwordx4 ... lds`): no
// staging registers, no LDS stores, no permutes. A wave load writes 1 KB of
// LDS (lane i's 16 bytes at 16 i), i.e. 1024 / (2 D) consecutive key rows of
// one cache block; which 16-byte piece each lane fetches realises an XOR
// swizzle of the rows' 16-byte chunks, so that the operand reads below are
// bank-conflict free on gfx950's LDS (64 banks of 4 bytes: a 16-byte read
// serves 16 lanes a cycle, an 8-byte read 32). With s = row / (256 / 2 D)
// (the row's 256-byte bank line): K chunk ^ (s mod 2 D / 16), so that 16
// consecutive key rows at one chunk fill all banks; V chunk ^ 4 (s mod
// D / 32), so that the 4 rows x 4 chunks a transposing read touches in 32
// lanes do.
// V stays in key-major rows; the V^T operand of the weighted sum is read
// with `ds_read_b64_tr_b16`, which within a group of 16 lanes hands lane l
// element l & 3 of the 4 bf16 addressed by lane (l >> 2) + 4 e, as its
// element e: lane j of group q (of 4) addresses key 16 a + 8 c + 4 (q >> 1)
// + (j >> 2), dims 32 dt + 16 (q & 1) + 4 (j & 3), for call c = 0, 1, which
// yields the 8 keys of the MFMA's k-order (the score layout's key order,
// see fa_vcol) at dim 32 dt + l % 32. The two stages are two LDS arrays and
// the step loop is unrolled by two, so a stage's loads and the other
// stage's reads are known apart. V rows past the chunk's last key are
// zeroed in LDS once the last step's loads are in (NaN bits in the cache
// tail must not reach an MFMA); K rows there are masked by selection.
// Steps are 32 keys (two cache blocks): the kernel then fits in 168
// registers and 32 KB of LDS, three waves per SIMD (64-key steps took 215
// registers: two).
constexpr int kFaDmaKeys = 32;
typedef short s16x8_t __attribute__((ext_vector_type(8)));
// 16 bytes per lane from a buffer into LDS at dst + 16 lane (dst wave-uniform).
__device__ __forceinline__ void fa_load_lds16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}
// Transposing LDS read of 4 bf16 (see the kernel comment).
__device__ __forceinline__ s16x4_t fa_read_tr16(const char* p) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <int D, int G>
__global__ __launch_bounds__(64 * G, 3) void paged_prefill_dma_kernel(
    const uint16_t* __restrict__ q_rot, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, const int32_t* __restrict__ table, int32_t mbps,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu, int32_t batch, int32_t hkv,
    int32_t num_blocks, int32_t total, int32_t max_new, float scale_log2, uint16_t* __restrict__ out,
    uint32_t* __restrict__ err, uint32_t* __restrict__ redo_word, uint32_t gen) {
    constexpr int ROWS = kFaRows;           // query tokens per workgroup (per wave and head)
    constexpr int KEYS = kFaDmaKeys;        // keys per step
    constexpr int NT = 64 * G;              // threads
    constexpr int ROWB = D * 2;             // bytes per K or V row in LDS
    constexpr int CPR16 = ROWB / 16;        // 16-byte chunks per row
    constexpr int RPL = 1024 / ROWB;        // rows per wave load
    constexpr int LPS = KEYS / RPL;      // wave loads per step (K; V alike)
    constexpr int LPW = (LPS + G - 1) / G;  // per wave
    constexpr int KB = KEYS * ROWB;      // bytes of K (and of V) per stage
    constexpr int NKK = D / 16;             // score MFMAs per 32-key half
    constexpr int NDT = D / 32;             // output dim tiles
    constexpr int NH = KEYS / 32;        // 32-key halves per step
    constexpr int BPS = KEYS / BS;       // cache blocks per step
    constexpr int RPB = 256 / ROWB;         // rows per 256-byte bank line
    static_assert(BS % RPL == 0, "a wave load stays in one cache block");
    static_assert(RPB >= 1 && CPR16 >= 4, "row of 64 to 256 bytes");
    auto swz_k = [](int r) { return (r / RPB) & (CPR16 - 1); };
    auto swz_v = [](int r) { return 4 * ((r / RPB) & (CPR16 / 4 - 1)); };
    __shared__ __align__(1024) char stage0[2 * KB];
    __shared__ __align__(1024) char stage1[2 * KB];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int g = static_cast<int>(blockIdx.x) % hkv;
    if (blockIdx.x == 0 && tid == 0) {
        for (int bb = 0; bb < batch; ++bb) {
            const int r0 = cu[bb], n = cu[bb + 1] - r0, c = ctx_lens[bb];
            if (r0 < 0 || n < 0 || r0 + n > total || n > max_new || c < 0 || c + n > mbps * BS)
                atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        }
    }
    const FaBlock fb = fa_block_of_rank<ROWS>(static_cast<int>(blockIdx.x) / hkv, ctx_lens, cu, batch,
                                              total, max_new, mbps, lane);
    if (fb.b < 0) return;
    const int b = __builtin_amdgcn_readfirstlane(fb.b);
    const int qblk = __builtin_amdgcn_readfirstlane(fb.y);
    const int h = g * G + w;
    const int hq = hkv * G;
    const int row0 = cu[b];
    const int nnew = cu[b + 1] - row0;
    const int ctx = ctx_lens[b];
    const int nqb = (nnew + ROWS - 1) / ROWS;
    const int j0 = (nqb - 1 - qblk) * ROWS;     // longest blocks first
    const int p_first = ctx + j0;
    const int p_last = ctx + min(j0 + ROWS, nnew) - 1;
    const int nks = p_last / KEYS + 1;       // steps holding keys 0 .. p_last
    const int ks_m = (p_first + 1) / KEYS;   // steps before this are unmasked for every query
    const int jq = j0 + col;                    // this lane's query token
    const bool q_ok = jq < nnew;
    const int pq = ctx + jq;
    const float sl2 = scale_log2;

    uint4 qop[NKK];
    {
        const uint16_t* qh = q_rot + (static_cast<size_t>(row0 + (q_ok ? jq : 0)) * hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qop[kk] = q_ok ? *reinterpret_cast<const uint4*>(qh + 16 * kk + 8 * half) : make_uint4(0, 0, 0, 0);
    }

    // Wave load u of a step is load li = w + G u (if li < LPS): key rows
    // RPL li .. + RPL - 1, in cache block (RPL li) / BS of the step.
    const uint32_t blk_bytes = static_cast<uint32_t>(hkv) * BS * ROWB;
    const uint32_t head_off = static_cast<uint32_t>(g) * BS * ROWB;
    const int last_blk = p_last / BS;
    const int32_t* trow = table + static_cast<size_t>(b) * mbps;
    int jb[LPW];
    uint32_t koff[LPW], voff[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int li = min(w + G * u, LPS - 1);
        const int r = RPL * li + lane / CPR16;              // the lane's row in the step
        const int cp = lane % CPR16;                        // its chunk position in LDS
        jb[u] = (RPL * li) / BS;
        koff[u] = head_off + static_cast<uint32_t>((r % BS) * ROWB + (cp ^ swz_k(r)) * 16);
        voff[u] = head_off + static_cast<uint32_t>((r % BS) * ROWB + (cp ^ swz_v(r)) * 16);
    }
    bool bad_id = false;
    int32_t ids[LPW];
    auto load_ids = [&](int s) {
        int32_t raw[LPW];
#pragma unroll
        for (int u = 0; u < LPW; ++u) raw[u] = trow[min(BPS * s + jb[u], last_blk)];
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const bool ok = raw[u] >= 0 && raw[u] < num_blocks;
            bad_id |= !ok;
            ids[u] = __builtin_amdgcn_readfirstlane(ok ? raw[u] : 0);
        }
    };
    auto dma = [&](char* buf) {
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            const int li = w + G * u;
            if (LPS % G == 0 || li < LPS) {
                const size_t base = static_cast<size_t>(ids[u]) * blk_bytes;
                fa_load_lds16(fa_rsrc(kc + base, blk_bytes), buf + 1024 * li, koff[u]);
                fa_load_lds16(fa_rsrc(vc + base, blk_bytes), buf + KB + 1024 * li, voff[u]);
            }
        }
    };
    const int rows_last = p_last + 1 - KEYS * (nks - 1);   // valid key rows of the last step
    auto zero_v_tail = [&](char* buf) {
        for (int i = rows_last * CPR16 + tid; i < KEYS * CPR16; i += NT)
            *reinterpret_cast<uint4*>(buf + KB + 16 * i) = make_uint4(0, 0, 0, 0);
    };

    f32x16_t oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
    float m = kNegInf, l = 0.f;
    // Per-lane parts of the operand addresses that the swizzle makes
    // non-additive; the rest (32-key halves, key groups, calls) are
    // immediate offsets. K: row 32 t + col, whose swizzle is col's. V^T: key
    // 16 a + 8 c + 4 (q >> 1) + (j >> 2), whose swizzle is that of j >> 2
    // (it depends on the key mod 4 only), 16-byte chunk
    // 4 dt + 2 (q & 1) + (j & 3) / 2, then 8 (j & 1) bytes in.
    const int gq = lane >> 4, jl = lane & 15;
    uint32_t koffs[NKK], voffs[NDT];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        koffs[kk] = static_cast<uint32_t>(col * ROWB + (((2 * kk + half) ^ swz_k(col)) * 16));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        voffs[dt] = static_cast<uint32_t>((4 * (gq >> 1) + (jl >> 2)) * ROWB +
                                          (((4 * dt + 2 * (gq & 1) + ((jl & 3) >> 1)) ^ swz_v(jl >> 2)) * 16) +
                                          8 * (jl & 1));

    auto compute = [&](int s, const char* buf) {
        const char* kb = buf;
        const char* vb = buf + KB;
        f32x16_t sacc[NH];
#pragma unroll
        for (int t = 0; t < NH; ++t) sacc[t] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                const uint4 a = *reinterpret_cast<const uint4*>(kb + koffs[kk] + 32 * t * ROWB);
                sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, qop[kk]), sacc[t], 0, 0, 0);
            }
        float sc[NH][16];
        if (s >= ks_m) {            // diagonal step: key position <= the query's own
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kp = KEYS * s + 32 * t + 8 * (i / 4) + 4 * half + (i % 4);
                    sc[t][i] = kp <= pq ? sacc[t][i] : kNegInf;
                }
        } else {
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[t][i] = sacc[t][i];
        }
        if (s == 0) {               // the fixed reference: largest score of the first step
            float mx = sc[0][0];
#pragma unroll
            for (int t = 0; t < NH; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[t][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
            m = q_ok ? mx : 0.f;
        }
        bf16x8_t pb[2 * NH];
#pragma unroll
        for (int t = 0; t < NH; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pb[2 * t + i / 8][i % 8] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[t][i], sl2, -m)));
        const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
        for (int a = 0; a < 2 * NH; ++a) {
            const bf16x8_t x = pb[a];
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones, l, false);
        }
#pragma unroll
        for (int a = 0; a < 2 * NH; ++a)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const char* vp = vb + voffs[dt] + 16 * a * ROWB;
                const s16x4_t v0 = fa_read_tr16(vp);
                const s16x4_t v1 = fa_read_tr16(vp + 8 * ROWB);
                const s16x8_t v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v), pb[a],
                                                                   oacc[dt], 0, 0, 0);
            }
    };

    // Step s reads one stage while step s + 1 is loaded into the other; one
    // barrier per step (after the stage's own loads are in), one more on the
    // step before the last when its V tail needs zeroing.
    auto step = [&](int s, const char* cur, char* nxt) {
        if (s + 1 < nks) dma(nxt);
        load_ids(min(s + 2, nks - 1));
        compute(s, cur);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (s + 1 == nks - 1 && rows_last < KEYS) {
            zero_v_tail(nxt);
            __syncthreads();
        }
    };
    load_ids(0);
    dma(stage0);
    load_ids(min(1, nks - 1));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nks == 1 && rows_last < KEYS) {
        zero_v_tail(stage0);
        __syncthreads();
    }
    for (int s = 0; s < nks; s += 2) {
        step(s, stage0, stage1);
        if (s + 1 < nks) step(s + 1, stage1, stage0);
    }
    if (bad_id && lane == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));

    const float lt = l + __shfl_xor(l, 32);
    if (q_ok) {
        const float inv = 1.f / lt;
        uint16_t* oh = out + (static_cast<size_t>(row0 + jq) * hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * dt + 8 * r4 + 4 * half;
                const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4] * inv)) |
                                    (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 1] * inv)) << 16);
                const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 2] * inv)) |
                                    (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * r4 + 3] * inv)) << 16);
                *reinterpret_cast<uint2*>(oh + d0) = make_uint2(w0, w1);
            }
    }
    if (__ballot(q_ok && !(lt <= kFixedHeadroomSum)) != 0 && lane == 0) atomicExch(redo_word, gen);
}

// Combine kernel: one workgroup per (query head, sequence). It rebuilds the
// same partition, and if the segment was cut into pieces, merges their
// partials in range order. Thread (d, cg) folds the pieces cg, cg + NCG, ...
// of head dim d into a running (max, sum, weighted acc) with 2^(m - max)
// rescaling; the NCG groups are then merged in order. One memory round trip
// for the partition, one per four pieces; a single rounding to bf16.
// Sequences with an out-of-range length (no tiles) get NaN outputs.
// F32OUT (the decoder layer): the merged output is stored in float32 to
// out_f32 instead of bf16.
template <int D, int G, bool F32OUT = false>
__global__ __launch_bounds__(256) void paged_attn_combine_kernel(
    const float* __restrict__ part_acc, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ ctx_lens, int32_t batch, int32_t mbps, int32_t hkv,
    int32_t max_ctx, int32_t grid_waves, int32_t min_tiles, uint16_t* __restrict__ out,
    float* __restrict__ out_f32) {
    constexpr int NCG = 256 / D;        // piece groups
    __shared__ int TP[kMaxBatch + 1];
    __shared__ float sm[NCG][D], sl[NCG][D], sa[NCG][D];
    const int hq_idx = blockIdx.x;      // query head
    const int b = blockIdx.y;
    const int g = hq_idx / G;
    const int h = hq_idx - g * G;
    const int t = threadIdx.x;
    const size_t orow = (static_cast<size_t>(b) * hkv * G + hq_idx) * D;
    uint16_t* o = F32OUT ? nullptr : out + orow;

    if (t < 64) {
        bool bad;
        build_tile_prefix(ctx_lens, batch, mbps, max_ctx, hkv, TP, &bad, t);
    }
    __syncthreads();
    const int T = TP[batch];
    const int nt = (TP[b + 1] - TP[b]) / hkv;
    if (nt == 0) {                                  // length out of range
        if (t < D) {
            if constexpr (F32OUT) out_f32[orow + t] = __builtin_nanf("");
            else o[t] = 0x7fc0;
        }
        return;
    }
    const int W = active_waves(T, grid_waves, min_tiles);
    const int A = TP[b] + g * nt;                  // first tile of the segment
    const int w_first = wave_of_tile(A, T, W);
    const int w_last = wave_of_tile(A + nt - 1, T, W);
    if (w_first == w_last) return;                 // finished by one wave
    const int npieces = w_last - w_first + 1;
    const int first_slot = 2 * w_first + (range_start(w_first, T, W) < A ? 1 : 0);
    // piece k lives in slot first_slot for k = 0, else 2 (w_first + k)

    const int d = t % D;
    const int cg = t / D;
    float m = kNegInf, l = 0.f, a = 0.f;
    for (int k0 = cg; k0 < npieces; k0 += 4 * NCG) {
        float2 ml[4];
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = k0 + u * NCG;
            ml[u] = make_float2(kNegInf, 0.f);
            v[u] = 0.f;
            if (k < npieces) {
                const size_t sl_idx = static_cast<size_t>(k == 0 ? first_slot : 2 * (w_first + k));
                ml[u] = part_ml[sl_idx * G + h];
                v[u] = part_acc[(sl_idx * G + h) * D + d];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (k0 + u * NCG >= npieces) break;
            const float mn = fmaxf(m, ml[u].x);
            const float fo = __builtin_amdgcn_exp2f(m - mn);     // 0 while m = -inf
            const float fn = __builtin_amdgcn_exp2f(ml[u].x - mn);
            l = l * fo + ml[u].y * fn;
            a = a * fo + v[u] * fn;
            m = mn;
        }
    }
    sm[cg][d] = m;
    sl[cg][d] = l;
    sa[cg][d] = a;
    __syncthreads();
    if (t < D) {
        float M = sm[0][t];
#pragma unroll
        for (int c2 = 1; c2 < NCG; ++c2) M = fmaxf(M, sm[c2][t]);
        float lt = 0.f, at = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < NCG; ++c2) {
            const float f = (sm[c2][t] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sm[c2][t] - M);
            lt = fmaf(sl[c2][t], f, lt);
            at = fmaf(sa[c2][t], f, at);
        }
        if constexpr (F32OUT) out_f32[orow + t] = at / lt;
        else o[t] = f32_to_bf16_rne(at / lt);
    }
}

// ===================================================================== gather
// Bit copies of the pool's rows (ESZ bytes per element) in logical order.
template <int D, int ESZ>
__global__ __launch_bounds__(256) void gather_kv_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ table, int32_t mbps, const int32_t* __restrict__ ctx_lens,
    int32_t hkv, int32_t num_blocks, int32_t len_extra, int32_t l_max,
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out, uint32_t* __restrict__ err) {
    const int lb = blockIdx.x;       // logical block
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int n = ctx_lens[b] + len_extra;
    if (n < 0 || n > l_max || (n + BS - 1) / BS > mbps) {
        if (lb == 0 && g == 0 && threadIdx.x == 0)
            atomicOr(err, static_cast<uint32_t>(MI_FAULT_CONTEXT_LEN));
        return;
    }
    if (lb * BS >= n) return;
    const int32_t blk = table[static_cast<size_t>(b) * mbps + lb];
    if (blk < 0 || blk >= num_blocks) {
        if (threadIdx.x == 0) atomicOr(err, static_cast<uint32_t>(MI_FAULT_BLOCK_ID));
        return;
    }
    constexpr int ROWB = D * ESZ;        // bytes per token row
    constexpr int PER_TOK = ROWB / 16;   // 16-byte pieces per token row
    for (int idx = threadIdx.x; idx < BS * PER_TOK; idx += blockDim.x) {
        const int t = idx / PER_TOK;
        const int e = (idx - t * PER_TOK) * 16;
        const int p = lb * BS + t;
        if (p >= n) continue;
        const size_t src = ((static_cast<size_t>(blk) * hkv + g) * BS + t) * ROWB + e;
        const size_t dst = ((static_cast<size_t>(b) * hkv + g) * l_max + p) * ROWB + e;
        *reinterpret_cast<uint4*>(k_out + dst) = *reinterpret_cast<const uint4*>(kc + src);
        *reinterpret_cast<uint4*>(v_out + dst) = *reinterpret_cast<const uint4*>(vc + src);
    }
}

// Prefetch depth of the attention tile ring and waves per CU of its grid.
// One wave per SIMD with one bf16 tile in flight beyond the one being
// consumed measured fastest on MI355X (long contexts and short batches
// alike): more or deeper streams only add pieces to combine. 8-bit tiles are
// half the bytes, so that cache keeps more of them in flight.
constexpr int kAttnPrefetch = 1;
constexpr int kAttnPrefetchFp8 = 2;
constexpr int kAttnWavesPerCU = 3;
// Query column blocks of 16 per wave of the prefill rescaling launch.
constexpr int kPrefillQB = 3;

// Grid of the attention kernel on the current device: CUs x min(waves per
// CU, resident workgroups per CU at the kernel's register budget), cached
// per device (the kernels differ only in G, all fit kAttnWavesPerCU).
template <typename K>
int attention_waves(K kernel) {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return mikv::kMaxAttnWaves;
    if (cached[dev] > 0) return cached[dev];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0)
        return mikv::kMaxAttnWaves;
    cached[dev] = std::min(mikv::kMaxAttnWaves, std::min(per_cu, kAttnWavesPerCU) * cus);
    return cached[dev];
}

// Upper bound of attention_waves() on the current device without naming a
// kernel: kAttnWavesPerCU waves on every CU (cached per device).
int resident_wave_bound() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return mikv::kMaxAttnWaves;
    if (cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return mikv::kMaxAttnWaves;
    cached[dev] = std::min(mikv::kMaxAttnWaves, kAttnWavesPerCU * cus);
    return cached[dev];
}

// The per-segment form of the two-call decode (no workspace, no combine).
template <int D, int G>
void launch_attn_seg(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out, const int32_t* table,
                     int32_t mbps, const int32_t* ctx, int32_t batch, float scale_log2, int32_t max_ctx,
                     hipStream_t st) {
    const int hkv = p->num_kv_heads;
    auto kern = mikv::pool_fp8(p) ? paged_attn_seg_kernel<D, G, kFmtFp8, kAttnPrefetchFp8>
                                  : paged_attn_seg_kernel<D, G, kFmtBf16, kAttnPrefetch>;
    hipLaunchKernelGGL(kern, dim3(hkv, batch), dim3(64 * kSegWaves), 0, st, q_rot,
                       static_cast<const uint8_t*>(p->k), static_cast<const uint8_t*>(p->v), table, mbps, ctx,
                       hkv, p->num_blocks, max_ctx, scale_log2, static_cast<const float*>(p->scales), out,
                       p->err);
}

// The dot-product form (pool flag MI_POOL_DECODE_DOT) of the two-call decode.
template <int D, int G>
void launch_attn_dot(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out, const int32_t* table,
                     int32_t mbps, const int32_t* ctx, int32_t batch, float scale_log2, int32_t max_ctx,
                     int32_t min_tiles, float* part_acc, float2* part_ml, hipStream_t st) {
    constexpr int LAM = DotShape<D, G>::LAM;
    constexpr int PF = DotShape<D, G>::PF;
    const int hkv = p->num_kv_heads;
    auto kern = mikv::pool_fp8(p) ? paged_attn_dot_kernel<D, G, LAM, kFmtFp8, PF>
                                  : paged_attn_dot_kernel<D, G, LAM, kFmtBf16, PF>;
    const int waves = mikv::attention_grid_waves(batch, hkv, max_ctx, min_tiles, attention_waves(kern));
    hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, st, q_rot, static_cast<const uint8_t*>(p->k),
                       static_cast<const uint8_t*>(p->v), table, mbps, ctx, batch, hkv, p->num_blocks, max_ctx,
                       min_tiles, scale_log2, static_cast<const float*>(p->scales), part_acc, part_ml, out,
                       p->err);
    hipLaunchKernelGGL((paged_attn_combine_kernel<D, G, false>), dim3(hkv * G, batch), dim3(256), 0, st,
                       part_acc, part_ml, ctx, batch, mbps, hkv, max_ctx, waves, min_tiles, out,
                       static_cast<float*>(nullptr));
}

template <int D, int G, bool STEP, bool LAYER>
void launch_attn_kernel(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                        const int32_t* table, int32_t mbps, const int32_t* ctx, int32_t batch,
                        float scale_log2, int32_t max_ctx, int32_t min_tiles, float* part_acc,
                        float2* part_ml, const StepToken& tok, const LayerIO& lio, hipStream_t st) {
    typedef typename CachePtr<STEP>::type CP;
    const int hkv = p->num_kv_heads;
    auto kern = mikv::pool_fp8(p) ? paged_attn_mfma_kernel<D, G, kFmtFp8, kAttnPrefetchFp8, STEP, LAYER>
                                  : paged_attn_mfma_kernel<D, G, kFmtBf16, kAttnPrefetch, STEP, LAYER>;
    const int waves = mikv::attention_grid_waves(batch, hkv, max_ctx, min_tiles, attention_waves(kern));
    hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, st, q_rot, static_cast<CP>(p->k),
                       static_cast<CP>(p->v), table, mbps, ctx, batch, hkv, p->num_blocks, max_ctx,
                       min_tiles, scale_log2, static_cast<const float*>(p->scales), part_acc, part_ml,
                       out, p->err, tok, lio);
    hipLaunchKernelGGL((paged_attn_combine_kernel<D, G, LAYER>), dim3(hkv * G, batch), dim3(256), 0, st,
                       part_acc, part_ml, ctx, batch, mbps, hkv, max_ctx, waves, min_tiles, out, lio.out);
}

// tok: NULL for the attention call, else the decode step's new token; lio:
// non-NULL for the decoder layer's attention.
template <int D, int G>
void launch_attn(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                 const int32_t* table, int32_t mbps, const int32_t* ctx, int32_t batch,
                 float scale_log2, int32_t max_ctx, int32_t min_tiles, float* part_acc,
                 float2* part_ml, const StepToken* tok, const LayerIO* lio, bool seg, hipStream_t st) {
    if (seg)
        launch_attn_seg<D, G>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx, st);
    else if (tok)
        launch_attn_kernel<D, G, true, false>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,
                                              min_tiles, part_acc, part_ml, *tok, LayerIO{}, st);
    else if (lio)
        launch_attn_kernel<D, G, false, true>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,
                                              min_tiles, part_acc, part_ml, StepToken{}, *lio, st);
    else if (p->flags & MI_POOL_DECODE_DOT)
        launch_attn_dot<D, G>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx, min_tiles, part_acc,
                              part_ml, st);
    else
        launch_attn_kernel<D, G, false, false>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,
                                               min_tiles, part_acc, part_ml, StepToken{}, LayerIO{}, st);
}

template <int D>
int dispatch_group(int G, const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                   const int32_t* table, int32_t mbps, const int32_t* ctx, int32_t batch,
                   float scale_log2, int32_t max_ctx, int32_t min_tiles, float* pa, float2* pm,
                   const StepToken* tok, const LayerIO* lio, bool seg, hipStream_t st) {
#define MIKV_G(GG)                                                                             \
    case GG:                                                                                   \
        launch_attn<D, GG>(p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,        \
                           min_tiles, pa, pm, tok, lio, seg, st);                              \
        return MI_OK;
    switch (G) {
        MIKV_G(1)
        MIKV_G(2)
        MIKV_G(3)
        MIKV_G(4)
        MIKV_G(5)
        MIKV_G(6)
        MIKV_G(7)
        MIKV_G(8)
        default: return MI_ERR_UNSUPPORTED;
    }
#undef MIKV_G
}

template <int D, int G>
void launch_prefill(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                    const int32_t* table, int32_t mbps, const int32_t* ctx, const int32_t* cu,
                    int32_t batch, int32_t total, int32_t max_new, float scale_log2, hipStream_t st) {
    const int hkv = p->num_kv_heads;
    const bool f8 = mikv::pool_fp8(p);
    uint32_t gen = ++p->prefill_gen;
    if (gen == 0) gen = ++p->prefill_gen;           // 0 is the word's initial value
    uint32_t* redo = p->err + mikv::kPrefillRedoWord;
    auto fixed = paged_prefill_fa_kernel<D, G, kFmtFp8>;
    auto rescale = f8 ? paged_prefill_rescale_kernel<D, G, kFmtFp8, kAttnPrefetchFp8, kPrefillQB>
                      : paged_prefill_rescale_kernel<D, G, kFmtBf16, kAttnPrefetch, kPrefillQB>;
    const dim3 grid_f(hkv * batch * ((max_new + kFaRows - 1) / kFaRows));
    const dim3 grid_r((max_new + BS * kPrefillQB - 1) / (BS * kPrefillQB), hkv * G, batch);
    if (f8)
        hipLaunchKernelGGL(fixed, grid_f, dim3(64 * G), 0, st, q_rot, static_cast<const uint8_t*>(p->k),
                           static_cast<const uint8_t*>(p->v), table, mbps, ctx, cu, batch, hkv, p->num_blocks,
                           total, max_new, scale_log2, static_cast<const float*>(p->scales), out, p->err,
                           redo, gen);
    else
        hipLaunchKernelGGL((paged_prefill_dma_kernel<D, G>), grid_f, dim3(64 * G), 0, st, q_rot,
                           static_cast<const uint8_t*>(p->k), static_cast<const uint8_t*>(p->v), table, mbps,
                           ctx, cu, batch, hkv, p->num_blocks, total, max_new, scale_log2, out, p->err, redo, gen);
    hipLaunchKernelGGL(rescale, grid_r, dim3(64), 0, st, q_rot, static_cast<const uint8_t*>(p->k),
                       static_cast<const uint8_t*>(p->v), table, mbps, ctx, cu, hkv, p->num_blocks,
                       total, max_new, scale_log2, static_cast<const float*>(p->scales), out, p->err,
                       redo, gen);
}

template <int D>
int dispatch_prefill(int G, const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                     const int32_t* table, int32_t mbps, const int32_t* ctx, const int32_t* cu,
                     int32_t batch, int32_t total, int32_t max_new, float scale_log2, hipStream_t st) {
#define MIKV_G(GG)                                                                             \
    case GG:                                                                                   \
        launch_prefill<D, GG>(p, q_rot, out, table, mbps, ctx, cu, batch, total, max_new,     \
                              scale_log2, st);                                                 \
        return MI_OK;
    switch (G) {
        MIKV_G(1)
        MIKV_G(2)
        MIKV_G(3)
        MIKV_G(4)
        MIKV_G(5)
        MIKV_G(6)
        MIKV_G(7)
        MIKV_G(8)
        default: return MI_ERR_UNSUPPORTED;
    }
#undef MIKV_G
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

namespace mikv {

int32_t default_split_tokens(int32_t, int32_t, int32_t) { return kDefaultSplitTokens; }

int attention_grid_waves(int32_t batch, int32_t hkv, int32_t max_ctx, int32_t min_tiles,
                         int resident) {
    // upper bound of the tile count: every sequence at max_context_len
    const int64_t t_upper = static_cast<int64_t>(batch) * hkv * ((max_ctx + BS) / BS);
    const int64_t by_work = (t_upper + min_tiles - 1) / min_tiles;
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(resident, by_work)));
}

size_t attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t split_tokens) {
    const int waves = attention_grid_waves(batch, num_kv_heads, max_context_len, split_tokens / BS,
                                           kMaxAttnWaves);
    const size_t slots = 2 * static_cast<size_t>(waves) * (num_q_heads / num_kv_heads);
    return align_up(slots * head_dim * sizeof(float), 256) + align_up(slots * sizeof(float2), 256);
}

int launch_write_decode_kv(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* q_rot, const int32_t* table, int32_t mbps,
                           const int32_t* ctx, int32_t batch, int32_t hq, double theta,
                           void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int hkv = p->num_kv_heads;
    const int items = (hq + hkv) * (p->head_dim / 2) + hkv * (p->head_dim / 8);
    const dim3 grid(batch, (items + 255) / 256);
    const RopeTable rope = make_rope_table(theta, p->head_dim);
    const bool f8 = pool_fp8(p);
    auto kern = p->head_dim == 128
                    ? (f8 ? write_decode_kv_kernel<128, kFmtFp8> : write_decode_kv_kernel<128, kFmtBf16>)
                    : (f8 ? write_decode_kv_kernel<64, kFmtFp8> : write_decode_kv_kernel<64, kFmtBf16>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q, k, v, q_rot, p->k, p->v, table, mbps, ctx, hq, hkv,
                       p->num_blocks, rope, static_cast<const float*>(p->scales), p->err);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

int launch_write_prefill_kv(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, uint16_t* q_rot, const int32_t* table, int32_t mbps,
                            const int32_t* ctx, const int32_t* cu, int32_t batch, int32_t tokens,
                            int32_t hq, double theta, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int hkv = p->num_kv_heads;
    const dim3 grid((tokens + kWpRows - 1) / kWpRows);
    const RopeTable rope = make_rope_table(theta, p->head_dim);
    const bool f8 = pool_fp8(p);
    auto kern = p->head_dim == 128
                    ? (f8 ? write_prefill_kv_kernel<128, kFmtFp8> : write_prefill_kv_kernel<128, kFmtBf16>)
                    : (f8 ? write_prefill_kv_kernel<64, kFmtFp8> : write_prefill_kv_kernel<64, kFmtBf16>);
    hipLaunchKernelGGL(kern, grid, dim3(kWpThreads), 0, st, q, k, v, q_rot, p->k, p->v, table, mbps, ctx,
                       cu, batch, tokens, hq, hkv, p->num_blocks, rope, static_cast<const float*>(p->scales),
                       p->err);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

// ----------------------------------------------- allocation-free decode
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the split-K
// partials of the decode attention in this fixed device array instead of a
// workspace. Every device the library runs on holds its own copy until the
// process ends. Host code never uses the array's name as an address: the
// address of the current device's copy comes from hipGetSymbolAddress, taken
// once per device at pool creation (setup_noalloc_scratch) and kept in
// g_scratch_addr.
namespace {

static __device__ __align__(256) uint8_t scratch[MI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

int setup_noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MI_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev]) return MI_OK;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MI_ERR_HIP;
    g_scratch_addr[dev] = ptr;
    return MI_OK;
}

void* noalloc_scratch(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_addr[dev];
}

namespace {

// ws_waves: the wave count the workspace's partial slots are laid out for
// (at least the grid the launch takes); 0 selects the bound the workspace
// queries use.
// default_split: the library's split was asked for; then a small workload of
// the plain two-call form (no step token, not the layer, not the dot form)
// takes the per-segment kernel.
int launch_decode(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out, const int32_t* table,
                  int32_t mbps, const int32_t* ctx, int32_t batch, int32_t hq, float scale,
                  int32_t max_ctx, int32_t split_tokens, void* ws, const StepToken* tok,
                  void* stream, int ws_waves = 0, const LayerIO* lio = nullptr, bool default_split = false) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int G = hq / p->num_kv_heads;
    const int min_tiles = split_tokens / BS;
    const int waves_bound = ws_waves > 0 ? ws_waves
                                         : attention_grid_waves(batch, p->num_kv_heads, max_ctx,
                                                                min_tiles, kMaxAttnWaves);
    const size_t slots = 2 * static_cast<size_t>(waves_bound) * G;
    float* pa = static_cast<float*>(ws);
    float2* pm = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                           align_up(slots * p->head_dim * sizeof(float), 256));
    const float scale_log2 = scale * 1.4426950408889634f;
    const bool seg = default_split && !tok && !lio && !(p->flags & MI_POOL_DECODE_DOT) &&
                     (max_ctx + BS) / BS <= kSegWaves * kSegMaxTilesPerWave &&
                     batch * p->num_kv_heads <= kSegMaxSegments;
    int rc;
    if (p->head_dim == 128)
        rc = dispatch_group<128>(G, p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,
                                 min_tiles, pa, pm, tok, lio, seg, st);
    else
        rc = dispatch_group<64>(G, p, q_rot, out, table, mbps, ctx, batch, scale_log2, max_ctx,
                                min_tiles, pa, pm, tok, lio, seg, st);
    if (rc != MI_OK) return rc;
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

}  // namespace

int launch_paged_gqa_decode(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                            const int32_t* table, int32_t mbps, const int32_t* ctx, int32_t batch,
                            int32_t hq, float scale, int32_t max_ctx, int32_t split_tokens,
                            void* ws, void* stream, bool default_split) {
    return launch_decode(p, q_rot, out, table, mbps, ctx, batch, hq, scale, max_ctx, split_tokens,
                         ws, nullptr, stream, 0, nullptr, default_split);
}

int launch_layer_attention(const mi_kv_pool_s* p, const uint16_t* q_hi, const uint16_t* q_lo,
                           float* out, const int32_t* table, int32_t mbps, const int32_t* ctx,
                           int32_t batch, int32_t hq, float scale, int32_t max_ctx, void* ws,
                           void* stream) {
    LayerIO lio;
    lio.q_lo = q_lo;
    lio.out = out;
    return launch_decode(p, q_hi, nullptr, table, mbps, ctx, batch, hq, scale, max_ctx,
                         kDefaultSplitTokens, ws, nullptr, stream, 0, &lio);
}

int launch_paged_gqa_decode_noalloc(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                                    const int32_t* table, int32_t mbps, const int32_t* ctx,
                                    int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                                    void* stream) {
    void* ws = noalloc_scratch(p->device);
    if (!ws) return MI_ERR_HIP;
    // the partial slots are laid out for the grid the launch takes (at most
    // kAttnWavesPerCU waves per CU), not for the workspace queries' bound
    const int min_tiles = kDefaultSplitTokens / BS;
    const int waves = attention_grid_waves(batch, p->num_kv_heads, max_ctx, min_tiles, resident_wave_bound());
    const size_t slots = 2 * static_cast<size_t>(waves) * (hq / p->num_kv_heads);
    const size_t need = align_up(slots * p->head_dim * sizeof(float), 256) + align_up(slots * sizeof(float2), 256);
    if (need > MI_NOALLOC_SCRATCH_BYTES) return MI_ERR_SCRATCH_TOO_SMALL;
    return launch_decode(p, q_rot, out, table, mbps, ctx, batch, hq, scale, max_ctx,
                         kDefaultSplitTokens, ws, nullptr, stream, waves, nullptr, true);
}

int launch_decode_step(const mi_kv_pool_s* p, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, uint16_t* q_rot, uint16_t* out, const int32_t* table,
                       int32_t mbps, const int32_t* ctx, int32_t batch, int32_t hq, double theta,
                       float scale, int32_t max_ctx, void* ws, void* stream) {
    StepToken tok;
    tok.q = q;
    tok.k = k;
    tok.v = v;
    tok.q_rot = q_rot;
    tok.rope = make_rope_table(theta, p->head_dim);
    return launch_decode(p, nullptr, out, table, mbps, ctx, batch, hq, scale, max_ctx,
                         kDefaultSplitTokens, ws, &tok, stream);
}

int launch_paged_prefill(const mi_kv_pool_s* p, const uint16_t* q_rot, uint16_t* out,
                         const int32_t* table, int32_t mbps, const int32_t* ctx, const int32_t* cu,
                         int32_t batch, int32_t total, int32_t max_new, int32_t hq, float scale,
                         void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int G = hq / p->num_kv_heads;
    const float scale_log2 = scale * 1.4426950408889634f;
    const int rc = p->head_dim == 128
                       ? dispatch_prefill<128>(G, p, q_rot, out, table, mbps, ctx, cu, batch, total,
                                               max_new, scale_log2, st)
                       : dispatch_prefill<64>(G, p, q_rot, out, table, mbps, ctx, cu, batch, total,
                                              max_new, scale_log2, st);
    if (rc != MI_OK) return rc;
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

}  // namespace mikv

// ============================================================== C entry points
namespace {

int check_common(const mi_kv_pool_s* p, int32_t batch, int32_t hq, int32_t mbps) {
    if (!p || batch < 0 || mbps <= 0) return MI_ERR_INVALID_ARG;
    if (!mikv::pool_has_device(p)) return MI_ERR_INVALID_ARG;
    if (!mikv::supported_group(hq, p->num_kv_heads)) return MI_ERR_UNSUPPORTED;
    return MI_OK;
}

}  // namespace

extern "C" int mi_write_decode_kv(mi_kv_pool_t p, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, uint16_t* q_rot, const int32_t* table,
                                  int32_t mbps, const int32_t* ctx, int32_t batch, int32_t hq,
                                  double theta, void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (batch == 0) return MI_OK;
    if (!q || !k || !v || !q_rot || !table || !ctx || !(theta > 0.0)) return MI_ERR_INVALID_ARG;
    return mikv::launch_write_decode_kv(p, q, k, v, q_rot, table, mbps, ctx, batch, hq, theta, stream);
}

extern "C" int mi_write_prefill_kv(mi_kv_pool_t p, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, uint16_t* q_rot, const int32_t* table,
                                   int32_t mbps, const int32_t* ctx, const int32_t* cu, int32_t batch,
                                   int32_t total_tokens, int32_t hq, double theta, void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (total_tokens < 0) return MI_ERR_INVALID_ARG;
    if (batch == 0 || total_tokens == 0) return MI_OK;
    if (!q || !k || !v || !q_rot || !table || !ctx || !cu || !(theta > 0.0)) return MI_ERR_INVALID_ARG;
    return mikv::launch_write_prefill_kv(p, q, k, v, q_rot, table, mbps, ctx, cu, batch, total_tokens,
                                         hq, theta, stream);
}

extern "C" int mi_paged_prefill_attention(mi_kv_pool_t p, const uint16_t* q_rot, uint16_t* out,
                                          const int32_t* table, int32_t mbps, const int32_t* ctx,
                                          const int32_t* cu, int32_t batch, int32_t total_tokens,
                                          int32_t max_new_tokens, int32_t hq, float scale,
                                          void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (total_tokens < 0 || max_new_tokens < 0 || batch > 65535) return MI_ERR_INVALID_ARG;
    if (batch == 0 || total_tokens == 0 || max_new_tokens == 0) return MI_OK;
    if (static_cast<int64_t>(p->num_kv_heads) * batch * ((max_new_tokens + kFaRows - 1) / kFaRows) *
            64 * (hq / p->num_kv_heads) > int64_t{0xffffffff})
        return MI_ERR_UNSUPPORTED;                  // threads of the one-dimensional grid
    if (!q_rot || !out || !table || !ctx || !cu || q_rot == out) return MI_ERR_INVALID_ARG;
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(p->head_dim));
    return mikv::launch_paged_prefill(p, q_rot, out, table, mbps, ctx, cu, batch, total_tokens,
                                      max_new_tokens, hq, scale, stream);
}

extern "C" size_t mi_paged_gqa_decode_split_workspace_bytes(mi_kv_pool_t p, int32_t batch,
                                                            int32_t hq, int32_t max_ctx,
                                                            int32_t split_tokens) {
    if (!p || batch < 0 || hq <= 0 || max_ctx < 0) return 0;
    if (split_tokens == 0) split_tokens = mikv::default_split_tokens(batch, p->num_kv_heads, max_ctx);
    if (split_tokens <= 0 || split_tokens % BS) return 0;
    if (!mikv::supported_group(hq, p->num_kv_heads) || batch > mikv::kMaxBatch) return 0;
    return mikv::attention_workspace_bytes(batch, hq, p->num_kv_heads, p->head_dim, max_ctx,
                                           split_tokens);
}

extern "C" size_t mi_paged_gqa_decode_workspace_bytes(mi_kv_pool_t p, int32_t batch, int32_t hq,
                                                      int32_t max_ctx) {
    return mi_paged_gqa_decode_split_workspace_bytes(p, batch, hq, max_ctx, 0);
}

extern "C" int mi_paged_gqa_decode_split(mi_kv_pool_t p, const uint16_t* q_rot, uint16_t* out,
                                         const int32_t* table, int32_t mbps, const int32_t* ctx,
                                         int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                                         int32_t split_tokens, void* ws, size_t ws_bytes,
                                         void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (max_ctx < 0 || split_tokens < 0) return MI_ERR_INVALID_ARG;
    const bool default_split = split_tokens == 0;
    if (split_tokens == 0) split_tokens = mikv::default_split_tokens(batch, p->num_kv_heads, max_ctx);
    if (split_tokens % BS) return MI_ERR_UNSUPPORTED;
    if (batch > mikv::kMaxBatch) return MI_ERR_UNSUPPORTED;
    if (batch == 0) return MI_OK;
    if (!q_rot || !out || !table || !ctx || !ws || q_rot == out) return MI_ERR_INVALID_ARG;
    if (ws_bytes < mikv::attention_workspace_bytes(batch, hq, p->num_kv_heads, p->head_dim, max_ctx,
                                                   split_tokens))
        return MI_ERR_WORKSPACE_TOO_SMALL;
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(p->head_dim));
    return mikv::launch_paged_gqa_decode(p, q_rot, out, table, mbps, ctx, batch, hq, scale, max_ctx,
                                         split_tokens, ws, stream, default_split);
}

extern "C" int mi_paged_gqa_decode(mi_kv_pool_t p, const uint16_t* q_rot, uint16_t* out,
                                   const int32_t* table, int32_t mbps, const int32_t* ctx,
                                   int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                                   void* ws, size_t ws_bytes, void* stream) {
    return mi_paged_gqa_decode_split(p, q_rot, out, table, mbps, ctx, batch, hq, scale, max_ctx, 0,
                                     ws, ws_bytes, stream);
}

extern "C" int mi_gather_kv(mi_kv_pool_t p, const int32_t* table, int32_t mbps, const int32_t* ctx,
                            int32_t batch, int32_t len_extra, void* k_out, void* v_out,
                            int32_t l_max, void* stream) {
    if (!p || !mikv::pool_has_device(p) || batch < 0 || mbps <= 0 || l_max < 0) return MI_ERR_INVALID_ARG;
    if (len_extra != 0 && len_extra != 1) return MI_ERR_INVALID_ARG;
    if (batch == 0 || l_max == 0) return MI_OK;
    if (!table || !ctx || !k_out || !v_out) return MI_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((l_max + BS - 1) / BS, p->num_kv_heads, batch);
    const bool f8 = mikv::pool_fp8(p);
    auto kern = p->head_dim == 128 ? (f8 ? gather_kv_kernel<128, 1> : gather_kv_kernel<128, 2>)
                                   : (f8 ? gather_kv_kernel<64, 1> : gather_kv_kernel<64, 2>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const uint8_t*>(p->k),
                       static_cast<const uint8_t*>(p->v), table, mbps, ctx, p->num_kv_heads,
                       p->num_blocks, len_extra, l_max, static_cast<uint8_t*>(k_out),
                       static_cast<uint8_t*>(v_out), p->err);
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" int mi_kv_pool_quantize(mi_kv_pool_t p, const uint16_t* k_src, const uint16_t* v_src,
                                   void* stream) {
    if (!p || !mikv::pool_has_device(p) || !mikv::pool_fp8(p) || !k_src || !v_src)
        return MI_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t pieces = static_cast<size_t>(p->num_blocks) * p->num_kv_heads * BS * p->head_dim / 8;
    const unsigned blocks = static_cast<unsigned>(std::min<size_t>((pieces + 255) / 256, 8192));
    auto kern = p->head_dim == 128 ? quantize_pool_kernel<128> : quantize_pool_kernel<64>;
    hipLaunchKernelGGL(kern, dim3(blocks, 2), dim3(256), 0, st, k_src, v_src,
                       static_cast<uint8_t*>(p->k), static_cast<uint8_t*>(p->v), pieces,
                       p->num_kv_heads, static_cast<const float*>(p->scales));
    return hipGetLastError() == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" int mi_paged_gqa_decode_step(mi_kv_pool_t p, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, uint16_t* q_rot, uint16_t* out,
                                        const int32_t* table, int32_t mbps, const int32_t* ctx,
                                        int32_t batch, int32_t hq, double theta, float scale,
                                        int32_t max_ctx, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (max_ctx < 0) return MI_ERR_INVALID_ARG;
    if (batch > mikv::kMaxBatch) return MI_ERR_UNSUPPORTED;
    if (batch == 0) return MI_OK;
    if (!q || !k || !v || !out || !table || !ctx || !ws || !(theta > 0.0)) return MI_ERR_INVALID_ARG;
    if (out == q || (q_rot && (q_rot == q || q_rot == out))) return MI_ERR_INVALID_ARG;
    if (ws_bytes < mikv::attention_workspace_bytes(batch, hq, p->num_kv_heads, p->head_dim, max_ctx,
                                                   mikv::kDefaultSplitTokens))
        return MI_ERR_WORKSPACE_TOO_SMALL;
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(p->head_dim));
    return mikv::launch_decode_step(p, q, k, v, q_rot, out, table, mbps, ctx, batch, hq, theta, scale,
                                    max_ctx, ws, stream);
}

extern "C" int mi_paged_gqa_decode_noalloc(mi_kv_pool_t p, const uint16_t* q_rot, uint16_t* out,
                                           const int32_t* table, int32_t mbps, const int32_t* ctx,
                                           int32_t batch, int32_t hq, float scale, int32_t max_ctx,
                                           void* stream) {
    int rc = check_common(p, batch, hq, mbps);
    if (rc != MI_OK) return rc;
    if (max_ctx < 0) return MI_ERR_INVALID_ARG;
    if (batch > mikv::kMaxBatch) return MI_ERR_UNSUPPORTED;
    if (batch == 0) return MI_OK;
    if (!q_rot || !out || !table || !ctx || q_rot == out) return MI_ERR_INVALID_ARG;
    if (!(scale > 0.f)) scale = 1.0f / sqrtf(static_cast<float>(p->head_dim));
    return mikv::launch_paged_gqa_decode_noalloc(p, q_rot, out, table, mbps, ctx, batch, hq, scale,
                                                 max_ctx, stream);
}

// tb.hip -- HIP kernels and C ABI of libtb.so: ternary-weight int8 FFN decode for gfx950.
//
// The path, after "perf(bonsai): decode and small packed batches read the FFN from a
// ternary copy through a dp4a GEMV" (sparkinfer PR #1154, Summary and commit message):
//   1. a Hadamard rotation emits one int8 copy of the activation, which gate and up share
//      (rotquant_kernel);
//   2. an integer dot-product GEMV streams the stored ternary blocks, stages the int8
//      activation once per workgroup, folds each block's scale into its integer sum, and
//      reduces with a lane shuffle tree (gemv_kernel);
//   3. packed steps of up to 8 rows give every row the bytes it gets alone: each row's lane
//      walk, block fold and reduction tree do not depend on the row count M.
//
// gfx950 mapping (the pages' sm_120 design is prior art; this is the CDNA4 one):
//   * wave64. A wave covers 4 weight rows x 16 "chunk lanes". A chunk is 16 bytes of codes:
//     64 ternary weights (half a block) or 128 sign weights (one block). In each iteration
//     the 16 lanes of a row read 256 contiguous bytes: fully coalesced 16-byte non-temporal
//     loads.
//   * 2-bit decode without a lookup in memory. For one 32-bit code word (16 weights):
//     and-masks 0x03030303 / 0x0C0C0C0C on w and on w >> 4 give byte selectors. v_perm_b32
//     maps each selector byte to the int8 weight {0, +1, -1, 0}; the 0x0C case uses perm's
//     selector values 4, 8 and 12 directly. That is 9 VALU ops per 16 weights, shared by
//     all M rows. Each resulting word holds weights {j, j+4, j+8, j+12}, so the activation
//     is staged in LDS as a 4x4 byte transpose of every 16-byte group, and
//     v_dot4c_i32_i8 consumes both words as they are.
//   * The activation LDS layout is [m][code word j][chunk c] of 16-byte groups, so the 16
//     lanes of a row read 256 consecutive bytes per ds_read_b128: no bank conflicts,
//     without padding. The 4 row groups of a wave read the same addresses (broadcast).
//   * The two half-block sums of a block are combined with one DPP quad_perm add (exact
//     integers). The fp32 fold is tau = (scale * dq) * float(isum), accumulated per lane in
//     block order, then a fixed __shfl_down tree over the lanes of the row.
//   * The sign format uses isum = 2 * dot(bits, q) - sum(q). Bits come from shift-and
//     (w >> j) & 0x01010101, with the activation staged as an 8x4 transpose, and sum(q) is
//     computed once per block while staging.
//   * No MFMA: with M <= 8 rows this is not a dense contraction. No floating-point atomics.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <cmath>
#include <mutex>

#include "tb.h"

namespace {

constexpr int kBlock = 128;
constexpr int kThreads = 256;         // 4 waves
constexpr int kRowsPerWG = 16;        // 4 waves x 4 row groups
constexpr int kChunkLanes = 16;

enum Mode { kModeY = 0, kModeGateUp = 1, kModeIsum = 2 };

// ------------------------------------------------------------------------------------
// Rotate + quantise: 16 lanes per 128-block, lane L holds elements 8L .. 8L+7.
// Stages of span 1, 2, 4 are inside a lane. Spans 8, 16, 32, 64 pair lane L with
// L ^ 1, 2, 4, 8. Ascending order; each butterfly is (a, b) -> (a + b, a - b) in fp32.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rotquant_kernel(const float *__restrict__ x,
                                                            long nblocks,
                                                            int8_t *__restrict__ q,
                                                            float *__restrict__ dq, float unit)
{
    const int lane16 = threadIdx.x & 15;
    const long blk = (long)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
    if (blk >= nblocks)
        return;  // the whole 16-lane group leaves together; shuffles stay inside a group

    const float *src = x + blk * kBlock + lane16 * 8;
    const float4 lo = *reinterpret_cast<const float4 *>(src);
    const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};

#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!(e & h)) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
        const bool upper = (lane16 & s) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float other = __shfl_xor(v[e], s, 16);
            v[e] = upper ? (other - v[e]) : (v[e] + other);
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
    for (int s = 1; s < 16; s <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, s, 16));

    uint32_t packed[2] = {0u, 0u};
    if (amax != 0.0f) {
        const float inv = 127.0f / amax;  // IEEE division (correctly rounded build)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float r = rintf(v[e] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            packed[e >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * (e & 3));
        }
    }
    *reinterpret_cast<uint2 *>(q + blk * kBlock + lane16 * 8) = make_uint2(packed[0], packed[1]);
    if (lane16 == 0)
        dq[blk] = amax != 0.0f ? amax * unit : 0.0f;
}

// ------------------------------------------------------------------------------------
// GEMV
// ------------------------------------------------------------------------------------
struct GemvArgs {
    const uint8_t *codes0;   // the matrix, or gate
    const uint16_t *scales0;
    const uint8_t *codes1;   // up (gate/up mode)
    const uint16_t *scales1;
    int n, k;
    const int8_t *q;         // [M][k]
    const float *dq;         // [M][k/128]
    float *out;              // y or h: [M][n]
    int32_t *isum;           // block-sum export: [M][n][k/128]
    int slice_chunks;        // chunks of K staged per LDS pass (multiple of 16)
};

__device__ __forceinline__ uint32_t byte_at(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

// 4x4 byte transpose: out[j] = (byte j of r0, byte j of r1, byte j of r2, byte j of r3).
__device__ __forceinline__ uint4 transpose4x4(uint4 r)
{
    uint4 o;
    o.x = byte_at(r.x, 0) | byte_at(r.y, 0) << 8 | byte_at(r.z, 0) << 16 | byte_at(r.w, 0) << 24;
    o.y = byte_at(r.x, 1) | byte_at(r.y, 1) << 8 | byte_at(r.z, 1) << 16 | byte_at(r.w, 1) << 24;
    o.z = byte_at(r.x, 2) | byte_at(r.y, 2) << 8 | byte_at(r.z, 2) << 16 | byte_at(r.w, 2) << 24;
    o.w = byte_at(r.x, 3) | byte_at(r.y, 3) << 8 | byte_at(r.z, 3) << 16 | byte_at(r.w, 3) << 24;
    return o;
}

// Ternary decode of one code word into the four int8x4 words {j, j+4, j+8, j+12}.
// Selector bytes 0..3 index the table 0x00FF0100 -> {0, +1, -1, 0}. For the masked field
// at bits 2..3 the selector is 4c: 0 -> byte 0 of S1 (0), 4 -> byte 0 of S0 (+1),
// 8 -> sign of bit 15 of S1 (0xFF = -1), 12 -> 0.
__device__ __forceinline__ void decode_ternary(uint32_t w, uint32_t &d0, uint32_t &d1,
                                               uint32_t &d2, uint32_t &d3)
{
    const uint32_t w4 = w >> 4;
    d0 = __builtin_amdgcn_perm(0u, 0x00FF0100u, w & 0x03030303u);
    d1 = __builtin_amdgcn_perm(1u, 0x00008000u, w & 0x0C0C0C0Cu);
    d2 = __builtin_amdgcn_perm(0u, 0x00FF0100u, w4 & 0x03030303u);
    d3 = __builtin_amdgcn_perm(1u, 0x00008000u, w4 & 0x0C0C0C0Cu);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Swap-adjacent-lanes add: lane 2i and 2i+1 both get their sum (exact integers).
__device__ __forceinline__ int pair_add(int v)
{
    return v + __builtin_amdgcn_update_dpp(0, v, 0xB1 /* quad_perm [1,0,3,2] */, 0xF, 0xF, false);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Weights are read exactly once per call: stream them past the caches.
__device__ __forceinline__ uint4 load_nt(const uint8_t *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float silu_gate(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// LDS layout (bytes): act [M][slice] | dq float [M][nb] | qsum int [M][nb] (sign only)
template <int M, int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr bool kTern = FMT == TB_FMT_TERNARY2;
    constexpr bool kTwo = MODE == kModeGateUp;
    constexpr int kWeightsPerChunk = kTern ? 64 : 128;

    const int k = a.k, n = a.n, nb = k / kBlock;
    const int C = k / kWeightsPerChunk;          // chunks per row
    const int S = a.slice_chunks;                // chunks per LDS pass
    const int tid = threadIdx.x;
    const int lane = tid & 63, cl = lane & 15;
    const int row = blockIdx.x * kRowsPerWG + (tid >> 6) * 4 + (lane >> 4);
    const bool row_ok = row < n;
    const size_t row_bytes = (size_t)C * 16;

    uint8_t *act = lds;
    float *dq_s = reinterpret_cast<float *>(lds + (size_t)M * S * kWeightsPerChunk);
    int *qsum_s = reinterpret_cast<int *>(dq_s + M * nb);

    // scales and dq (and for sign, per-block sum(q)) for the whole row are staged once
    if (MODE != kModeIsum)
        for (int i = tid; i < M * nb; i += kThreads)
            dq_s[i] = a.dq[i];
    if (!kTern) {
        for (int i = tid; i < M * nb; i += kThreads) {
            const int8_t *src = a.q + (size_t)i * kBlock;  // [m][b] blocks are contiguous
            int s = 0;
            for (int j = 0; j < kBlock; j += 16) {
                const uint4 g = *reinterpret_cast<const uint4 *>(src + j);
                s = dot4(g.x, 0x01010101u, s);
                s = dot4(g.y, 0x01010101u, s);
                s = dot4(g.z, 0x01010101u, s);
                s = dot4(g.w, 0x01010101u, s);
            }
            qsum_s[i] = s;
        }
    }

    float acc0[M], acc1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        acc0[m] = 0.0f;
        acc1[m] = 0.0f;
    }

    const uint8_t *rp0 = a.codes0 + (size_t)(row_ok ? row : 0) * row_bytes;
    const uint8_t *rp1 = kTwo ? a.codes1 + (size_t)(row_ok ? row : 0) * row_bytes : nullptr;
    const uint16_t *sp0 = a.scales0 + (size_t)(row_ok ? row : 0) * nb;
    const uint16_t *sp1 = kTwo ? a.scales1 + (size_t)(row_ok ? row : 0) * nb : nullptr;

    for (int c0 = 0; c0 < C; c0 += S) {
        const int sc = min(S, C - c0);  // chunks in this slice
        __syncthreads();                // previous slice fully consumed
        // ---- stage q[:, c0 .. c0+sc) into LDS, transposed -----------------------------
        if (kTern) {
            // one unit = 16 activations = one code word's worth
            const int units = M * sc * 4;
            for (int u = tid; u < units; u += kThreads) {
                const int m = u / (sc * 4), g = u % (sc * 4);
                const int c = g >> 2, j = g & 3;
                const uint4 r = *reinterpret_cast<const uint4 *>(
                    a.q + (size_t)m * k + (size_t)(c0 + c) * 64 + j * 16);
                *reinterpret_cast<uint4 *>(act + (size_t)m * S * 64 + ((size_t)j * S + c) * 16) =
                    transpose4x4(r);
            }
        } else {
            // one unit = 32 activations = one dword of sign bits; 8 words out (2 x uint4)
            const int units = M * sc * 4;
            for (int u = tid; u < units; u += kThreads) {
                const int m = u / (sc * 4), g = u % (sc * 4);
                const int c = g >> 2, d = g & 3;
                const uint8_t *src = reinterpret_cast<const uint8_t *>(a.q) + (size_t)m * k +
                                     (size_t)(c0 + c) * 128 + d * 32;
                const uint4 lo = *reinterpret_cast<const uint4 *>(src);
                const uint4 hi = *reinterpret_cast<const uint4 *>(src + 16);
                const uint32_t r[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                // word j = (q[j], q[8+j], q[16+j], q[24+j]); q[8p+j] is byte j&3 of r[2p + j/4]
                uint32_t o[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    o[j] = byte_at(r[0 + (j >> 2)], j & 3) | byte_at(r[2 + (j >> 2)], j & 3) << 8 |
                           byte_at(r[4 + (j >> 2)], j & 3) << 16 |
                           byte_at(r[6 + (j >> 2)], j & 3) << 24;
                uint8_t *dst = act + (size_t)m * S * 128;
                *reinterpret_cast<uint4 *>(dst + ((size_t)(d * 2 + 0) * S + c) * 16) =
                    make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4 *>(dst + ((size_t)(d * 2 + 1) * S + c) * 16) =
                    make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
        __syncthreads();

        // ---- stream this slice's codes -------------------------------------------------
        for (int cc = cl; cc < ((sc + 15) & ~15); cc += kChunkLanes) {
            const int c = c0 + cc;
            const bool ok = row_ok && cc < sc;
            const uint4 w0 = ok ? load_nt(rp0 + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
            const uint4 w1 = (kTwo && ok) ? load_nt(rp1 + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
            const int b = kTern ? (c >> 1) : c;
            const float s0 = ok ? half_bits_to_float(sp0[b]) : 0.0f;
            const float s1 = (kTwo && ok) ? half_bits_to_float(sp1[b]) : 0.0f;

            int is0[M], is1[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                is0[m] = 0;
                is1[m] = 0;
            }
            if (kTern) {
                const uint32_t cw0[4] = {w0.x, w0.y, w0.z, w0.w};
                const uint32_t cw1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t d0, d1, d2, d3, e0 = 0, e1 = 0, e2 = 0, e3 = 0;
                    decode_ternary(cw0[j], d0, d1, d2, d3);
                    if (kTwo)
                        decode_ternary(cw1[j], e0, e1, e2, e3);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const uint4 av = *reinterpret_cast<const uint4 *>(
                            act + (size_t)m * S * 64 + ((size_t)j * S + (ok ? cc : 0)) * 16);
                        is0[m] = dot4(d0, av.x, is0[m]);
                        is0[m] = dot4(d1, av.y, is0[m]);
                        is0[m] = dot4(d2, av.z, is0[m]);
                        is0[m] = dot4(d3, av.w, is0[m]);
                        if (kTwo) {
                            is1[m] = dot4(e0, av.x, is1[m]);
                            is1[m] = dot4(e1, av.y, is1[m]);
                            is1[m] = dot4(e2, av.z, is1[m]);
                            is1[m] = dot4(e3, av.w, is1[m]);
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    is0[m] = pair_add(is0[m]);
                    if (kTwo)
                        is1[m] = pair_add(is1[m]);
                }
            } else {
                const uint32_t cw0[4] = {w0.x, w0.y, w0.z, w0.w};
                const uint32_t cw1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint32_t bits0[4], bits1[4] = {0, 0, 0, 0};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            bits0[j] = (cw0[d] >> (4 * h + j)) & 0x01010101u;
                            if (kTwo)
                                bits1[j] = (cw1[d] >> (4 * h + j)) & 0x01010101u;
                        }
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            const uint4 av = *reinterpret_cast<const uint4 *>(
                                act + (size_t)m * S * 128 +
                                ((size_t)(d * 2 + h) * S + (ok ? cc : 0)) * 16);
                            is0[m] = dot4(bits0[0], av.x, is0[m]);
                            is0[m] = dot4(bits0[1], av.y, is0[m]);
                            is0[m] = dot4(bits0[2], av.z, is0[m]);
                            is0[m] = dot4(bits0[3], av.w, is0[m]);
                            if (kTwo) {
                                is1[m] = dot4(bits1[0], av.x, is1[m]);
                                is1[m] = dot4(bits1[1], av.y, is1[m]);
                                is1[m] = dot4(bits1[2], av.z, is1[m]);
                                is1[m] = dot4(bits1[3], av.w, is1[m]);
                            }
                        }
                    }
                }
                if (ok) {
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const int qs = qsum_s[m * nb + b];
                        is0[m] = 2 * is0[m] - qs;
                        if (kTwo)
                            is1[m] = 2 * is1[m] - qs;
                    }
                }
            }

            if (!ok)
                continue;
            if (MODE == kModeIsum) {
                if (!kTern || !(cl & 1)) {
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        a.isum[((size_t)m * n + row) * nb + b] = is0[m];
                }
                continue;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float d = dq_s[m * nb + b];
                acc0[m] += (s0 * d) * (float)is0[m];
                if (kTwo)
                    acc1[m] += (s1 * d) * (float)is1[m];
            }
        }
    }

    if (MODE == kModeIsum)
        return;

    // ---- shuffle tree over the lanes of each row (odd lanes of the ternary format hold
    //      duplicates of their even neighbour, so they are skipped) -------------------------
#pragma unroll
    for (int off = kTern ? 2 : 1; off < kChunkLanes; off <<= 1) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            acc0[m] += __shfl_down(acc0[m], off, kChunkLanes);
            if (kTwo)
                acc1[m] += __shfl_down(acc1[m], off, kChunkLanes);
        }
    }
    if (cl == 0 && row_ok) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            a.out[(size_t)m * n + row] = kTwo ? silu_gate(acc0[m], acc1[m]) : acc0[m];
    }
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
using GemvFn = void (*)(GemvArgs);

template <int FMT, int MODE>
GemvFn pick_gemv(int m)
{
    switch (m) {
    case 1: return gemv_kernel<1, FMT, MODE>;
    case 2: return gemv_kernel<2, FMT, MODE>;
    case 3: return gemv_kernel<3, FMT, MODE>;
    case 4: return gemv_kernel<4, FMT, MODE>;
    case 5: return gemv_kernel<5, FMT, MODE>;
    case 6: return gemv_kernel<6, FMT, MODE>;
    case 7: return gemv_kernel<7, FMT, MODE>;
    case 8: return gemv_kernel<8, FMT, MODE>;
    default: return nullptr;
    }
}

GemvFn pick(int fmt, int mode, int m)
{
    if (fmt == TB_FMT_TERNARY2) {
        if (mode == kModeY) return pick_gemv<TB_FMT_TERNARY2, kModeY>(m);
        if (mode == kModeGateUp) return pick_gemv<TB_FMT_TERNARY2, kModeGateUp>(m);
        return pick_gemv<TB_FMT_TERNARY2, kModeIsum>(m);
    }
    if (mode == kModeY) return pick_gemv<TB_FMT_SIGN1, kModeY>(m);
    if (mode == kModeGateUp) return pick_gemv<TB_FMT_SIGN1, kModeGateUp>(m);
    return pick_gemv<TB_FMT_SIGN1, kModeIsum>(m);
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_lds_limit[kMaxDevices];  // 0 = not queried yet

int device_lds_limit(int *limit)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TB_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_lds_limit[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            return TB_EHIP;
        g_lds_limit[dev] = v;
    }
    *limit = g_lds_limit[dev];
    return TB_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
Range range_of(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_matrix(const tb_matrix *w)
{
    if (!w || !w->codes || !w->scales)
        return TB_EINVAL;
    if (w->n < 1 || w->k < kBlock || w->k % kBlock)
        return TB_EINVAL;
    if (w->fmt != TB_FMT_TERNARY2 && w->fmt != TB_FMT_SIGN1)
        return TB_EINVAL;
    if (!aligned16(w->codes) || !aligned16(w->scales))
        return TB_EALIGN;
    return TB_OK;
}

size_t codes_bytes(const tb_matrix *w)
{
    return (size_t)w->n * (size_t)w->k / (w->fmt == TB_FMT_TERNARY2 ? 4 : 8);
}
size_t scales_bytes(const tb_matrix *w) { return (size_t)w->n * (size_t)(w->k / kBlock) * 2; }

int check_rows(int m) { return (m >= 1 && m <= TB_MAX_ROWS) ? TB_OK : TB_EINVAL; }

int launch_rotquant(const float *x, int m, int k, int8_t *q, float *dq, hipStream_t stream)
{
    const long nblocks = (long)m * (k / kBlock);
    const int grid = (int)((nblocks + kThreads / 16 - 1) / (kThreads / 16));
    const float unit = static_cast<float>(1.0 / (127.0 * std::sqrt(128.0)));
    hipLaunchKernelGGL(rotquant_kernel, dim3(grid), dim3(kThreads), 0, stream, x, nblocks, q, dq,
                       unit);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

// LDS bytes for a given slice; the slice shrinks until the workgroup fits the device limit.
int plan_lds(int fmt, int m, int k, int limit, int *slice_chunks, size_t *lds_bytes)
{
    const int wpc = fmt == TB_FMT_TERNARY2 ? 64 : 128;
    const int C = k / wpc, nb = k / kBlock;
    const size_t fixed = (size_t)m * nb * 4 * (fmt == TB_FMT_TERNARY2 ? 1 : 2);
    int S = (C + 15) & ~15;
    for (;;) {
        const size_t bytes = (size_t)m * S * wpc + fixed;
        if (bytes <= (size_t)limit) {
            *slice_chunks = S;
            *lds_bytes = bytes;
            return TB_OK;
        }
        if (S <= 16)
            return TB_EUNSUPPORTED;
        S = ((S / 2) + 15) & ~15;
    }
}

int launch_gemv(int mode, const tb_matrix *w0, const tb_matrix *w1, const int8_t *q,
                const float *dq, int m, float *out, int32_t *isum, hipStream_t stream)
{
    int limit = 0;
    int rc = device_lds_limit(&limit);
    if (rc)
        return rc;
    GemvArgs a;
    a.codes0 = static_cast<const uint8_t *>(w0->codes);
    a.scales0 = w0->scales;
    a.codes1 = w1 ? static_cast<const uint8_t *>(w1->codes) : nullptr;
    a.scales1 = w1 ? w1->scales : nullptr;
    a.n = w0->n;
    a.k = w0->k;
    a.q = q;
    a.dq = dq;
    a.out = out;
    a.isum = isum;
    size_t lds = 0;
    rc = plan_lds(w0->fmt, m, w0->k, limit, &a.slice_chunks, &lds);
    if (rc)
        return rc;
    GemvFn fn = pick(w0->fmt, mode, m);
    if (!fn)
        return TB_EINVAL;
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return TB_EHIP;
    const int grid = (w0->n + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

// Validates a GEMV-shaped call: activations q/dq of m rows against matrix w.
int check_activation(const tb_matrix *w, const int8_t *q, const float *dq, int m)
{
    if (!q || !dq)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(dq))
        return TB_EALIGN;
    (void)w;
    (void)m;
    return TB_OK;
}

}  // namespace

// ====================================================================================
// C ABI
// ====================================================================================
extern "C" {

int tb_abi_version(void) { return TB_ABI_VERSION; }

const char *tb_status_str(int status)
{
    switch (status) {
    case TB_OK: return "ok";
    case TB_EINVAL: return "invalid argument";
    case TB_EALIGN: return "pointer not 16-byte aligned";
    case TB_EUNSUPPORTED: return "unsupported shape for this build or device";
    case TB_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int tb_rotate_quant_i8(const float *x, int m, int k, int8_t *q, float *dq, void *stream)
{
    if (check_rows(m) || k < kBlock || k % kBlock || !x || !q || !dq)
        return TB_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(dq))
        return TB_EALIGN;
    const Range rx = range_of(x, (size_t)m * k * 4), rq = range_of(q, (size_t)m * k),
                rd = range_of(dq, (size_t)m * (k / kBlock) * 4);
    if (overlaps(rx, rq) || overlaps(rx, rd) || overlaps(rq, rd))
        return TB_EINVAL;
    return launch_rotquant(x, m, k, q, dq, static_cast<hipStream_t>(stream));
}

int tb_gemv_ternary(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                    void *stream)
{
    int rc = check_matrix(w);
    if (rc)
        return rc;
    if (check_rows(m) || !y)
        return TB_EINVAL;
    if ((rc = check_activation(w, q, dq, m)))
        return rc;
    if (!aligned16(y))
        return TB_EALIGN;
    const Range ry = range_of(y, (size_t)m * w->n * 4);
    if (overlaps(ry, range_of(w->codes, codes_bytes(w))) ||
        overlaps(ry, range_of(w->scales, scales_bytes(w))) ||
        overlaps(ry, range_of(q, (size_t)m * w->k)) ||
        overlaps(ry, range_of(dq, (size_t)m * (w->k / kBlock) * 4)))
        return TB_EINVAL;
    return launch_gemv(kModeY, w, nullptr, q, dq, m, y, nullptr, static_cast<hipStream_t>(stream));
}

int tb_ffn_gateup_silu(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                       const float *dq, int m, float *h, void *stream)
{
    int rc = check_matrix(wg);
    if (rc)
        return rc;
    if ((rc = check_matrix(wu)))
        return rc;
    if (wg->n != wu->n || wg->k != wu->k || wg->fmt != wu->fmt)
        return TB_EINVAL;
    if (check_rows(m) || !h)
        return TB_EINVAL;
    if ((rc = check_activation(wg, q, dq, m)))
        return rc;
    if (!aligned16(h))
        return TB_EALIGN;
    const Range rh = range_of(h, (size_t)m * wg->n * 4);
    if (overlaps(rh, range_of(wg->codes, codes_bytes(wg))) ||
        overlaps(rh, range_of(wg->scales, scales_bytes(wg))) ||
        overlaps(rh, range_of(wu->codes, codes_bytes(wu))) ||
        overlaps(rh, range_of(wu->scales, scales_bytes(wu))) ||
        overlaps(rh, range_of(q, (size_t)m * wg->k)) ||
        overlaps(rh, range_of(dq, (size_t)m * (wg->k / kBlock) * 4)))
        return TB_EINVAL;
    return launch_gemv(kModeGateUp, wg, wu, q, dq, m, h, nullptr,
                       static_cast<hipStream_t>(stream));
}

int tb_ffn_down(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                float *y, void *stream)
{
    int rc = check_matrix(wd);
    if (rc)
        return rc;
    if (check_rows(m) || !h || !qh_ws || !dqh_ws || !y)
        return TB_EINVAL;
    if (!aligned16(h) || !aligned16(qh_ws) || !aligned16(dqh_ws) || !aligned16(y))
        return TB_EALIGN;
    const int k = wd->k;
    const Range rh = range_of(h, (size_t)m * k * 4), rq = range_of(qh_ws, (size_t)m * k),
                rd = range_of(dqh_ws, (size_t)m * (k / kBlock) * 4),
                ry = range_of(y, (size_t)m * wd->n * 4),
                rc_ = range_of(wd->codes, codes_bytes(wd)),
                rs = range_of(wd->scales, scales_bytes(wd));
    const Range outs[3] = {rq, rd, ry};
    const Range ins[3] = {rh, rc_, rs};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return TB_EINVAL;
    if (overlaps(rq, rd) || overlaps(rq, ry) || overlaps(rd, ry))
        return TB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = launch_rotquant(h, m, k, qh_ws, dqh_ws, s)))
        return rc;
    return launch_gemv(kModeY, wd, nullptr, qh_ws, dqh_ws, m, y, nullptr, s);
}

int tb_gemv_block_sums(const tb_matrix *w, const int8_t *q, int m, int32_t *isum, void *stream)
{
    int rc = check_matrix(w);
    if (rc)
        return rc;
    if (check_rows(m) || !q || !isum)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(isum))
        return TB_EALIGN;
    const Range ri = range_of(isum, (size_t)m * w->n * (w->k / kBlock) * 4);
    if (overlaps(ri, range_of(w->codes, codes_bytes(w))) ||
        overlaps(ri, range_of(w->scales, scales_bytes(w))) || overlaps(ri, range_of(q, (size_t)m * w->k)))
        return TB_EINVAL;
    return launch_gemv(kModeIsum, w, nullptr, q, nullptr, m, nullptr, isum,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"

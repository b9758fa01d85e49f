// tb_lut.h -- lookup-table GEMV for 1-bit sign weights in a row-interleaved layout (gfx950).
//
// After the bonsai-edge-serve README (kernels/ section): a 1-bit kernel built like the 2-bit
// one spends the same instructions per weight on half the bytes, and the remedy named
// there is a lookup-table kernel over a row-interleaved weight layout. The gfx950 form of
// that idea:
//   * Layout TB_FMT_SIGN1_RI4. Rows in groups of four ("quads"); for each quad and 128-block
//     the four rows' 16-byte sign blocks are byte-interleaved: byte r of 32-bit word j is
//     byte j of row r's block (weights 8j .. 8j+7). Scales likewise: [n/4][nb][4] fp16.
//   * Tables. For a pair of activations (q0, q1) the four sums over the weights whose sign
//     bit is set, {0, q0, q1, q0 + q1}, indexed by the pair's two bits. Split into nibbles
//     (q = 16 qh + ql, ql in 0..15, qh in -8..7) every entry fits a byte: the low table
//     {0, ql0, ql1, ql0 + ql1} and the high table {qh0, qh1, qh0 + qh1} biased by +16.
//   * Lookups. (w >> 2t) & 0x03030303 puts the two bits of pair t of all four rows of a
//     word into the four selector bytes of v_perm_b32: one instruction looks up four
//     rows in a register-resident table. The bytes add as packed sums (eight lookups of
//     at most 30 each stay below 256) and widen to 16-bit fields.
//   * The integer result per (row, block) is isum = 2 D - sum(q), D = 16 (H - 16 * 64) + L
//     for the high and low sums H, L over the block's 64 pairs: exact.
//   * A wave keeps the tables of one step (16 blocks) in registers and sweeps the CU's quads
//     for that step: lane (b, c) = (lane / 4, lane % 4) holds pairs 16c .. 16c+15 of block b,
//     16 low and 16 high tables per activation row (32 registers), so this kernel takes at
//     most two rows.
//   * Fold: the lane terms (s * dq) * isum move to lane 16 r + b (ds_bpermute) and take the
//     sign format's fixed row tree, and step partials are summed in step order from +0, as
//     in every other kernel here: y is bit-identical to tb_gemv_ternary on the same weights
//     in the TB_FMT_SIGN1 layout.
#pragma once

#include "tb_device.h"

namespace tblut {

using namespace tbk;

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 2;
constexpr int kDepth = 2;   // code loads in flight per wave

struct LutArgs {
    const uint8_t *codes;     // [n/4][nb][16] 32-bit words (row-interleaved)
    const uint16_t *scales;   // [n/4][nb][4]
    int n, k;
    const int8_t *q;          // [M][k]
    const float *dq;          // [M][k/128]
    float *out;               // [M][n]
    int32_t *isum;            // [M][n][k/128] (block-sum export)
    uint32_t codes_bytes, scales_bytes;
};

// Row-interleave a sign matrix: one thread per output word.
__global__ void sign_interleave_kernel(const uint8_t *__restrict__ codes,
                                       const uint16_t *__restrict__ scales, int n, int nb,
                                       uint32_t *__restrict__ codes_ri,
                                       uint16_t *__restrict__ scales_ri)
{
    const size_t words = (size_t)(n / 4) * nb * 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t quad = i / ((size_t)nb * 16), b = (i / 16) % nb, j = i % 16;
        uint32_t w = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w |= (uint32_t)codes[((4 * quad + r) * nb + b) * 16 + j] << (8 * r);
        codes_ri[i] = w;
        if (j < 4)
            scales_ri[(quad * nb + b) * 4 + j] = scales[(4 * quad + j) * nb + b];
    }
}

// Widen packed byte sums into 16-bit fields: f02 gets bytes 0 and 2, f13 bytes 1 and 3.
__device__ __forceinline__ void widen(uint32_t acc, uint32_t &f02, uint32_t &f13)
{
    f02 += acc & 0x00ff00ffu;
    f13 += (acc >> 8) & 0x00ff00ffu;
}

template <int M, bool ISUM>
__global__ __launch_bounds__(kThreads) void gemv_lut_kernel(LutArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    static_assert(M >= 1 && M <= kMaxRows, "the tables of one row take 32 registers");
    const int n = a.n, k = a.k, nb = k / kBlock;
    const int I = (nb + 15) / 16;   // steps of 16 blocks
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bl = lane >> 2, c = lane & 3;   // block within the step, quarter of the block
    const int G = gridDim.x, cu = blockIdx.x;
    const int T = n / 4;
    const int tA = part_lo(T, G, cu), nq = part_lo(T, G, cu + 1) - tA;
    const int J = nq * I;
    const int i0 = part_lo(J, kWaves, wave), i1 = part_lo(J, kWaves, wave + 1);
    float *part_s = reinterpret_cast<float *>(lds);   // [quad][step][row][m]

    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes, a.codes_bytes);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.scales, a.scales_bytes);
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.q, (uint32_t)(M * k));
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(a.dq, ISUM ? 0u : (uint32_t)(M * nb * 4));
    const __amdgpu_buffer_rsrc_t ro = ISUM ? buffer_rsrc(a.isum, (uint32_t)((size_t)M * n * nb * 4))
                                           : buffer_rsrc(a.out, (uint32_t)(M * n * 4));

    // code word offset of item i for this lane (16 bytes: words 4c .. 4c+3 of block b)
    auto code_off = [&](int i) -> uint32_t {
        if (i >= i1)
            return kOutOfRange;
        const int s = i / nq, quad = tA + (i - s * nq);
        const int b = s * 16 + bl;
        return b < nb ? (uint32_t)(((size_t)quad * nb + b) * 64 + c * 16) : kOutOfRange;
    };

    uint32_t lo[M][16], hi[M][16];
    int qsum[M];
    float dqv[M];
    int cur_step = -1;
    auto build = [&](int s) {
        const int b = s * 16 + bl;
        const uint32_t qo = b < nb ? (uint32_t)(b * kBlock + c * 32) : kOutOfRange;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint4 v0 = buffer_load16(rq, qo, m * k);
            const uint4 v1 = buffer_load16(rq, qo, m * k + 16);
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            int sum = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sum = dot4(w[e], 0x01010101u, sum);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // pair p = 2e + h: activations bytes 2h and 2h + 1 of word e
                    const int q0 = (int)(int8_t)(w[e] >> (16 * h));
                    const int q1 = (int)(int8_t)(w[e] >> (16 * h + 8));
                    const uint32_t l0 = (uint32_t)q0 & 15u, l1 = (uint32_t)q1 & 15u;
                    const uint32_t h0 = (uint32_t)((q0 >> 4) + 16), h1 = (uint32_t)((q1 >> 4) + 16);
                    lo[m][2 * e + h] = (l0 << 8) | (l1 << 16) | ((l0 + l1) << 24);
                    hi[m][2 * e + h] = 16u | (h0 << 8) | (h1 << 16) | ((h0 + h1 - 16u) << 24);
                }
            }
            sum += (int)row_xor((uint32_t)sum, 1);
            sum += (int)row_xor((uint32_t)sum, 2);
            qsum[m] = sum;
            dqv[m] = ISUM ? 0.0f : __uint_as_float(buffer_load_u32(rd, b < nb ? (uint32_t)(b * 4) : kOutOfRange, m * nb * 4));
        }
    };

    uint4 ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        ring[d] = buffer_load16_nt(rc, code_off(i0 + d));

    for (int i = i0; i < i1; ++i) {
        const int s = i / nq, lq = i - s * nq, quad = tA + lq;
        if (s != cur_step) {
            build(s);
            cur_step = s;
        }
        const uint4 cw = ring[0];
#pragma unroll
        for (int d = 0; d + 1 < kDepth; ++d)
            ring[d] = ring[d + 1];
        ring[kDepth - 1] = buffer_load16_nt(rc, code_off(i + kDepth));
        const int b = s * 16 + bl;
        // lookups: 16 pairs, widened every 8
        uint32_t L02[M], L13[M], H02[M], H13[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            L02[m] = L13[m] = H02[m] = H13[m] = 0u;
        const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t al[M], ah[M];
#pragma unroll
            for (int m = 0; m < M; ++m)
                al[m] = ah[m] = 0u;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * half + jj;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t sel = (words[j] >> (2 * t)) & 0x03030303u;
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        al[m] += __builtin_amdgcn_perm(0u, lo[m][4 * j + t], sel);
                        ah[m] += __builtin_amdgcn_perm(0u, hi[m][4 * j + t], sel);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                widen(al[m], L02[m], L13[m]);
                widen(ah[m], H02[m], H13[m]);
            }
        }
        // the block's four quarters: lanes 4 b .. 4 b + 3
        int isum[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            uint32_t v[4] = {L02[m], L13[m], H02[m], H13[m]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] += row_xor(v[e], 1);
                v[e] += row_xor(v[e], 2);
            }
            // row c of the quad: fields (rows 0, 2 | 1, 3), low or high half
            const uint32_t lsel = (c & 1) ? v[1] : v[0], hsel = (c & 1) ? v[3] : v[2];
            const int Ls = (int)((lsel >> ((c & 2) ? 16 : 0)) & 0xffffu);
            const int Hs = (int)((hsel >> ((c & 2) ? 16 : 0)) & 0xffffu);
            const int D = 16 * (Hs - 16 * 64) + Ls;
            isum[m] = 2 * D - qsum[m];
        }
        const uint32_t row = (uint32_t)(quad * 4 + c);
        if constexpr (ISUM) {
            const uint32_t o = b < nb ? (uint32_t)(((size_t)row * nb + b) * 4) : kOutOfRange;
#pragma unroll
            for (int m = 0; m < M; ++m)
                __builtin_amdgcn_raw_buffer_store_b32((uint32_t)isum[m], ro, o, m * n * nb * 4, 0);
        } else {
            const float sc = half_bits_to_float(buffer_load_u16(
                rs, b < nb ? (uint32_t)((((size_t)quad * nb + b) * 4 + c) * 2) : kOutOfRange));
            // lane 16 r + b takes the term of (row r, block b) from lane 4 b + r
            const int src = (4 * (lane & 15) + (lane >> 4)) * 4;
            float p0[M], p1[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float t = (sc * dqv[m]) * (float)isum[m];
                p0[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(t)));
                p1[m] = 0.0f;
            }
            row_tree<M, TB_FMT_SIGN1, false>(p0, p1);
            if ((lane & 15) == 0) {
                float *ps = part_s + ((size_t)(lq * I + s) * 4 + (lane >> 4)) * M;
#pragma unroll
                for (int m = 0; m < M; ++m)
                    ps[m] = p0[m];
            }
        }
    }
    if constexpr (!ISUM) {
        __syncthreads();
        for (int t = tid; t < nq * 4 * M; t += kThreads) {
            const int lq = t / (4 * M), r = (t / M) % 4, m = t % M;
            const float *ps = part_s + ((size_t)lq * I * 4 + r) * M + m;
            float y = 0.0f;
            for (int s = 0; s < I; ++s)
                y += ps[(size_t)s * 4 * M];
            a.out[(size_t)m * n + (tA + lq) * 4 + r] = y;
        }
    }
}

}  // namespace tblut

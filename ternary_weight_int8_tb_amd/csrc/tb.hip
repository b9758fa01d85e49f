// tb.hip -- HIP kernels and C ABI of libtb.so: ternary-weight int8 FFN decode for gfx950.
//
// The path, after "perf(bonsai): decode and small packed batches read the FFN from a
// ternary copy through a dp4a GEMV" (sparkinfer PR #1154, Summary and commit message):
//   1. the activation is rotated (block Hadamard) and quantised to int8 once, and both gate
//      and up read that copy (rotquant_kernel, or inside the gate/up launch: stage_rotate);
//   2. an integer dot-product GEMV streams the stored ternary blocks, stages the int8
//      activation once per workgroup, folds each block's scale into its integer sum, and
//      reduces with a lane shuffle tree (gemv_ring_kernel, gemv_sliced_kernel);
//   3. packed steps of up to 8 rows give every row the bytes it gets alone: each row's lane
//      walk, block fold and reduction tree do not depend on the row count M (and the
//      *_batch calls carry that to 32 rows).
//
// gfx950 mapping (the pages' sm_120 design is prior art; this is the CDNA4 one):
//   * wave64. A wave covers 4 weight rows x 16 "chunk lanes". A chunk is 16 bytes of codes:
//     64 ternary weights (half a block) or 128 sign weights (one block). In each step the
//     16 lanes of a row read 256 contiguous bytes: coalesced 16-byte non-temporal loads.
//   * Streaming (gemv_ring_kernel): one workgroup of 16 waves per CU stages the int8
//     activation once (or rotates the fp32 input itself, for a few rows); each CU owns an
//     equal share of the row tiles, and its waves take (tile, step) items from an LDS
//     counter, loads running one (gate/up) or two (one matrix) items ahead in a register
//     ring. Each step's partial sums meet in LDS and are added in step order.
//   * 2-bit decode with v_perm_b32 (9 VALU ops per 16 weights, shared by all M rows),
//     v_dot4c_i32_i8 against the LDS-staged transposed activation, one DPP add to join the
//     two half-block sums, an fp32 term per block, a fixed DPP tree per row and step, and
//     the step partials summed in step order (tb_device.h).
//   * With M <= 32 rows this is not a dense contraction: the roof is HBM. From M = 5 on
//     gate/up (both formats), and from M = 6 (ternary) or 7 (sign) on the single GEMV, the
//     integer dot products go to v_mfma_i32_16x16x64_i8, where that measures faster:
//     gemv_mfma_pack_kernel (two blocks per MFMA) up to 8 rows, gemv_mfma_kernel (16-row
//     tiles) for batches of 9 to 16 rows, and for ternary gate/up of 17 to 32 rows in one
//     launch (two 16-column groups, k staged in two phases). The block-sum export follows the gate/up
//     threshold, so it runs the matrix-core integer core at every M where production does.
//   * The down stage can also run split over k (tb_ffn_down_split, from 4 rows where it
//     measures faster): each workgroup of gemv_mfma_pack_kernel<..., KS> takes one step of
//     one row group, rotates its own blocks of h, and writes step partials that
//     split_fold_kernel adds in step order, so the results are the same bits. Batches of
//     9 to 32 rows (tb_ffn_down_split_batch) split the same way on gemv_mfma_kernel<..., KS>,
//     whose B operands hold 16 rows, or 32 in two column groups sharing each decoded weight
//     operand (ternary), so the down weights are read once per batch.
//   * The streaming kernels take their leading arguments as scalars that the build
//     preloads into SGPRs, so a launch's first loads wait for no argument fetch.
//   * 1-bit weights in the row-interleaved layout take a lookup-table GEMV (tb_lut.h).
//   * No floating-point atomics.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "tb.h"
#include "tb_device.h"
#include "tb_layers.h"
#include "tb_lut.h"

// Device scratch of tb_ffn_down_noalloc: rotquant(h) and its block scales, for callers that
// cannot allocate. Each GPU holds its own copy until the process ends. Host code never uses
// this name as an address: the device address comes from hipGetSymbolAddress, per device.
constexpr size_t kNoAllocScratchBytes = TB_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

using namespace tbk;

#ifndef TB_ROT_THREADS
#define TB_ROT_THREADS 256
#endif
// 16 lanes per 128-block; 64, 128 and 256 threads per workgroup measure alike in the
// 64-layer stream, 1024 costs 0.8 µs/layer at M=1
constexpr int kRotThreads = TB_ROT_THREADS;
constexpr int kSlicedThreads = 256;
#ifndef TB_RING_WAVES
#define TB_RING_WAVES 16
#endif
#ifndef TB_RING_DEPTH_TWO
#define TB_RING_DEPTH_TWO 1
#endif
#ifndef TB_RING_DEPTH_ONE
#define TB_RING_DEPTH_ONE 2
#endif
constexpr int kRingWaves = TB_RING_WAVES;
constexpr int kRingThreads = 64 * kRingWaves;
// items in flight per wave: 2 KB of codes either way (a gate/up item holds both
// matrices). At the FFN shapes, 64-layer stream at M=1: 23.05 µs/layer against 23.72
// with 2 and 3 items; also faster at M = 2 … 5 and for sign weights.
constexpr int kRingDepthTwo = TB_RING_DEPTH_TWO;   // gate + up
constexpr int kRingDepthOne = TB_RING_DEPTH_ONE;   // one matrix
#ifndef TB_MFMA_DEPTH
#define TB_MFMA_DEPTH 1
#endif
// items in flight per wave in the MFMA kernel (measured at M = 8: ternary gate/up 17.4 µs
// at depth 1 against 19.7 at depth 2, one matrix 18.9 against 20.2; sign gate/up, which
// fits 12 waves only at depth 1, 17.3-17.8 there against 19.8-20.8 at depth 2 on 8 waves)
constexpr int kMfmaDepth = TB_MFMA_DEPTH;
// Activation units staged per thread and round by the matrix-core kernels (16 bytes per
// ternary unit, 32 per sign unit): one round covers M=8 at k = 17408, so every staging load
// is in flight at once. 64-layer stream at M=8, µs/layer with 4 / 6 / 9 / 12 ternary units:
// 36.81-36.88 / 36.89 / 36.45 / 36.08 (no spills at 12: 96 registers).
#ifndef TB_MFMA_STAGE_TERN
#define TB_MFMA_STAGE_TERN 12
#endif
#ifndef TB_MFMA_STAGE_SIGN
#define TB_MFMA_STAGE_SIGN 6
#endif
#ifndef TB_STAGE_FIRST
#define TB_STAGE_FIRST 0
#endif
#ifndef TB_PACK_DEPTH
#define TB_PACK_DEPTH 1
#endif
// items in flight per wave in gemv_mfma_pack_kernel
constexpr int kPackDepth = TB_PACK_DEPTH;
#ifndef TB_PACK_SIGN_WAVES
#define TB_PACK_SIGN_WAVES 12
#endif
// M from which a GEMV runs on the matrix cores, per weight format, for gate/up and for one
// matrix (tb_gemv_ternary, the down GEMV). The MFMA kernel takes about the same time for
// every M, the dot-product kernel grows with M; the crossings measured at the FFN shapes
// (hidden 5120, inter 17408): ternary gate/up 17.3 µs against about 18 at M = 5 (at M = 4
// the dot-product kernel is 0.5-1 µs faster), ternary down (with the rotation of h) 17.8
// against 18.6 at M = 6, sign down 18.6 against 19.3 at M = 7, sign gate/up 17.1-17.4
// against 18.2-19.7 at M = 5 (a tie at M = 4).
// matrix-core GEMV with two blocks per MFMA for M <= 8 (gemv_mfma_pack_kernel)
#ifndef TB_MFMA_PACK
#define TB_MFMA_PACK 1
#endif
#ifndef TB_MFMA_MIN_ROWS_TERN
#define TB_MFMA_MIN_ROWS_TERN 5
#endif
#ifndef TB_MFMA_MIN_ROWS_TERN_ONE
#define TB_MFMA_MIN_ROWS_TERN_ONE 6
#endif
#ifndef TB_MFMA_MIN_ROWS_SIGN
#define TB_MFMA_MIN_ROWS_SIGN 5
#endif
#ifndef TB_MFMA_MIN_ROWS_SIGN_ONE
#define TB_MFMA_MIN_ROWS_SIGN_ONE 7
#endif
// When tb_ffn_down_split takes the split over k (otherwise tb_ffn_down's route): from
// TB_SPLIT_MIN_ROWS rows while the unsplit GEMV runs on the dot-product kernel, and on the
// matrix cores only for k >= TB_SPLIT_MIN_K, where the unsplit kernel stages M * k codes in
// every CU. µs per call, unsplit against split, ternary: 5120 x 17408 M=2 10.66 / 12.64, M=4
// 13.88 / 12.94, M=6 16.36 / 13.83, M=8 17.33 / 14.52 (sign M=8 18.49 / 15.88); 9216 x 5120
// M=4 11.09 / 10.28, M=8 10.82 / 11.43; 5120 x 4096 M=4 8.55 / 8.52, M=8 9.06 / 9.60.
#ifndef TB_SPLIT_MIN_ROWS
#define TB_SPLIT_MIN_ROWS 4
#endif
#ifndef TB_SPLIT_MIN_K
#define TB_SPLIT_MIN_K 8192
#endif
constexpr int mfma_min_rows(bool ternary, bool gateup)
{
    return ternary ? (gateup ? TB_MFMA_MIN_ROWS_TERN : TB_MFMA_MIN_ROWS_TERN_ONE)
                   : (gateup ? TB_MFMA_MIN_ROWS_SIGN : TB_MFMA_MIN_ROWS_SIGN_ONE);
}
typedef int v4i __attribute__((ext_vector_type(4)));

enum Mode { kModeY = 0, kModeGateUp = 1, kModeIsum = 2 };

__global__ __launch_bounds__(kRotThreads) void rotquant_kernel(const float *__restrict__ x,
                                                               long nblocks,
                                                               int8_t *__restrict__ q,
                                                               float *__restrict__ dq, float unit)
{
    const long blk = (long)blockIdx.x * (kRotThreads / 16) + (threadIdx.x >> 4);
    if (blk >= nblocks)
        return;  // the whole 16-lane group leaves together; its shuffles stay inside it
    rotquant16<false>(x + blk * kBlock, q + blk * kBlock, dq + blk, threadIdx.x & 15, unit);
}

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
    int slice_chunks;        // LDS slots per pass (sliced kernel)
    uint32_t codes_bytes;    // per matrix, < 2^31 (buffer addressing)
    uint32_t scales_bytes;
    // fp32 input rotated in the kernel (gemv_ring_kernel with ROTX): x [M][k]; workgroup 0
    // writes its codes and block terms to qx [M][k] and dqx [M][k/128]
    const float *x;
    int8_t *qx;
    float *dqx;
    float unit;              // fp32(1 / (127 sqrt(128)))
    // down stage split over k (gemv_mfma_pack_kernel and gemv_mfma_kernel with KS): row
    // groups, and the step partials it writes, part[s][m][row] with part_rows rows m per
    // step (x holds h; qx, dqx receive rotquant(h))
    int groups;
    float *part;
    int part_rows;
    int act_rows;            // rows of h (gemv_mfma_kernel with KS: 1 <= act_rows <= M)
};

// The arguments of a streaming kernel from its leading scalar arguments (preloaded into
// SGPRs) and the rest in GemvArgs: p0, p1 the (first) matrix; gate/up: p2, p3 the up matrix
// and p4 the activation; one matrix: p2 the activation and p3 its block terms. The
// activation is q, or x for a kernel that rotates it. Buffer sizes follow from n and k.
template <int FMT, bool TWO>
__device__ __forceinline__ GemvArgs with_leading_args(const GemvArgs &in, const void *p0,
                                                      const void *p1, const void *p2,
                                                      const void *p3, const void *p4, int pn, int pk)
{
    GemvArgs a = in;
    a.codes0 = static_cast<const uint8_t *>(p0);
    a.scales0 = static_cast<const uint16_t *>(p1);
    if (TWO) {
        a.codes1 = static_cast<const uint8_t *>(p2);
        a.scales1 = static_cast<const uint16_t *>(p3);
    }
    a.q = static_cast<const int8_t *>(TWO ? p4 : p2);
    a.x = static_cast<const float *>(TWO ? p4 : p2);
    if (!TWO)
        a.dq = static_cast<const float *>(p3);
    a.n = pn;
    a.k = pk;
    a.codes_bytes = (uint32_t)((size_t)pn * (size_t)pk / (FMT == TB_FMT_TERNARY2 ? 4u : 8u));
    a.scales_bytes = (uint32_t)(((size_t)pn * (size_t)(pk / kBlock) * 2u + 3u) & ~(size_t)3);
    return a;
}

// Writes the results of one finished row (lane 0 of the row's 16 lanes).
template <int M, int MODE>
__device__ __forceinline__ void store_row(const GemvArgs &a, int row, const float (&acc0)[M],
                                          const float (&acc1)[M])
{
#pragma unroll
    for (int m = 0; m < M; ++m)
        a.out[(size_t)m * a.n + row] = MODE == kModeGateUp ? silu_gate(acc0[m], acc1[m]) : acc0[m];
}

// ------------------------------------------------------------------------------------
// Stages the int8 activation q[M][k] into the step-major LDS layout and the block terms
// dq as [b][m] (zero padded by one step of blocks, so ragged lanes read zeros). For the
// sign format it also adds sum(q) per block into qsum_s (LDS integer adds: exact in any
// order; qsum_s starts at zero). The loads of the first round go out before `prologue`
// (the weight stream's first loads) and their LDS stores after it, so the activation is
// not queued behind the weights: one vmcnt counts a wave's loads in issue order.
// ------------------------------------------------------------------------------------
template <int M, int FMT, int MODE, int NTHREADS, bool MFMA_LAYOUT, class Prologue>
__device__ __forceinline__ void stage_activation(const GemvArgs &a, uint8_t *act, float *dq_s,
                                                 int *qsum_s, Prologue &&prologue)
{
    constexpr int kBlocksPerStep = kChunkLanes / Fmt<FMT>::kChunksPerBlock;
    constexpr int kStageRound = MFMA_LAYOUT ? (FMT == TB_FMT_TERNARY2 ? TB_MFMA_STAGE_TERN : TB_MFMA_STAGE_SIGN) : 4;
    constexpr int kTermRound = 2;
    const int tid = threadIdx.x, k = a.k, nb = k / kBlock;
    const int per_row = (k / Fmt<FMT>::kWeightsPerChunk) * 4, units = M * per_row;
    const int nterm = (nb + kBlocksPerStep) * M;
    // Unit numbering: row-major (m, g) for the step-major layout; (g, m) for the MFMA
    // layout, whose slot of unit (g, m) is g * M + m, so that consecutive threads store
    // consecutive 16-byte slots (the other order makes 32-way LDS bank conflicts).
    auto split = [&](int unit, int &m, int &g) {
        if constexpr (MFMA_LAYOUT) {
            m = unit % M;
            g = unit / M;
        } else {
            unit_split<M>(unit, per_row, m, g);
        }
    };
    auto unit_load = [&](StageUnit<FMT> &u, int unit) {
        int m, g;
        split(unit, m, g);
        stage_unit_load_step<M, FMT, false>(u, a.q, k, m, g);
    };
    auto unit_store = [&](const StageUnit<FMT> &u, int unit) {
        int m, g;
        split(unit, m, g);
        if constexpr (MFMA_LAYOUT)
            stage_unit_store_mfma<M, FMT>(u, act, m, g);
        else
            stage_unit_store_step<M, FMT>(u, act, m, g);
        if (FMT == TB_FMT_SIGN1) {
            const uint32_t w[8] = {u.lo.x, u.lo.y, u.lo.z, u.lo.w, u.hi.x, u.hi.y, u.hi.z, u.hi.w};
            int sum = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sum = dot4(w[e], 0x01010101u, sum);
            atomicAdd(qsum_s + (g >> 2) * M + m, sum);
        }
    };
    // Beyond the first round (a large M * k), in rounds of kStageRound units per thread,
    // before the prologue: the compiler waits for every outstanding load at the exit of a
    // loop that loads, so such a loop between the prologue and the barrier would hold the
    // barrier until the whole weight prologue has arrived.
    for (int u0 = tid + kStageRound * NTHREADS; u0 - tid < units; u0 += kStageRound * NTHREADS) {
        StageUnit<FMT> more[kStageRound];
#pragma unroll
        for (int r = 0; r < kStageRound; ++r)
            if (u0 + r * NTHREADS < units)
                unit_load(more[r], u0 + r * NTHREADS);
#pragma unroll
        for (int r = 0; r < kStageRound; ++r)
            if (u0 + r * NTHREADS < units)
                unit_store(more[r], u0 + r * NTHREADS);
    }
    for (int i = tid + kTermRound * NTHREADS; i < nterm; i += NTHREADS) {
        const int b = i / M, m = i % M;
        dq_s[i] = (MODE != kModeIsum && b < nb) ? a.dq[m * nb + b] : 0.0f;
    }
    // the first round: loads, the prologue, stores (straight-line code, exact waits)
    StageUnit<FMT> su[kStageRound];
#pragma unroll
    for (int r = 0; r < kStageRound; ++r)
        if (tid + r * NTHREADS < units)
            unit_load(su[r], tid + r * NTHREADS);
    float dv[kTermRound];
#pragma unroll
    for (int r = 0; r < kTermRound; ++r) {
        const int i = tid + r * NTHREADS, b = i / M, m = i % M;
        dv[r] = (MODE != kModeIsum && i < nterm && b < nb) ? a.dq[m * nb + b] : 0.0f;
    }
#if !TB_STAGE_FIRST
    prologue();
#endif
#pragma unroll
    for (int r = 0; r < kStageRound; ++r)
        if (tid + r * NTHREADS < units)
            unit_store(su[r], tid + r * NTHREADS);
#pragma unroll
    for (int r = 0; r < kTermRound; ++r)
        if (tid + r * NTHREADS < nterm)
            dq_s[tid + r * NTHREADS] = dv[r];
#if TB_STAGE_FIRST
    prologue();
#endif
}

// ------------------------------------------------------------------------------------
// Staging from the fp32 input x[M][k]: every workgroup rotates and quantises all M k/128
// blocks itself, one 16-lane group per block, with rotquant_regs (the arithmetic of
// rotquant_kernel, so codes and terms are bit-identical to a separate rotate-quantise
// call), and stores the codes straight into the step-major layout, the block terms into
// dq_s (zero padded by one step of blocks) and, sign format, the code sums into qsum_s.
// Workgroup 0 also writes the codes and terms to qx and dqx. The x loads of the first
// kXRounds rounds go out before `prologue` (the weight stream's first loads), so they
// are not queued behind them; later rounds load after it.
// ------------------------------------------------------------------------------------
template <int M, int FMT, int NTHREADS, class Prologue>
__device__ __forceinline__ void stage_rotate(const GemvArgs &a, uint8_t *act, float *dq_s,
                                             int *qsum_s, Prologue &&prologue)
{
    constexpr int kGroups = NTHREADS / 16, kXRounds = 2;
    constexpr int kBlocksPerStep = kChunkLanes / Fmt<FMT>::kChunksPerBlock;
    const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
    const int k = a.k, nb = k / kBlock, Z = M * nb;
    const bool out = blockIdx.x == 0;
    auto load = [&](float (&v)[8], int z) {
        const float *src = a.x + (size_t)(z / nb) * k + (size_t)(z % nb) * kBlock + l16 * 8;
        const float4 lo = *reinterpret_cast<const float4 *>(src);
        const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    };
    auto block = [&](float (&v)[8], int z) {
        const int m = z / nb, b = z % nb;
        uint32_t pk[2];
        float dq;
        int qsum;
        rotquant_regs(v, l16, a.unit, pk, dq, qsum);
        store_block_step<M, FMT>(act, m, b, l16, pk);
        if (l16 == 0) {
            dq_s[b * M + m] = dq;
            if (FMT == TB_FMT_SIGN1)
                qsum_s[b * M + m] = qsum;
        }
        if (out) {
            *reinterpret_cast<uint2 *>(a.qx + (size_t)m * k + (size_t)b * kBlock + l16 * 8) =
                make_uint2(pk[0], pk[1]);
            if (l16 == 0)
                a.dqx[m * nb + b] = dq;
        }
    };
    // (a 16-lane group takes or skips a block as a whole: its row shuffles stay inside it)
    float xv[kXRounds][8];
#pragma unroll
    for (int r = 0; r < kXRounds; ++r)
        if (grp + r * kGroups < Z)
            load(xv[r], grp + r * kGroups);
    for (int i = Z + tid; i < (nb + kBlocksPerStep) * M; i += NTHREADS) {
        dq_s[i] = 0.0f;
        if (FMT == TB_FMT_SIGN1)
            qsum_s[i] = 0;
    }
    prologue();
#pragma unroll
    for (int r = 0; r < kXRounds; ++r)
        if (grp + r * kGroups < Z)
            block(xv[r], grp + r * kGroups);
    for (int z = grp + kXRounds * kGroups; z < Z; z += kGroups) {
        float v[8];
        load(v, z);
        block(v, z);
    }
}

// ------------------------------------------------------------------------------------
// Streaming GEMV: one workgroup per CU, the whole activation staged once in LDS
// (step-major layout).
//   * A row tile is 4 rows; workgroup c owns the contiguous tiles [tA, tB) of a near-equal
//     split of all tiles over the grid, so every CU streams the same bytes.
//   * An item is one step of one tile: in step i, lane cl of a row reads chunk 16 i + cl.
//     The waves of a workgroup share its items through an LDS counter: a wave takes the
//     next item when it refills a ring slot, so waves that the SIMD arbiter serves less
//     often simply take fewer items (the older wave on a SIMD is favoured).
//   * Loads run a few items ahead of the math in a register ring.
// Fold order (the same in every kernel here, and independent of M, of the grid and of
// which wave took which item; so a batched row is bit-identical to the row run alone):
// a step's partial is the fixed 16-lane row tree of the lanes' terms (s * dq) * isum; a
// row's output is the sum of its step partials in step order, starting from +0. The step
// partials meet in LDS.
//
// The loop is written for the VALU budget: at M = 1 one 1 KB wave item needs 52 VALU ops
// of decode and dot products, so the rest is kept to a handful. Rows past n, empty slots
// and ragged chunks use out-of-range buffer offsets, which read zeros.
// ROTX: the activation arrives as fp32 x and each workgroup rotates and quantises it
// itself (stage_rotate), which saves a launch on the decode path.
// ------------------------------------------------------------------------------------
//
// Launch: the leading arguments (the matrices, the activation, n, k, the grid) are
// separate scalars, which the command processor preloads into SGPRs (built with
// -amdgpu-kernarg-preload-count), so the first loads wait for no kernel-argument fetch;
// the rest comes in GemvArgs. With ROTX every wave issues its first weight items (static:
// wave w takes w + 16 d) right behind its x loads, before any barrier; the item counter
// starts after the staging barrier. (Without ROTX the counter hands out every item but the
// first: measured faster there.)
template <int M, int FMT, int MODE, bool ROTX = false>
__global__ __launch_bounds__(kRingThreads) void gemv_ring_kernel(const void *p0, const void *p1,
                                                                 const void *p2, const void *p3,
                                                                 const void *p4, int pn, int pk,
                                                                 int pg, GemvArgs a_in)
{
    GemvArgs a = with_leading_args<FMT, MODE == kModeGateUp>(a_in, p0, p1, p2, p3, p4, pn, pk);
    static_assert(!ROTX || MODE != kModeIsum, "the block-sum export takes int8 input");
    extern __shared__ __align__(16) uint8_t lds[];
    using L = StepLayout<M, FMT>;
    constexpr bool kTwo = MODE == kModeGateUp;
    constexpr int kWpc = Fmt<FMT>::kWeightsPerChunk;
    constexpr int kCpb = Fmt<FMT>::kChunksPerBlock;
    constexpr int kBlocksPerStep = kChunkLanes / kCpb;   // 8 ternary, 16 sign
    // (the block-sum export runs one item deep: it keeps the sign export's registers below
    // the 128 a wave has, where two items spilled from M = 4 on)
    constexpr int kDepth = MODE == kModeIsum ? 1 : kTwo ? kRingDepthTwo : kRingDepthOne;

    const int k = a.k, n = a.n, nb = k / kBlock;
    const int C = k / kWpc;                 // chunks per row
    const int I = (C + kChunkLanes - 1) / kChunkLanes;   // steps per tile
    const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15, rl = lane >> 4;
    const int G = pg, c = blockIdx.x;
    const int T = (n + kRowsPerWave - 1) / kRowsPerWave;
    const int tA = part_lo(T, G, c), tB = part_lo(T, G, c + 1);
    const int J = (tB - tA) * I;            // this workgroup's items
    const uint32_t row_bytes = (uint32_t)C * 16u;

    uint8_t *act = lds;
    // block terms, zero padded by one step of blocks so ragged lanes read zeros
    float *dq_s = reinterpret_cast<float *>(lds + (size_t)I * L::kStepBytes);
    int *qsum_s = reinterpret_cast<int *>(dq_s + (size_t)(nb + kBlocksPerStep) * M);
    int *ctr_s = qsum_s + (FMT == TB_FMT_SIGN1 ? (nb + kBlocksPerStep) * M : 0);   // item counter
    // step partials [item][row in tile][m][gate, up] (gate only for one matrix)
    constexpr int kParts = kTwo ? 2 : 1;
    float *part_s = reinterpret_cast<float *>(ctr_s + 4);

    const __amdgpu_buffer_rsrc_t rout =
        MODE == kModeIsum ? buffer_rsrc(a.isum, (uint32_t)((size_t)M * n * nb * 4))
                          : buffer_rsrc(a.out, (uint32_t)((size_t)M * n * 4));
    const __amdgpu_buffer_rsrc_t rc0 = buffer_rsrc(a.codes0, a.codes_bytes);
    const __amdgpu_buffer_rsrc_t rsc0 = buffer_rsrc(a.scales0, a.scales_bytes);
    const __amdgpu_buffer_rsrc_t rc1 = buffer_rsrc(kTwo ? a.codes1 : a.codes0, a.codes_bytes);
    const __amdgpu_buffer_rsrc_t rsc1 = buffer_rsrc(kTwo ? a.scales1 : a.scales0, a.scales_bytes);

    if (!ROTX) {
        if (tid == 0)
            *ctr_s = kRingWaves;   // wave w starts with item w
        if (FMT == TB_FMT_SIGN1)   // the staging adds code sums into qsum_s
            for (int i = tid; i < (nb + kBlocksPerStep) * M; i += kRingThreads)
                qsum_s[i] = 0;
        __syncthreads();
    }

    // ---- issue side ------------------------------------------------------------------
    // The wave's items increase, so (tile, step) follow by carrying the step over.
    // Lanes whose chunk is past C in the last step of a row (ragged k) read zeros.
    const uint32_t ragged = (C % kChunkLanes != 0 && cl >= C % kChunkLanes) ? kOutOfRange : 0u;
    int gidx = 0, gtile = 0, gstep = 0;   // the wave's last taken item and its (tile, step)
    auto advance_to = [&](int idx) {
        gstep += idx - gidx;
        gidx = idx;
        while (gstep >= I) {
            gstep -= I;
            ++gtile;
        }
    };
    uint4 rb0[kDepth], rb1[kDepth];
    // scales travel as 32-bit values: 16-bit ring entries would be packed in pairs, and
    // packing waits for the loads
    uint32_t rs0[kDepth], rs1[kDepth];
    int rit[kDepth];   // the slot's item as tile << 16 | step, or -1
    int pending = tid >> 6;   // the next item, taken one issue ahead (LDS add in flight)
    // Offsets split into a per-lane part (row in tile, chunk lane) and a wave-uniform part
    // (tile, step) passed as the buffer soffset, so an issue costs almost no VALU. The
    // uniform part of a scale offset is a multiple of 4, so aligning the lane part to the
    // 4-byte word gives the word of (row, block).
    const uint32_t lane_off = (uint32_t)rl * row_bytes + (uint32_t)cl * 16u;
    const uint32_t lane_soff = (((uint32_t)rl * (uint32_t)nb + (uint32_t)(cl / kCpb)) * 2u) & ~3u;
    auto issue = [&](uint4 &w0, uint4 &w1, uint32_t &s0, uint32_t &s1, int &it, bool take) {
        const int idx = __builtin_amdgcn_readfirstlane(pending);
        uint32_t off = kOutOfRange, soff = kOutOfRange;
        int so = 0, sso = 0;
        it = -1;
        if (idx < J) {
            advance_to(idx);
            it = gtile << 16 | gstep;
            const int row0 = (tA + gtile) * kRowsPerWave;
            so = row0 * (int)row_bytes + gstep * 256;
            sso = (row0 * nb + gstep * kBlocksPerStep) * 2;
            const uint32_t extra = gstep == I - 1 ? ragged : 0u;
            off = lane_off | extra;
            soff = lane_soff | extra;
            if (row0 + kRowsPerWave > n && rl >= n - row0) {   // rows past n (last tile)
                off = kOutOfRange;
                soff = kOutOfRange;
            }
            // take the next item now; the add completes while this one streams
            if (take) {
                int v = 0;
                if (lane == 0)
                    v = atomicAdd(ctr_s, 1);
                pending = v;
            }
        }
        w0 = buffer_load16_nt(rc0, off, so);
        s0 = buffer_load_u32(rsc0, soff, sso);
        if (kTwo) {
            w1 = buffer_load16_nt(rc1, off, so);
            s1 = buffer_load_u32(rsc1, soff, sso);
        } else {
            w1 = make_uint4(0, 0, 0, 0);
            s1 = 0;
        }
    };

    // ---- staging (q and the block terms; the ring prologue between loads and stores)
    auto prologue = [&]() {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (ROTX)   // static first items: no counter before the barrier
                pending = (tid >> 6) + kRingWaves * d;
            issue(rb0[d], rb1[d], rs0[d], rs1[d], rit[d], !ROTX);
        }
    };
    if constexpr (ROTX)
        stage_rotate<M, FMT, kRingThreads>(a, act, dq_s, qsum_s, prologue);
    else
        stage_activation<M, FMT, MODE, kRingThreads, false>(a, act, dq_s, qsum_s, prologue);
    if (ROTX && tid == 0)
        *ctr_s = kRingWaves * kDepth;   // the prologue took items w + 16 d
    __syncthreads();
    if (ROTX) {
        int v = 0;
        if (lane == 0)
            v = atomicAdd(ctr_s, 1);
        pending = v;
    }

    // ---- compute side -----------------------------------------------------------------
    const uint8_t *lds_lane = act + cl * 16;
    const int blk_lane = cl / kCpb;                 // block of this lane within a step
    auto consume = [&](const uint4 &w0, const uint4 &w1, uint32_t sw0, uint32_t sw1, int it) {
        const int tile = it >> 16, step = it & 0xffff;
        const uint32_t row = (uint32_t)((tA + tile) * kRowsPerWave + rl);
        const int blk = step * kBlocksPerStep + blk_lane;
        int is0[M], is1[M];
        chunk_sums_step<M, FMT, kTwo>(w0, w1, lds_lane + (size_t)step * L::kStepBytes, is0, is1);
        const int *cqs = qsum_s + blk * M;
        if (MODE == kModeIsum) {
            // the export writes every valid block once (even lane of a ternary pair)
            const bool wr = row < (uint32_t)n && step * kChunkLanes + cl < C && (kCpb == 1 || !(cl & 1));
            const uint32_t o = (row * (uint32_t)nb + (uint32_t)blk) * 4u;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int v = FMT == TB_FMT_SIGN1 ? 2 * is0[m] - cqs[m] : is0[m];
                __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, rout, wr ? o : kOutOfRange,
                                                      m * n * nb * 4, 0);
            }
            return;
        }
        // the scale is the half of the loaded word at bit 16 * (block index parity)
        const uint32_t cshift = ((row * (uint32_t)nb + (uint32_t)blk_lane) & 1u) * 16u;
        const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(sw0, cshift, 16));
        const float s1 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(sw1, cshift, 16));
        const float *cdq = dq_s + blk * M;
        float p0[M], p1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            int v0 = is0[m], v1 = is1[m];
            if (FMT == TB_FMT_SIGN1) {
                v0 = 2 * v0 - cqs[m];
                v1 = 2 * v1 - cqs[m];
            }
            const float dqv = cdq[m];
            p0[m] = (s0 * dqv) * (float)v0;
            p1[m] = kTwo ? (s1 * dqv) * (float)v1 : 0.0f;
        }
        row_tree<M, FMT, kTwo>(p0, p1);
        if (cl == 0) {
            float *ps = part_s + ((size_t)((tile * I + step) * kRowsPerWave + rl) * M) * kParts;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                ps[kParts * m] = p0[m];
                if (kTwo)
                    ps[kParts * m + 1] = p1[m];
            }
        }
    };
    for (;;) {
        bool any = false;
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            // Consume the slot first, then refill it: the refill reuses the slot's
            // registers (no copy at the loop latch, which would wait for every load), and
            // the scheduling barrier keeps consume/refill interleaved slot by slot.
            if (rit[d] >= 0) {
                consume(rb0[d], rb1[d], rs0[d], rs1[d], rit[d]);
                any = true;
            }
            issue(rb0[d], rb1[d], rs0[d], rs1[d], rit[d], true);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!any)
            break;
    }
    if (MODE == kModeIsum)
        return;

    // ---- every row: its step partials in step order, from +0 ------------------------
    __syncthreads();
    const int ntl = tB - tA;
    for (int i = tid; i < ntl * kRowsPerWave * M; i += kRingThreads) {
        const int tl = i / (kRowsPerWave * M), r = (i / M) % kRowsPerWave, m = i % M;
        const int row = (tA + tl) * kRowsPerWave + r;
        if (row >= n)
            continue;
        const float *ps = part_s + ((size_t)(tl * I * kRowsPerWave + r) * M + m) * kParts;
        float g = 0.0f, u = 0.0f;
        for (int s = 0; s < I; ++s) {
            g += ps[(size_t)s * kRowsPerWave * M * kParts];
            if (kTwo)
                u += ps[(size_t)s * kRowsPerWave * M * kParts + 1];
        }
        a.out[(size_t)m * n + row] = kTwo ? silu_gate(g, u) : g;
    }
}

// The workgroups of a split over k, G row groups x Ik steps. Ternary: in step-major order
// e = s * G + g, dealt to the XCDs in contiguous ranges: the dispatcher sends consecutive
// workgroup indices to consecutive XCDs, so workgroup b takes e = (b % 8) * per + b / 8.
// The row groups of one step then share one XCD's L2 for that step's h, and the steps that
// share a scale line mostly land on one or two XCDs. The grid is rounded up to a multiple
// of 8; the padding workgroups return at once. Measured (down stage at 5120 x 17408, us per
// call): ternary m = 4 13.40 -> 12.99, 8 14.55 -> 14.37, 16 19.68 -> 19.43, 32 30.86 ->
// 30.34; sign m = 8 15.79 -> 16.03, so sign keeps the row-group-major order b = g Ik + s.
constexpr int kXcds = 8;
__host__ __device__ constexpr bool split_xcd(int fmt) { return fmt == TB_FMT_TERNARY2; }
__host__ __device__ constexpr int split_grid(int nwg, int fmt)
{
    return split_xcd(fmt) ? (nwg + kXcds - 1) / kXcds * kXcds : nwg;
}
template <int FMT>
__device__ __forceinline__ bool split_index(int G, int Ik, int &g, int &s)
{
    const int nwg = G * Ik, b = (int)blockIdx.x;
    if constexpr (split_xcd(FMT)) {
        const int per = (nwg + kXcds - 1) / kXcds;
        const int e = (b % kXcds) * per + b / kXcds;
        if (e >= nwg)
            return false;
        s = e / G;
        g = e - s * G;
    } else {
        if (b >= nwg)
            return false;
        g = b / Ik;
        s = b - g * Ik;
    }
    return true;
}

// Threads per workgroup of gemv_mfma_kernel: 16 waves for ternary; 12 for sign, whose
// 16-block steps need 156-160 registers, more than the 128 a wave has at 16 waves per CU
// (sign down at M=8: 17.7-17.8 µs at 12 waves against 18.9-19.1 at 8). With two 16-column
// groups (M > 16) each wave holds twice the sums and trees: 12 and 8 waves.
__host__ __device__ constexpr int mfma_threads(int fmt, int m = 16)
{
    return fmt == TB_FMT_TERNARY2 ? (m > 16 ? 768 : 1024) : (m > 16 ? 512 : 768);
}
// Threads per workgroup of gemv_mfma_pack_kernel.
#ifndef TB_PACK_TERN_WAVES
#define TB_PACK_TERN_WAVES 16
#endif
__host__ __device__ constexpr int pack_threads(int fmt)
{
    return fmt == TB_FMT_TERNARY2 ? 64 * TB_PACK_TERN_WAVES : 64 * TB_PACK_SIGN_WAVES;
}

// ------------------------------------------------------------------------------------
// Batched streaming GEMV on the matrix cores (ternary and sign weights, M >= 5 to 7 rows).
// With M rows the dot products cost M VALU instructions per 4 weights and lane; here
// v_mfma_i32_16x16x64_i8 takes them, and the VALU keeps the decode and the fold.
//   * Workgroup c owns the rows of the same 4-row tiles [tA, tB) as in gemv_ring_kernel
//     and covers them with 16-row tiles; rows past its range read zeros and are not written.
//   * An item is one step (256 code bytes per row: 8 ternary or 16 sign blocks) of one
//     16-row tile and one matrix. Lane (i, g) = (lane % 16, lane / 16) loads 16 contiguous
//     code bytes of row i per load (the 4 lanes of a row read 64 bytes); lane swaps
//     (v_permlane32_swap, and for sign v_permlane16_swap) then trade code words between
//     the lane groups, so that for each block the four groups hold 32 of its weights each.
//     Per block, two decoded 16-byte groups (ternary: two code words; sign: 0/1 bytes of
//     one 32-bit word, isum = 2 D - sum(q)) are the A operands of two MFMAs;
//     the B operands are the matching transposed 16-byte activation groups (column j =
//     activation row j), so the two MFMAs leave the block's exact integer sums in D: lane
//     l holds rows 4 (l / 16) + r, r = 0..3, of activation row l % 16. The activation is
//     staged as [step][chunk][code word][row] (sign: [step][chunk][word][half][row]) so
//     that the 16 lanes of a B operand read consecutive 16-byte slots; the step-major
//     layout of the other kernels has the rows 256 bytes apart, and its 8-way bank
//     conflicts made this kernel slower than the VALU one.
//   * The block term (s * dq) * isum, the step tree over the step's blocks, and the step
//     sum in step order from +0 are those of the other kernels (row_tree reads lane L - off,
//     so lane 0 of a row ends with ((t0 + t7) + (t6 + t5)) + ((t4 + t3) + (t2 + t1)) over
//     the block terms t, and the same pattern over 16 blocks for sign), so every row is
//     bit-identical to the row computed alone.
//   * The weight loads carry no non-temporal hint: the two 64-byte halves of a row's line
//     come from neighbouring loads, and with the hint the second half was fetched again.
//   * A block's scales reach the fold lanes with ds_bpermute from the lanes that loaded
//     them (the blocks of row i that the lane's code load covers; nb must be a multiple
//     of 2 (ternary) or 4 (sign)).
//   * Sign runs 12 waves per CU: its 16-block steps need more than the 128 registers a
//     wave has at 16.
// ------------------------------------------------------------------------------------
template <int M, int FMT, int MODE, bool KS = false, bool KP = false>
__global__ __launch_bounds__(mfma_threads(FMT, M)) void gemv_mfma_kernel(GemvArgs a)
{
    static_assert(M >= 1 && M <= 32, "one or two 16-column B operands");
    static_assert(M <= 16 || KS || KP, "two column groups stage one step, or k in two phases");
    static_assert(!KS || MODE == kModeY, "the split over k is the down stage");
    static_assert(!KP || (!KS && MODE == kModeGateUp && FMT == TB_FMT_TERNARY2),
                  "k in two phases: ternary gate/up");
    extern __shared__ __align__(16) uint8_t lds[];
    using L = StepLayout<M, FMT>;
    constexpr bool kTern = FMT == TB_FMT_TERNARY2;
    constexpr bool kTwo = MODE == kModeGateUp;
    constexpr int kParts = kTwo ? 2 : 1;
    constexpr int kMatShift = kTwo ? 1 : 0;   // gate/up: item = ((tile, step), matrix)
    constexpr int kBps = kTern ? 8 : 16;      // blocks per step (256 code bytes per row)
    constexpr int kBpl = kBps / 4;            // blocks per 16-byte load of the 4 lanes of a row
    constexpr int kDepth = kMfmaDepth;
    constexpr int kThreads = mfma_threads(FMT, M), kWaves = kThreads / 64;
    constexpr bool kIsum = MODE == kModeIsum;
    constexpr int kCG = (M + 15) / 16;   // 16-column groups of D (activation rows 16 cg + i)

    const int k = a.k, n = a.n, nb = k / kBlock;
    const int C = k / Fmt<FMT>::kWeightsPerChunk, Ik = (C + kChunkLanes - 1) / kChunkLanes;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    // KS: workgroup (g, s) of a.groups row groups x Ik steps covers step s of group g;
    // otherwise workgroup c covers all steps of share c of the grid
    const int G = KS ? a.groups : (int)gridDim.x;
    int c = (int)blockIdx.x, s0 = 0;   // s0: the step of KS items
    if (KS && !split_index<FMT>(G, Ik, c, s0))
        return;
    // KP: the steps in two phases, [0, Sp) then [Sp, Ik), each staged in turn; a row's step
    // partials of phase 0 are summed (in step order, from +0) into its first slot before
    // phase 1 writes the next slots, so the row's sum keeps the order of the other kernels
    const int Sp = KP ? (Ik + 1) / 2 : Ik;
    int I = KS ? 1 : Sp;                                // steps per tile in this phase
    const int NS = KP ? max(Sp, 1 + Ik - Sp) : I;       // partial slots per row
    int slot0 = 0;                                      // the phase's first slot
    const int nbl = KS ? kBps : nb;                     // blocks of the staged activation
    const int rows = (KS || KP) ? a.act_rows : M;       // live activation rows (<= M)
    const int T = (n + kRowsPerWave - 1) / kRowsPerWave;
    const int R0 = part_lo(T, G, c) * kRowsPerWave;
    const int R1 = min(part_lo(T, G, c + 1) * kRowsPerWave, n);
    const int tiles16 = (R1 - R0 + 15) / 16;
    int J = (tiles16 * I) << kMatShift;                 // this workgroup's items (this phase)
    const uint32_t row_bytes = (uint32_t)C * 16u;

    uint8_t *act = lds;
    float *dq_s = reinterpret_cast<float *>(lds + (size_t)I * L::kStepBytes);
    int *qsum_s = reinterpret_cast<int *>(dq_s + (size_t)(nbl + kBps) * M);
    int *ctr_s = qsum_s + (kTern ? 0 : (nbl + kBps) * M);
    float *part_s = reinterpret_cast<float *>(ctr_s + 4);   // [row - R0][step][m][part]

    const __amdgpu_buffer_rsrc_t rout =
        buffer_rsrc(a.isum, kIsum ? (uint32_t)((size_t)M * n * nb * 4) : 0u);
    if (tid == 0)
        *ctr_s = kWaves;   // wave w starts with item w
    if (!kTern && !KS)
        for (int i = tid; i < (nb + kBps) * M; i += kThreads)
            qsum_s[i] = 0;
    __syncthreads();

    // ---- issue side: as in gemv_ring_kernel, with a per-lane and a wave-uniform offset
    int gidx = 0, gtile = 0, gstep = 0;
    auto advance_to = [&](int idx) {
        gstep += idx - gidx;
        gidx = idx;
        while (gstep >= I) {
            gstep -= I;
            ++gtile;
        }
    };
    // Load q of a step: lane g reads bytes 64 q + 16 g .. + 15 of its row: half g & 1 of
    // block 2 q + (g >> 1) (ternary) or all of block 4 q + g (sign). Its scale load is the
    // word (ternary) or the two words (sign) holding the scales of blocks kBpl g .. of row i.
    const uint32_t lane_off = (uint32_t)li * row_bytes + (uint32_t)lg * 16u;
    const uint32_t lane_soff = ((uint32_t)li * (uint32_t)nb + (uint32_t)(lg * kBpl)) * 2u;
    uint4 rc[kDepth][4];
    u32x2 rs[kDepth];
    int rit[kDepth];   // matrix << 30 | tile << 16 | step, or -1
    int pending = tid >> 6;
    auto issue = [&](int d) {
        const int idx = __builtin_amdgcn_readfirstlane(pending);
        uint32_t off = kOutOfRange, soff = kOutOfRange;
        int so = 0, sso = 0, nbk = 0, mat = 0;
        rit[d] = -1;
        if (idx < J) {
            advance_to(idx >> kMatShift);
            mat = idx & (kTwo ? 1 : 0);
            rit[d] = mat << 30 | gtile << 16 | gstep;
            const int row0 = R0 + gtile * 16;
            const int wstep = s0 + gstep;            // the step in the weight rows
            so = row0 * (int)row_bytes + wstep * 256;
            sso = (row0 * nb + wstep * kBps) * 2;
            nbk = min(kBps, nb - wstep * kBps);   // blocks of this step inside the row
            if (row0 + li < R1) {
                off = lane_off;
                soff = (!kIsum && wstep * kBps + lg * kBpl < nb) ? lane_soff : kOutOfRange;
            }
            int v = 0;
            if (lane == 0)
                v = atomicAdd(ctr_s, 1);
            pending = v;
        }
        // (the descriptors are built per issue from wave-uniform values: arrays of them
        // would live in scratch)
        const __amdgpu_buffer_rsrc_t rcm = buffer_rsrc(mat ? a.codes1 : a.codes0, a.codes_bytes);
        const __amdgpu_buffer_rsrc_t rsm = buffer_rsrc(mat ? a.scales1 : a.scales0, a.scales_bytes);
        // (nbk is a multiple of kBpl: the blocks of one load are all in or all out)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            rc[d][q] = buffer_load16(rcm, q * kBpl < nbk ? off + (uint32_t)q * 64u : kOutOfRange, so);
        if (kTern) {
            rs[d].x = buffer_load_u32(rsm, soff, sso);
            rs[d].y = 0u;
        } else {
            rs[d] = __builtin_amdgcn_raw_buffer_load_b64(rsm, soff, sso, 0);
        }
    };

    // KP: the int8 codes of steps [ps0, ps0 + pI) of rows < act_rows into the matrix-core
    // layout (unit (g, m), g = 4 c + j over the phase's chunks, slot g M + m), the first
    // round's loads before the weight prologue
    auto stage_phase = [&](int ps0, int pI) {
        constexpr int kR = 4;
        const int units = 64 * pI * M;
        auto uload = [&](StageUnit<FMT> &su, int u) {   // (chunks past C: zeros, not read)
            const int m = u % M, g = u / M;
            su.lo = (m < rows && ps0 * 16 + g / 4 < C)
                        ? *reinterpret_cast<const uint4 *>(a.q + (size_t)m * k + (size_t)(ps0 * 64 + g) * 16)
                        : make_uint4(0u, 0u, 0u, 0u);
        };
        StageUnit<FMT> su[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r)
            if (tid + r * kThreads < units)
                uload(su[r], tid + r * kThreads);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(d);
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int u = tid + r * kThreads;
            if (u < units)
                stage_unit_store_mfma<M, FMT>(su[r], act, u % M, u / M);
        }
        for (int u = tid + kR * kThreads; u < units; u += kThreads) {
            StageUnit<FMT> t;
            uload(t, u);
            stage_unit_store_mfma<M, FMT>(t, act, u % M, u / M);
        }
    };
    if constexpr (KS) {
        // h loads of step s0's blocks first (up to kPre rounds), then the weight prologue,
        // then the rotation (as in gemv_mfma_pack_kernel: the two kernels share the LDS slot
        // layout); later rounds load after the prologue
        constexpr int kGroups16 = kThreads / 16;
        constexpr int kRounds = (M * kBps + kGroups16 - 1) / kGroups16;
        constexpr int kPre = kRounds < 6 ? kRounds : 6;
        const int l16 = tid & 15, grp = tid >> 4;
        const int b0 = s0 * kBps, nbs = min(kBps, nb - b0), Z = rows * nbs;
        auto hload = [&](float (&v)[8], int z) {
            const int m = z / nbs, bl = z - m * nbs;
            const float *src = a.x + (size_t)m * k + (size_t)(b0 + bl) * kBlock + l16 * 8;
            const float4 lo = *reinterpret_cast<const float4 *>(src);
            const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        };
        auto hblock = [&](float (&v)[8], int z) {   // (a 16-lane group takes a block whole)
            const int m = z / nbs, bl = z - m * nbs;
            uint32_t pk[2];
            float dq;
            int qsum;
            rotquant_regs(v, l16, a.unit, pk, dq, qsum);
            store_block_mfma<M, FMT>(act, m, bl, l16, pk);
            if (l16 == 0) {
                dq_s[bl * M + m] = dq;
                if (!kTern)
                    qsum_s[bl * M + m] = qsum;
            }
            if (c == 0) {   // row group 0 writes rotquant(h)
                *reinterpret_cast<uint2 *>(a.qx + (size_t)m * k + (size_t)(b0 + bl) * kBlock + l16 * 8) =
                    make_uint2(pk[0], pk[1]);
                if (l16 == 0)
                    a.dqx[(size_t)m * nb + b0 + bl] = dq;
            }
        };
        float hv[kPre][8];
#pragma unroll
        for (int r = 0; r < kPre; ++r)
            if (grp + r * kGroups16 < Z)
                hload(hv[r], grp + r * kGroups16);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(d);
        // block terms [block][m] of the blocks past the step's end read zero (their codes
        // are zero too); rows past act_rows feed only D columns that are never stored
        for (int i = nbs * M + tid; i < 2 * kBps * M; i += kThreads) {
            dq_s[i] = 0.0f;
            if (!kTern)
                qsum_s[i] = 0;
        }
#pragma unroll
        for (int r = 0; r < kPre; ++r)
            if (grp + r * kGroups16 < Z)
                hblock(hv[r], grp + r * kGroups16);
        for (int z = grp + kPre * kGroups16; z < Z; z += kGroups16) {
            float v[8];
            hload(v, z);
            hblock(v, z);
        }
    } else if constexpr (KP) {
        // the block terms of all steps once (zero for rows past act_rows and blocks past
        // k), then phase 0's codes
        for (int i = tid; i < (nb + kBps) * M; i += kThreads) {
            const int b = i / M, m = i - b * M;
            dq_s[i] = (b < nb && m < rows) ? a.dq[(size_t)m * nb + b] : 0.0f;
        }
        stage_phase(0, Sp);
    } else {
        stage_activation<M, FMT, MODE, kThreads, true>(a, act, dq_s, qsum_s, [&]() {
#pragma unroll
            for (int d = 0; d < kDepth; ++d)
                issue(d);
        });
    }
    __syncthreads();

    // ---- compute side
    // activation row of this lane's B and D column in column group cg: 16 cg + li
    int mB[kCG];
#pragma unroll
    for (int cg = 0; cg < kCG; ++cg)
        mB[cg] = 16 * cg + li < M ? 16 * cg + li : M - 1;
    auto consume = [&](int d) {
        const int mat = rit[d] >> 30, tile = (rit[d] >> 16) & 0x3fff, step = rit[d] & 0xffff;
        // The lane groups exchange code words so that each MFMA sees one block.
        //   ternary: after one swap between the lane halves, words x, y of load q hold block
        //   2 q and z, w block 2 q + 1; group g covers weights 64 (g & 1) + 32 (g >> 1) + 0..15
        //   (x, z) and + 16..31 (y, w). B: chunk 2 kb + (g & 1), code words 2 (g >> 1), + 1.
        //   sign: a 4 x 4 transpose of dwords over the lane groups (a swap between the halves,
        //   then between the 16-lane rows): word t of load q holds dword g (weights
        //   32 g .. 32 g + 31) of block 4 q + t. B: chunk kb, dword g, halves 0 and 1.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (kTern) {
                const u32x2 s0 = __builtin_amdgcn_permlane32_swap(rc[d][q].x, rc[d][q].z, false, false);
                const u32x2 s1 = __builtin_amdgcn_permlane32_swap(rc[d][q].y, rc[d][q].w, false, false);
                rc[d][q] = make_uint4(s0.x, s1.x, s0.y, s1.y);
            } else {
                const u32x2 s0 = __builtin_amdgcn_permlane32_swap(rc[d][q].x, rc[d][q].z, false, false);
                const u32x2 s1 = __builtin_amdgcn_permlane32_swap(rc[d][q].y, rc[d][q].w, false, false);
                const u32x2 t0 = __builtin_amdgcn_permlane16_swap(s0.x, s1.x, false, false);
                const u32x2 t1 = __builtin_amdgcn_permlane16_swap(s0.y, s1.y, false, false);
                rc[d][q] = make_uint4(t0.x, t0.y, t1.x, t1.y);
            }
        }
        const uint8_t *sbase = act + (size_t)step * L::kStepBytes +
                               (kTern ? (((lg & 1) * 4 + 2 * (lg >> 1)) * M) * 16 : ((2 * lg) * M) * 16);
        // The step tree in the order row_tree produces (each level adds lane L - off), taken
        // as a balanced tree over the blocks in the order 0, kBps - 1, .., 1:
        // ((t0 + t7) + (t6 + t5)) + ((t4 + t3) + (t2 + t1)) for ternary, the same over 16
        // blocks for sign. lv holds the pending left subtrees per level.
        float lv[kCG][4][4], tot[kCG][4];
        // byte address of this lane's row group for ds_bpermute, made opaque here so the
        // compiler forms the per-block addresses in the loop instead of keeping all of them
        // live across it (which spills)
        int pbase = 16 * lg;
        asm volatile("" : "+v"(pbase));
#pragma unroll
        for (int o = 0; o < kBps; ++o) {
            const int kb = o == 0 ? 0 : kBps - o;
            const int blk = ((KS ? 0 : s0) + step) * kBps + kb;   // its block terms in dq_s
            uint32_t w[8];
            if (kTern) {
                const uint4 cw = rc[d][kb >> 1];
                decode_ternary((kb & 1) ? cw.z : cw.x, w[0], w[1], w[2], w[3]);
                decode_ternary((kb & 1) ? cw.w : cw.y, w[4], w[5], w[6], w[7]);
            } else {
                const uint4 cw = rc[d][kb >> 2];
                const uint32_t dw = (kb & 3) == 0 ? cw.x : (kb & 3) == 1 ? cw.y : (kb & 3) == 2 ? cw.z : cw.w;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    w[j] = (dw >> j) & 0x01010101u;
            }
            const v4i a0 = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            const v4i a1 = {(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            // both formats: a block's B groups are 8 slots of M rows apart
            v4i acc[kCG];
            float dqv[kCG];
            int qs[kCG];
#pragma unroll
            for (int cg = 0; cg < kCG; ++cg) {
                const uint8_t *bp = sbase + (size_t)mB[cg] * 16 + (size_t)kb * 8 * M * 16;
                const v4i b0 = *reinterpret_cast<const v4i *>(bp);
                const v4i b1 = *reinterpret_cast<const v4i *>(bp + M * 16);
                acc[cg] = v4i{0, 0, 0, 0};
                acc[cg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[cg], 0, 0, 0);
                acc[cg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[cg], 0, 0, 0);
                dqv[cg] = dq_s[blk * M + mB[cg]];
                qs[cg] = kTern ? 0 : qsum_s[blk * M + mB[cg]];
            }
            if constexpr (kIsum) {
                // the block-sum export: D's exact sums, before any scale, for the live
                // activation rows of rows inside this workgroup's range
#pragma unroll
                for (int cg = 0; cg < kCG; ++cg) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = R0 + tile * 16 + 4 * lg + r, mr = 16 * cg + li;
                        const bool wr = mr < M && row < R1 && blk < nb;
                        const int v = kTern ? acc[cg][r] : 2 * acc[cg][r] - qs[cg];
                        __builtin_amdgcn_raw_buffer_store_b32(
                            (uint32_t)v, rout, wr ? (uint32_t)(((mr * n + row) * nb + blk) * 4) : kOutOfRange, 0, 0);
                    }
                }
                if (!kTern)
                    __builtin_amdgcn_sched_barrier(0);
                continue;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // the scale of row 4 lg + r and block kb, from the lane that loaded it
                const uint32_t word = (kTern || ((kb >> 1) & 1) == 0) ? rs[d].x : rs[d].y;
                const uint32_t sw = (uint32_t)__builtin_amdgcn_ds_bpermute(
                    pbase + (16 * (kb / kBpl) + r) * 4, (int)word);
                const float sv = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(sw, (kb & 1) * 16, 16));
#pragma unroll
                for (int cg = 0; cg < kCG; ++cg) {
                    const int isum = kTern ? acc[cg][r] : 2 * acc[cg][r] - qs[cg];
                    float v = (sv * dqv[cg]) * (float)isum;
                    bool done = false;
#pragma unroll
                    for (int l = 0; l < 4; ++l) {
                        if (!done) {
                            if ((o >> l) & 1) {
                                v = lv[cg][r][l] + v;
                            } else {
                                lv[cg][r][l] = v;
                                done = true;
                            }
                        }
                    }
                    if (o == kBps - 1)
                        tot[cg][r] = v;
                }
            }
            // sign: one block at a time (hoisting the LDS reads of the 16 blocks of a step
            // spills)
            if (!kTern)
                __builtin_amdgcn_sched_barrier(0);
        }
        if (!kIsum) {
#pragma unroll
            for (int cg = 0; cg < kCG; ++cg) {
                const int mr = 16 * cg + li;
                if (mr < rows) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lrow = tile * 16 + 4 * lg + r;   // row - R0
                        if (R0 + lrow < R1)
                            part_s[((size_t)(lrow * NS + slot0 + step) * M + mr) * kParts + mat] = tot[cg][r];
                    }
                }
            }
        }
    };
    auto run_ring = [&]() {
        for (;;) {
            bool any = false;
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                if (rit[d] >= 0) {
                    consume(d);
                    any = true;
                }
                issue(d);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!any)
                break;
        }
    };
    run_ring();
    if constexpr (KP) {
        __syncthreads();
        // phase 0's partials of each row, in step order from +0, into its first slot
        for (int i = tid; i < (R1 - R0) * rows * kParts; i += kThreads) {
            const int lrow = i / (rows * kParts), rem = i - lrow * rows * kParts;
            float *ps = part_s + ((size_t)lrow * NS * M + rem / kParts) * kParts + rem % kParts;
            float v = 0.0f;
            for (int st = 0; st < Sp; ++st)
                v += ps[(size_t)st * M * kParts];
            ps[0] = v;
        }
        // phase 1: the next steps, the item counter and the issue state from the start
        s0 = Sp;
        I = Ik - Sp;
        J = (tiles16 * I) << kMatShift;
        slot0 = 1;
        gidx = 0;
        gtile = 0;
        gstep = 0;
        pending = tid >> 6;
        if (tid == 0)
            *ctr_s = kWaves;
        __syncthreads();
        stage_phase(Sp, I);
        __syncthreads();
        run_ring();
    }

    if (kIsum)
        return;
    __syncthreads();
    if constexpr (KS) {   // the step partials [s0][m][row], summed by the fold launch
        for (int i = tid; i < (R1 - R0) * rows; i += kThreads) {
            const int lrow = i / rows, m = i - lrow * rows;
            a.part[((size_t)s0 * a.part_rows + m) * n + R0 + lrow] = part_s[(size_t)lrow * M + m];
        }
        return;
    }
    // ---- every row: its step partials in step order, from +0 (KP: phase 0's sum, then
    // phase 1's steps)
    const int NF = KP ? 1 + Ik - Sp : I;
    for (int i = tid; i < (R1 - R0) * rows; i += kThreads) {
        const int lrow = i / rows, m = i - lrow * rows;
        const float *ps = part_s + ((size_t)lrow * NS * M + m) * kParts;
        float g = 0.0f, u = 0.0f;
        for (int st = 0; st < NF; ++st) {
            g += ps[(size_t)st * M * kParts];
            if (kTwo)
                u += ps[(size_t)st * M * kParts + 1];
        }
        a.out[(size_t)m * n + R0 + lrow] = kTwo ? silu_gate(g, u) : g;
    }
}

// ------------------------------------------------------------------------------------
// Batched streaming GEMV on the matrix cores with two blocks per MFMA (2 <= M <= 8 rows).
// The B operand of v_mfma_i32_16x16x64_i8 has 16 columns; with M <= 8 activation rows,
// columns 0..7 carry the rows of one block of a pair and columns 8..15 those of the other.
// The A operand's lane groups split the same way (groups 0, 1: k 0..31, the first block;
// groups 2, 3: k 32..63, the second), and the B lanes of the other block read zeros, so
// after four MFMAs D holds both blocks' exact integer sums for 16 weight rows and M
// activation rows, with no unused column. The fold (block terms and step tree) then costs
// half of what a 16-column D with M live columns would.
//   * Ternary: lane (i, g) loads 16 code bytes of row i per load q, chunk 4 q + g: half g & 1
//     of block 2 q + (g >> 1). That is the pair (2 q, 2 q + 1) split as above, so the code
//     words go to the MFMAs as loaded, decoded by v_perm_b32. The step tree
//     ((t0 + t7) + (t6 + t5)) + ((t4 + t3) + (t2 + t1)) takes the odd blocks' terms from the
//     lane eight columns over (DPP row rotate by 8).
//   * Sign: the pairs are (e, e - 1 mod 16) for even e, the first level of the sign step
//     tree. Lane group g loads the whole block {4 q, 4 q + 2, 4 q - 1, 4 q + 1}[g] per load q;
//     one v_permlane16_swap per dword pair (odd 16-lane rows of the first operand with even
//     rows of the second) leaves every lane 64 weights of each of the load's two pairs:
//     even groups dwords 2, 3 and odd groups dwords 0, 1 of their block.
//   * Block scales: each lane loads the scale word(s) of the blocks its code load covers;
//     a per-wave LDS scratch laid out [block][row] then gives each D lane its four rows'
//     scales in one 8-byte read.
// Rows, items, the ring and the step sum are those of gemv_mfma_kernel, and the fold order
// is the one every kernel here uses, so a batched row is bit-identical to the row alone.
// ------------------------------------------------------------------------------------
// LDS carve-up of gemv_mfma_pack_kernel, shared with the host (16-byte aligned sections):
// the activation (MFMA layout), block terms dq [b][m], code sums (sign), the item counter,
// a zero region read as B by inactive lanes, per-wave scale scratch, then the step partials.
constexpr int kPackZeroBytes = 1024;
// per wave: the scales of one item, [block in step][row in tile] as uint16
__host__ __device__ constexpr int pack_scratch_bytes(int fmt) { return (fmt == TB_FMT_TERNARY2 ? 8 : 16) * 16 * 2; }
struct PackLds {
    size_t dq, qsum, ctr, zero, scratch, part;
};
__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }
__host__ __device__ inline PackLds pack_lds(int M, int fmt, int k, int waves)
{
    const bool tern = fmt == TB_FMT_TERNARY2;
    const int wpc = tern ? 64 : 128, bps = tern ? 8 : 16, nb = k / 128;
    const int I = (k / wpc + 15) / 16;
    PackLds p;
    p.dq = (size_t)I * (tern ? 1024 : 2048) * M;
    p.qsum = align16(p.dq + (size_t)(nb + bps) * M * 4);
    p.ctr = align16(p.qsum + (tern ? 0 : (size_t)(nb + bps) * M * 4));
    p.zero = align16(p.ctr + 16);
    p.scratch = p.zero + kPackZeroBytes;
    p.part = p.scratch + (size_t)waves * pack_scratch_bytes(fmt);
    return p;
}

template <int M, int FMT, int MODE, bool KS = false>
__global__ __launch_bounds__(pack_threads(FMT)) void gemv_mfma_pack_kernel(const void *p0, const void *p1,
                                                                           const void *p2, const void *p3,
                                                                           const void *p4, int pn, int pk,
                                                                           int pg, GemvArgs a_in)
{
    // leading arguments preloaded into SGPRs, as for gemv_ring_kernel
    const GemvArgs a = with_leading_args<FMT, MODE == kModeGateUp>(a_in, p0, p1, p2, p3, p4, pn, pk);
    static_assert(M >= 1 && M <= 8, "two blocks per MFMA: at most 8 activation rows");
    extern __shared__ __align__(16) uint8_t lds[];
    using L = StepLayout<M, FMT>;
    constexpr bool kTern = FMT == TB_FMT_TERNARY2;
    constexpr bool kTwo = MODE == kModeGateUp;
    constexpr bool kIsum = MODE == kModeIsum;
    constexpr int kParts = kTwo ? 2 : 1;
    constexpr int kMatShift = kTwo ? 1 : 0;   // gate/up: item = ((tile, step), matrix)
    constexpr int kBps = kTern ? 8 : 16;      // blocks per step (256 code bytes per row)
    constexpr int kBpl = kBps / 4;            // blocks per scale load of one lane
    // items in flight per wave: the split over k measured slower with 2 or 3 (the h loads
    // queue behind the weight prologue of the whole chip, and more weight in flight delays
    // them further: down stage at M = 4 / 6 / 8, µs per call, 13.12 / 13.77 / 14.28 at 1,
    // 14.26 / 14.97 / 15.42 at 2, 15.48 / 16.26 / 16.68 at 3; rotating h before issuing the
    // weight prologue: 13.95 / 14.98 / 14.75)
    constexpr int kDepth = kPackDepth;
    constexpr int kThreads = pack_threads(FMT), kWaves = kThreads / 64;
    constexpr int kScratch = pack_scratch_bytes(FMT);   // per wave: scales [block][row], uint16

    static_assert(!KS || MODE == kModeY, "the split over k is the down stage");
    const int k = a.k, n = a.n, nb = k / kBlock;
    const int C = k / Fmt<FMT>::kWeightsPerChunk, Ik = (C + kChunkLanes - 1) / kChunkLanes;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // KS: workgroup (g, s) of a.groups row groups x Ik steps covers step s of group g;
    // otherwise workgroup c covers all steps of share c of the grid
    const int G = KS ? a.groups : pg;
    int c = (int)blockIdx.x, s0 = 0;   // s0: the step of KS items
    if (KS && !split_index<FMT>(G, Ik, c, s0))
        return;
    const int I = KS ? 1 : Ik;                          // steps per tile in this workgroup
    const int T = (n + kRowsPerWave - 1) / kRowsPerWave;
    const int R0 = part_lo(T, G, c) * kRowsPerWave;
    const int R1 = min(part_lo(T, G, c + 1) * kRowsPerWave, n);
    const int J = (((R1 - R0 + 15) / 16) * I) << kMatShift;   // this workgroup's items
    const uint32_t row_bytes = (uint32_t)C * 16u;

    const PackLds pl = pack_lds(M, FMT, KS ? kBps * kBlock : k, kWaves);
    uint8_t *act = lds;
    float *dq_s = reinterpret_cast<float *>(lds + pl.dq);
    int *qsum_s = reinterpret_cast<int *>(lds + pl.qsum);
    int *ctr_s = reinterpret_cast<int *>(lds + pl.ctr);
    const uint8_t *zero_s = lds + pl.zero;                                     // B of inactive lanes
    uint16_t *sc_s = reinterpret_cast<uint16_t *>(lds + pl.scratch + wave * kScratch);
    float *part_s = reinterpret_cast<float *>(lds + pl.part);   // [row - R0][step][m][part]

    const __amdgpu_buffer_rsrc_t rout =
        buffer_rsrc(a.isum, kIsum ? (uint32_t)((size_t)M * n * nb * 4) : 0u);
    if (tid == 0)
        *ctr_s = kWaves;   // wave w starts with item w
    for (int i = tid; i < kPackZeroBytes / 4; i += kThreads)
        reinterpret_cast<uint32_t *>(lds + pl.zero)[i] = 0u;
    if (!kTern && !KS)
        for (int i = tid; i < (nb + kBps) * M; i += kThreads)
            qsum_s[i] = 0;
    __syncthreads();

    int gidx = 0, gtile = 0, gstep = 0;
    auto advance_to = [&](int idx) {
        gstep += idx - gidx;
        gidx = idx;
        while (gstep >= I) {
            gstep -= I;
            ++gtile;
        }
    };
    // Code loads: ternary lane (i, g) reads bytes 64 q + 16 g .. + 15 of its row's step (load
    // q = 0..3); sign lane (i, g) reads block bq(g) = {4 q, 4 q + 2, 4 q - 1 mod 16, 4 q + 1}[g].
    // In sign load q, group 2 reads 16 bytes before the others' base, except in load 0, where
    // its block 15 lies 240 bytes after it.
    const int sgofs = lg == 0 ? 0 : lg == 1 ? 32 : lg == 2 ? -16 : 16;
    const uint32_t lane_off = (uint32_t)li * row_bytes + (uint32_t)(kTern ? lg * 16 : sgofs + (lg == 2 ? 256 : 0));
    auto code_block = [&](int q) -> int {   // sign: the block (in the step) of this lane's load q
        return lg == 0 ? 4 * q : lg == 1 ? 4 * q + 2 : lg == 2 ? ((4 * q + 15) & 15) : 4 * q + 1;
    };
    // Scale loads: the word (ternary) or two words (sign) holding the scales of blocks
    // kBpl g .. of row i.
    const uint32_t lane_soff = ((uint32_t)li * (uint32_t)nb + (uint32_t)(lg * kBpl)) * 2u;
    uint4 rc[kDepth][4];
    u32x2 rs[kDepth];
    int rit[kDepth];   // matrix << 30 | tile << 16 | step, or -1
    int pending = tid >> 6;
    auto issue = [&](int d) {
        const int idx = __builtin_amdgcn_readfirstlane(pending);
        uint32_t off = kOutOfRange, soff = kOutOfRange;
        int so = 0, sso = 0, nbk = 0, mat = 0;
        rit[d] = -1;
        if (idx < J) {
            advance_to(idx >> kMatShift);
            mat = idx & (kTwo ? 1 : 0);
            rit[d] = mat << 30 | gtile << 16 | gstep;
            const int row0 = R0 + gtile * 16;
            const int wstep = s0 + gstep;            // the step in the weight rows
            so = row0 * (int)row_bytes + wstep * 256;
            sso = (row0 * nb + wstep * kBps) * 2;
            nbk = min(kBps, nb - wstep * kBps);   // blocks of this step inside the row
            if (row0 + li < R1) {
                off = lane_off;
                soff = (!kIsum && wstep * kBps + lg * kBpl < nb) ? lane_soff : kOutOfRange;
            }
            int v = 0;
            if (lane == 0)
                v = atomicAdd(ctr_s, 1);
            pending = v;
        }
        const __amdgpu_buffer_rsrc_t rcm = buffer_rsrc(mat ? a.codes1 : a.codes0, a.codes_bytes);
        const __amdgpu_buffer_rsrc_t rsm = buffer_rsrc(mat ? a.scales1 : a.scales0, a.scales_bytes);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t o;
            if (kTern) {
                // (nbk is even: both blocks of a load are in or out)
                o = 2 * q < nbk ? off + (uint32_t)q * 64u : kOutOfRange;
            } else {
                // (nbk is a multiple of 4; load 0's group 2 reads block 15)
                const uint32_t extra = (lg == 2 && q > 0) ? 256u : 0u;
                o = code_block(q) < nbk ? off + (uint32_t)q * 64u - extra : kOutOfRange;
                if (off == kOutOfRange)
                    o = kOutOfRange;
            }
            rc[d][q] = buffer_load16(rcm, o, so);
        }
        if (kTern) {
            rs[d].x = buffer_load_u32(rsm, soff, sso);
            rs[d].y = 0u;
        } else {
            rs[d] = __builtin_amdgcn_raw_buffer_load_b64(rsm, soff, sso, 0);
        }
    };

    if constexpr (KS) {
        // h loads of step s0's blocks first, then the weight prologue, then the rotation
        constexpr int kGroups16 = kThreads / 16;
        constexpr int kRounds = (M * kBps + kGroups16 - 1) / kGroups16;
        const int l16 = tid & 15, grp = tid >> 4;
        const int b0 = s0 * kBps, nbs = min(kBps, nb - b0), Z = M * nbs;
        float hv[kRounds][8];
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int z = grp + r * kGroups16;
            if (z < Z) {
                const int m = z / nbs, bl = z - m * nbs;
                const float *src = a.x + (size_t)m * k + (size_t)(b0 + bl) * kBlock + l16 * 8;
                const float4 lo = *reinterpret_cast<const float4 *>(src);
                const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
                hv[r][0] = lo.x; hv[r][1] = lo.y; hv[r][2] = lo.z; hv[r][3] = lo.w;
                hv[r][4] = hi.x; hv[r][5] = hi.y; hv[r][6] = hi.z; hv[r][7] = hi.w;
            }
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(d);
        for (int i = Z + tid; i < 2 * kBps * M; i += kThreads) {   // [block][m] past the step
            dq_s[i] = 0.0f;
            if (!kTern)
                qsum_s[i] = 0;
        }
        // (the zero slots of blocks past nbs: chunks past C read zero weights; their
        // activation slots are never multiplied by a nonzero code)
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int z = grp + r * kGroups16;
            if (z < Z) {   // (a 16-lane group takes or skips a block as a whole)
                const int m = z / nbs, bl = z - m * nbs;
                uint32_t pk[2];
                float dq;
                int qsum;
                rotquant_regs(hv[r], l16, a.unit, pk, dq, qsum);
                store_block_mfma<M, FMT>(act, m, bl, l16, pk);
                if (l16 == 0) {
                    dq_s[bl * M + m] = dq;
                    if (!kTern)
                        qsum_s[bl * M + m] = qsum;
                }
                if (c == 0) {   // row group 0 writes rotquant(h)
                    *reinterpret_cast<uint2 *>(a.qx + (size_t)m * k + (size_t)(b0 + bl) * kBlock + l16 * 8) =
                        make_uint2(pk[0], pk[1]);
                    if (l16 == 0)
                        a.dqx[(size_t)m * nb + b0 + bl] = dq;
                }
            }
        }
    } else {
        stage_activation<M, FMT, MODE, kThreads, true>(a, act, dq_s, qsum_s, [&]() {
#pragma unroll
            for (int d = 0; d < kDepth; ++d)
                issue(d);
        });
    }
    __syncthreads();

    // ---- compute side
    const int col = li, hsel = col >> 3, mcol = col & 7;
    const int mB = mcol < M ? mcol : M - 1;            // dq / code-sum row of this D column
    // this lane's B: the columns of its block half, rows < M; others read the zero region
    const bool bval = hsel == (lg >> 1) && mcol < M;
    auto consume = [&](int d) {
        const int mat = rit[d] >> 30, tile = (rit[d] >> 16) & 0x3fff, step = rit[d] & 0xffff;
        // this item's scales to the wave's scratch, [block in step][row in tile]
        if (!kIsum) {
            if (kTern) {
                sc_s[(2 * lg) * 16 + li] = (uint16_t)(rs[d].x & 0xffffu);
                sc_s[(2 * lg + 1) * 16 + li] = (uint16_t)(rs[d].x >> 16);
            } else {
                sc_s[(4 * lg) * 16 + li] = (uint16_t)(rs[d].x & 0xffffu);
                sc_s[(4 * lg + 1) * 16 + li] = (uint16_t)(rs[d].x >> 16);
                sc_s[(4 * lg + 2) * 16 + li] = (uint16_t)(rs[d].y & 0xffffu);
                sc_s[(4 * lg + 3) * 16 + li] = (uint16_t)(rs[d].y >> 16);
            }
        }
        const uint8_t *sact = act + (size_t)step * L::kStepBytes;
        constexpr int kPairs = kBps / 2;
        float t[kPairs][4];
        // one block pair: 4 MFMAs, then the terms of D
        auto pair = [&](int p, int blk_hi, const uint8_t *bbase, auto &&a_operand) {
            v4i acc = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v4i av, bv;
                a_operand(s, av, bv, bbase);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
            }
            const int blk = step * kBps + blk_hi;   // this lane's D block
            const int qs = kTern ? 0 : qsum_s[blk * M + mB];
            if constexpr (kIsum) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = R0 + tile * 16 + 4 * lg + r;
                    const bool wr = mcol < M && row < R1 && blk < nb;
                    const int v = kTern ? acc[r] : 2 * acc[r] - qs;
                    __builtin_amdgcn_raw_buffer_store_b32(
                        (uint32_t)v, rout, wr ? (uint32_t)(((mcol * n + row) * nb + blk) * 4) : kOutOfRange, 0, 0);
                }
            } else {
                const float dqv = dq_s[blk * M + mB];
                const uint2 sw = *reinterpret_cast<const uint2 *>(sc_s + (blk - step * kBps) * 16 + 4 * lg);
                const uint32_t s4[2] = {sw.x, sw.y};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sv = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(s4[r >> 1], (r & 1) * 16, 16));
                    const int isum = kTern ? acc[r] : 2 * acc[r] - qs;
                    t[p][r] = (sv * dqv) * (float)isum;
                }
            }
        };
        if constexpr (kTern) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t cw[4] = {rc[d][q].x, rc[d][q].y, rc[d][q].z, rc[d][q].w};
                // B: chunk 4 q + g, code word s, row mB: [chunk][word][row] x 16 bytes
                const uint8_t *bb = bval ? sact + ((size_t)((4 * q + lg) * 4) * M + mB) * 16 : zero_s;
                pair(q, 2 * q + hsel, bb, [&](int s, v4i &av, v4i &bv, const uint8_t *b) {
                    uint32_t d0, d1, d2, d3;
                    decode_ternary(cw[s], d0, d1, d2, d3);
                    av = v4i{(int)d0, (int)d1, (int)d2, (int)d3};
                    bv = *reinterpret_cast<const v4i *>(b + s * M * 16);
                });
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // pair A = (4 q, 4 q - 1) in H', pair B = (4 q + 2, 4 q + 1) in L'
                const u32x2 s0 = __builtin_amdgcn_permlane16_swap(rc[d][q].z, rc[d][q].x, false, false);
                const u32x2 s1 = __builtin_amdgcn_permlane16_swap(rc[d][q].w, rc[d][q].y, false, false);
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const uint32_t dw[2] = {h2 == 0 ? s0.x : s0.y, h2 == 0 ? s1.x : s1.y};
                    const int e = 4 * q + 2 * h2;                       // the pair's even block
                    const int myblk = (lg < 2) ? e : ((e + 15) & 15);   // this lane's A block
                    const int dblk = hsel == 0 ? e : ((e + 15) & 15);   // this lane's D block
                    // B: block myblk, dword (odd group: 0, 1; even group: 2, 3) + s, half h
                    const int dbase = (lg & 1) ? 0 : 2;
                    const uint8_t *bb =
                        bval ? sact + ((size_t)(2 * (4 * myblk + dbase)) * M + mB) * 16 : zero_s;
                    pair(2 * q + h2, dblk, bb, [&](int s, v4i &av, v4i &bv, const uint8_t *b) {
                        const uint32_t w = dw[s >> 1];
                        const int h = s & 1;
                        av = v4i{(int)((w >> (4 * h + 0)) & 0x01010101u), (int)((w >> (4 * h + 1)) & 0x01010101u),
                                 (int)((w >> (4 * h + 2)) & 0x01010101u), (int)((w >> (4 * h + 3)) & 0x01010101u)};
                        // dword dbase + (s >> 1), half h: slots (2 * (4 blk + dword) + h) * M + m
                        bv = *reinterpret_cast<const v4i *>(b + (size_t)(2 * (s >> 1) + h) * M * 16);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if constexpr (!kIsum) {
            float tot[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (kTern) {
                    // pairs p = (2p, 2p + 1); even lanes hold t(2p), the lane 8 over t(2p + 1)
                    const float P3 = t[0][r] + row_down(t[3][r], 8);   // t0 + t7
                    const float P2 = t[3][r] + row_down(t[2][r], 8);   // t6 + t5
                    const float P1 = t[2][r] + row_down(t[1][r], 8);   // t4 + t3
                    const float P0 = t[1][r] + row_down(t[0][r], 8);   // t2 + t1
                    tot[r] = (P3 + P2) + (P1 + P0);
                } else {
                    // pair p = 2 q + h2 has blocks (2p, 2p - 1): P_2p = t(2p) + t(2p - 1)
                    float P[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        P[p] = t[p][r] + row_down(t[p][r], 8);
                    tot[r] = ((P[0] + P[7]) + (P[6] + P[5])) + ((P[4] + P[3]) + (P[2] + P[1]));
                }
                // computed here, with every lane active: left free, the adds sink into the
                // store's branch below while the row rotations (DPP, which read other lanes)
                // stay out, so each rotation costs a move of its own instead of riding on
                // its add
                asm volatile("" : "+v"(tot[r]));
            }
            if (hsel == 0 && mcol < M) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lrow = tile * 16 + 4 * lg + r;   // row - R0
                    if (R0 + lrow < R1)
                        part_s[((size_t)(lrow * I + step) * M + mcol) * kParts + mat] = tot[r];
                }
            }
        }
    };
    for (;;) {
        bool any = false;
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (rit[d] >= 0) {
                consume(d);
                any = true;
            }
            issue(d);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!any)
            break;
    }
    if (kIsum)
        return;
    __syncthreads();
    if constexpr (KS) {   // the step partials [s0][m][row], summed by the fold launch
        for (int i = tid; i < (R1 - R0) * M; i += kThreads) {
            const int lrow = i / M, m = i % M;
            a.part[((size_t)s0 * a.part_rows + m) * n + R0 + lrow] = part_s[(size_t)lrow * M + m];
        }
        return;
    }
    // ---- every row: its step partials in step order, from +0
    for (int i = tid; i < (R1 - R0) * M; i += kThreads) {
        const int lrow = i / M, m = i % M;
        const float *ps = part_s + ((size_t)lrow * I * M + m) * kParts;
        float g = 0.0f, u = 0.0f;
        for (int st = 0; st < I; ++st) {
            g += ps[(size_t)st * M * kParts];
            if (kTwo)
                u += ps[(size_t)st * M * kParts + 1];
        }
        a.out[(size_t)m * n + R0 + lrow] = kTwo ? silu_gate(g, u) : g;
    }
}

// The fold of the down stage split over k: y[m][row] = the row's step partials
// part[s][m][row] summed in step order from +0. One thread per (m, row); its partials'
// loads go out sixteen at a time (consecutive threads read consecutive rows).
constexpr int kFoldThreads = 256;
constexpr int kFoldLoads = 16;
__global__ __launch_bounds__(kFoldThreads) void split_fold_kernel(const float *__restrict__ part,
                                                                  int steps, int n, int mn,
                                                                  float *__restrict__ y)
{
    const int i = blockIdx.x * kFoldThreads + threadIdx.x;   // = m * n + row
    if (i >= mn)
        return;
    float acc = 0.0f;
    for (int s0 = 0; s0 < steps; s0 += kFoldLoads) {
        float v[kFoldLoads];
#pragma unroll
        for (int u = 0; u < kFoldLoads; ++u)
            v[u] = s0 + u < steps ? part[(size_t)(s0 + u) * mn + i] : 0.0f;
#pragma unroll
        for (int u = 0; u < kFoldLoads; ++u)
            if (s0 + u < steps)
                acc += v[u];
    }
    y[i] = acc;
}

// ------------------------------------------------------------------------------------
// Sliced GEMV: for a K * M too large to stage at once. The activation is staged in
// slices of S chunks; each workgroup covers 16 rows. The per-row arithmetic is the same
// as in the ring kernel: lane cl folds chunks 16 i + cl in order of i.
// ------------------------------------------------------------------------------------
template <int M, int FMT, int MODE>
__global__ __launch_bounds__(kSlicedThreads) void gemv_sliced_kernel(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr bool kTwo = MODE == kModeGateUp;
    constexpr int kWpc = Fmt<FMT>::kWeightsPerChunk;
    constexpr int kCpb = Fmt<FMT>::kChunksPerBlock;

    const int k = a.k, n = a.n, nb = k / kBlock;
    const int C = k / kWpc;
    const int S = a.slice_chunks;
    const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15;
    const int row = blockIdx.x * (kSlicedThreads / 64) * kRowsPerWave + (tid >> 6) * 4 + (lane >> 4);
    const bool row_ok = row < n;
    const size_t row_bytes = (size_t)C * 16;

    uint8_t *act = lds;
    float *dq_s = reinterpret_cast<float *>(lds + (size_t)M * S * kWpc);
    int *qsum_s = reinterpret_cast<int *>(dq_s + M * nb);
    stage_block_terms<M, FMT, false>(dq_s, qsum_s, a.dq, a.q, nb, MODE != kModeIsum, tid,
                                     kSlicedThreads);

    // the row's sum of step partials (the streaming kernel's fold order)
    float tot0[M], tot1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        tot0[m] = 0.0f;
        tot1[m] = 0.0f;
    }
    const uint8_t *rp0 = a.codes0 + (size_t)(row_ok ? row : 0) * row_bytes;
    const uint8_t *rp1 = kTwo ? a.codes1 + (size_t)(row_ok ? row : 0) * row_bytes : nullptr;
    const uint16_t *sp0 = a.scales0 + (size_t)(row_ok ? row : 0) * nb;
    const uint16_t *sp1 = kTwo ? a.scales1 + (size_t)(row_ok ? row : 0) * nb : nullptr;

    for (int c0 = 0; c0 < C; c0 += S) {
        const int sc = min(S, C - c0);
        __syncthreads();   // previous slice consumed
        stage_act<M, FMT, false>(act, S, a.q, k, c0, sc, tid, kSlicedThreads);
        __syncthreads();
        for (int cc = cl; cc < ((sc + 15) & ~15); cc += kChunkLanes) {   // one step
            const int c = c0 + cc;
            const bool ok = row_ok && cc < sc;
            const int b = c / kCpb;
            const uint4 w0 = ok ? load_nt(rp0 + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
            const uint4 w1 = (kTwo && ok) ? load_nt(rp1 + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
            const float s0 = ok ? half_bits_to_float(sp0[b]) : 0.0f;
            const float s1 = (kTwo && ok) ? half_bits_to_float(sp1[b]) : 0.0f;
            int is0[M], is1[M];
            chunk_sums<M, FMT, kTwo>(w0, w1, act, S, ok ? cc : 0, is0, is1);
            if (MODE == kModeIsum) {
                if (ok && (kCpb == 1 || !(cl & 1))) {
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        a.isum[((size_t)m * n + row) * nb + b] =
                            FMT == TB_FMT_SIGN1 ? 2 * is0[m] - qsum_s[m * nb + b] : is0[m];
                }
                continue;
            }
            // the step partial: row tree of the lanes' terms (zero for lanes without a chunk)
            const int bb = ok ? b : 0;
            float p0[M], p1[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                int v0 = is0[m], v1 = is1[m];
                if (FMT == TB_FMT_SIGN1) {
                    v0 = 2 * v0 - qsum_s[m * nb + bb];
                    v1 = 2 * v1 - qsum_s[m * nb + bb];
                }
                const float dqv = dq_s[m * nb + bb];
                p0[m] = ok ? (s0 * dqv) * (float)v0 : 0.0f;
                p1[m] = (kTwo && ok) ? (s1 * dqv) * (float)v1 : 0.0f;
            }
            row_tree<M, FMT, kTwo>(p0, p1);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                tot0[m] += p0[m];
                tot1[m] += p1[m];
            }
        }
    }
    if (MODE == kModeIsum)
        return;
    if (cl == 0 && row_ok)
        store_row<M, MODE>(a, row, tot0, tot1);
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
using GemvFn = void (*)(GemvArgs);
// gemv_ring_kernel and gemv_mfma_pack_kernel: leading scalar arguments, then GemvArgs
using RingFn = void (*)(const void *, const void *, const void *, const void *, const void *, int,
                       int, int, GemvArgs);

#define TB_KERNEL_TABLE(NAME)                                                                  \
    template <int FMT, int MODE>                                                               \
    GemvFn NAME##_pick_m(int m)                                                                \
    {                                                                                          \
        switch (m) {                                                                           \
        case 1: return NAME<1, FMT, MODE>;                                                     \
        case 2: return NAME<2, FMT, MODE>;                                                     \
        case 3: return NAME<3, FMT, MODE>;                                                     \
        case 4: return NAME<4, FMT, MODE>;                                                     \
        case 5: return NAME<5, FMT, MODE>;                                                     \
        case 6: return NAME<6, FMT, MODE>;                                                     \
        case 7: return NAME<7, FMT, MODE>;                                                     \
        case 8: return NAME<8, FMT, MODE>;                                                     \
        default: return nullptr;                                                               \
        }                                                                                      \
    }                                                                                          \
    GemvFn NAME##_pick(int fmt, int mode, int m)                                               \
    {                                                                                          \
        if (fmt == TB_FMT_TERNARY2) {                                                          \
            if (mode == kModeY) return NAME##_pick_m<TB_FMT_TERNARY2, kModeY>(m);               \
            if (mode == kModeGateUp) return NAME##_pick_m<TB_FMT_TERNARY2, kModeGateUp>(m);     \
            return NAME##_pick_m<TB_FMT_TERNARY2, kModeIsum>(m);                               \
        }                                                                                      \
        if (mode == kModeY) return NAME##_pick_m<TB_FMT_SIGN1, kModeY>(m);                      \
        if (mode == kModeGateUp) return NAME##_pick_m<TB_FMT_SIGN1, kModeGateUp>(m);            \
        return NAME##_pick_m<TB_FMT_SIGN1, kModeIsum>(m);                                      \
    }

template <int FMT, int MODE>
RingFn gemv_ring_kernel_pick_m(int m)
{
    switch (m) {
    case 1: return gemv_ring_kernel<1, FMT, MODE>;
    case 2: return gemv_ring_kernel<2, FMT, MODE>;
    case 3: return gemv_ring_kernel<3, FMT, MODE>;
    case 4: return gemv_ring_kernel<4, FMT, MODE>;
    case 5: return gemv_ring_kernel<5, FMT, MODE>;
    case 6: return gemv_ring_kernel<6, FMT, MODE>;
    case 7: return gemv_ring_kernel<7, FMT, MODE>;
    case 8: return gemv_ring_kernel<8, FMT, MODE>;
    default: return nullptr;
    }
}
RingFn gemv_ring_kernel_pick(int fmt, int mode, int m)
{
    if (fmt == TB_FMT_TERNARY2) {
        if (mode == kModeY) return gemv_ring_kernel_pick_m<TB_FMT_TERNARY2, kModeY>(m);
        if (mode == kModeGateUp) return gemv_ring_kernel_pick_m<TB_FMT_TERNARY2, kModeGateUp>(m);
        return gemv_ring_kernel_pick_m<TB_FMT_TERNARY2, kModeIsum>(m);
    }
    if (mode == kModeY) return gemv_ring_kernel_pick_m<TB_FMT_SIGN1, kModeY>(m);
    if (mode == kModeGateUp) return gemv_ring_kernel_pick_m<TB_FMT_SIGN1, kModeGateUp>(m);
    return gemv_ring_kernel_pick_m<TB_FMT_SIGN1, kModeIsum>(m);
}
// Launches gemv_ring_kernel or gemv_mfma_pack_kernel: the leading scalar arguments are the
// matrices, the activation act (q, or x with ROTX), n, k and the grid (see the kernel).
void launch_ring(RingFn fn, int grid, size_t lds, hipStream_t stream, const GemvArgs &a,
                 const void *act, int threads = kRingThreads)
{
    const bool two = a.codes1 != nullptr;
    const void *p2 = two ? static_cast<const void *>(a.codes1) : act;
    const void *p3 = two ? static_cast<const void *>(a.scales1) : static_cast<const void *>(a.dq);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, stream,
                       static_cast<const void *>(a.codes0), static_cast<const void *>(a.scales0),
                       p2, p3, two ? act : nullptr, a.n, a.k, grid, a);
}
TB_KERNEL_TABLE(gemv_sliced_kernel)

template <int FMT, int MODE>
GemvFn gemv_mfma_pick_m(int m)
{
    switch (m) {
    case 4: return gemv_mfma_kernel<4, FMT, MODE>;
    case 5: return gemv_mfma_kernel<5, FMT, MODE>;
    case 6: return gemv_mfma_kernel<6, FMT, MODE>;
    case 7: return gemv_mfma_kernel<7, FMT, MODE>;
    case 8: return gemv_mfma_kernel<8, FMT, MODE>;
    case 9: return gemv_mfma_kernel<9, FMT, MODE>;
    case 10: return gemv_mfma_kernel<10, FMT, MODE>;
    case 11: return gemv_mfma_kernel<11, FMT, MODE>;
    case 12: return gemv_mfma_kernel<12, FMT, MODE>;
    case 13: return gemv_mfma_kernel<13, FMT, MODE>;
    case 14: return gemv_mfma_kernel<14, FMT, MODE>;
    case 15: return gemv_mfma_kernel<15, FMT, MODE>;
    case 16: return gemv_mfma_kernel<16, FMT, MODE>;
    default: return nullptr;
    }
}
template <int FMT, int MODE>
RingFn gemv_mfma_pack_pick_m(int m)
{
    switch (m) {
    case 2: return gemv_mfma_pack_kernel<2, FMT, MODE>;
    case 3: return gemv_mfma_pack_kernel<3, FMT, MODE>;
    case 4: return gemv_mfma_pack_kernel<4, FMT, MODE>;
    case 5: return gemv_mfma_pack_kernel<5, FMT, MODE>;
    case 6: return gemv_mfma_pack_kernel<6, FMT, MODE>;
    case 7: return gemv_mfma_pack_kernel<7, FMT, MODE>;
    case 8: return gemv_mfma_pack_kernel<8, FMT, MODE>;
    default: return nullptr;
    }
}
static_assert(mfma_min_rows(true, true) >= 2 && mfma_min_rows(true, false) >= 2 &&
                  mfma_min_rows(false, true) >= 2 && mfma_min_rows(false, false) >= 2,
              "gemv_mfma_pack_kernel is instantiated for M = 2 .. 8");

constexpr int kMaxWideRows = 16;   // rows of one gemv_mfma_kernel launch in the batch calls
#ifndef TB_GATEUP_PHASED
#define TB_GATEUP_PHASED 1
#endif
constexpr int kMaxDevices = 64;
struct DeviceInfo {
    int lds_limit = 0;   // 0 = not queried yet
    int cus = 0;
};
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];
// Kernels whose dynamic LDS limit has been raised, per device, with the limit set: the
// attribute is set once per kernel and size instead of on every launch.
constexpr int kMaxRaised = 512;
struct Raised {
    const void *fn;
    int lds;
};
Raised g_raised[kMaxDevices][kMaxRaised];
int g_nraised[kMaxDevices];
uint8_t *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's address of `scratch` (looked up once per device, with it current).
int scratch_address(uint8_t **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TB_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return TB_EHIP;
        g_scratch[dev] = static_cast<uint8_t *>(p);
    }
    *out = g_scratch[dev];
    return TB_OK;
}

int device_info(DeviceInfo *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TB_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (d.lds_limit == 0) {
        int lds = 0, cus = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            lds <= 0 || cus <= 0)
            return TB_EHIP;
        d.lds_limit = lds;
        d.cus = cus;
    }
    *out = d;
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
    if (w->fmt != TB_FMT_TERNARY2 && w->fmt != TB_FMT_SIGN1 && w->fmt != TB_FMT_SIGN1_RI4)
        return TB_EINVAL;
    if (w->fmt == TB_FMT_SIGN1_RI4 && w->n % 4)
        return TB_EINVAL;
    if (!aligned16(w->codes) || !aligned16(w->scales))
        return TB_EALIGN;
    // buffer addressing: each array must stay below 2 GiB
    const size_t nb = (size_t)(w->k / kBlock);
    const size_t cb = (size_t)w->n * (size_t)w->k / (w->fmt == TB_FMT_TERNARY2 ? 4 : 8);
    if (cb >= ((size_t)1 << 31) || (size_t)w->n * nb * 2 >= ((size_t)1 << 31))
        return TB_EUNSUPPORTED;
    return TB_OK;
}

size_t codes_bytes(const tb_matrix *w)
{
    return (size_t)w->n * (size_t)w->k / (w->fmt == TB_FMT_TERNARY2 ? 4 : 8);
}
size_t scales_bytes(const tb_matrix *w) { return (size_t)w->n * (size_t)(w->k / kBlock) * 2; }

int check_rows(int m, int max_rows = TB_MAX_ROWS) { return (m >= 1 && m <= max_rows) ? TB_OK : TB_EINVAL; }

float dq_unit() { return static_cast<float>(1.0 / (127.0 * std::sqrt(128.0))); }

int launch_rotquant(const float *x, int m, int k, int8_t *q, float *dq, hipStream_t stream)
{
    const long nblocks = (long)m * (k / kBlock);
    const int grid = (int)((nblocks + kRotThreads / 16 - 1) / (kRotThreads / 16));
    hipLaunchKernelGGL(rotquant_kernel, dim3(grid), dim3(kRotThreads), 0, stream, x, nblocks, q,
                       dq, dq_unit());
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

size_t block_terms_bytes(int fmt, int m, int nb)
{
    return (size_t)m * nb * 4 * (fmt == TB_FMT_TERNARY2 ? 1 : 2);
}

// Raise fn's dynamic LDS limit to at least lds bytes on the current device (once).
int raise_lds(const void *fn, size_t lds)
{
    if (lds <= 65536)
        return TB_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TB_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    Raised *tab = g_raised[dev];
    int &cnt = g_nraised[dev];
    for (int i = 0; i < cnt; ++i)
        if (tab[i].fn == fn && tab[i].lds >= (int)lds)
            return TB_OK;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return TB_EHIP;
    for (int i = 0; i < cnt; ++i)
        if (tab[i].fn == fn) {
            tab[i].lds = (int)lds;
            return TB_OK;
        }
    if (cnt < kMaxRaised)
        tab[cnt++] = Raised{fn, (int)lds};
    return TB_OK;
}

int set_lds(GemvFn fn, size_t lds) { return raise_lds(reinterpret_cast<const void *>(fn), lds); }

// LDS bytes of gemv_mfma_kernel for m rows of a matrix of n rows and k inputs on a grid of
// `grid` workgroups (activation, block terms, code sums, item counter, step partials).
size_t mfma_lds_bytes(int fmt, int mode, int n, int k, int m, int grid)
{
    const bool tern = fmt == TB_FMT_TERNARY2;
    const int wpc = tern ? 64 : 128, nb = k / kBlock;
    const int steps = (k / wpc + kChunkLanes - 1) / kChunkLanes;
    const long tiles = (n + kRowsPerWave - 1) / kRowsPerWave;
    const size_t rows_cu = (size_t)((tiles + grid - 1) / grid) * kRowsPerWave;
    const size_t bps = tern ? 8 : 16;
    return (size_t)steps * (tern ? 1024 : 2048) * m + (size_t)m * (nb + bps) * 4 * (tern ? 1 : 2) + 16 +
           rows_cu * steps * m * (mode == kModeGateUp ? 2 : 1) * 4;
}

// Rows of a batch above 8 run on gemv_mfma_kernel with all 16 B columns live: whether m
// such rows fit this device and shape.
bool wide_fits(const DeviceInfo &info, int mode, const tb_matrix *w, int m)
{
    const bool tern = w->fmt == TB_FMT_TERNARY2;
    if ((w->k / kBlock) % (tern ? 2 : 4))
        return false;
    const long tiles = (w->n + kRowsPerWave - 1) / kRowsPerWave;
    const int grid = (int)(tiles < info.cus ? tiles : info.cus);
    return mfma_lds_bytes(w->fmt, mode, w->n, w->k, m, grid) <= (size_t)info.lds_limit;
}

// LDS bytes of gemv_ring_kernel for m rows on a grid of `grid` workgroups: the step-major
// activation, the block terms (and sign code sums) zero padded by one step of blocks, the
// item counter, and the step partials of the largest workgroup's items.
size_t ring_lds_bytes(const tb_matrix *w, int mode, int m, int grid)
{
    const bool tern = w->fmt == TB_FMT_TERNARY2;
    const int C = w->k / (tern ? 64 : 128), nb = w->k / kBlock;
    const int steps = (C + kChunkLanes - 1) / kChunkLanes;
    const long tiles = (w->n + kRowsPerWave - 1) / kRowsPerWave;
    const size_t step_bytes = (size_t)(tern ? 1024 : 2048) * m;
    const size_t pad_blocks = (size_t)(kChunkLanes / (tern ? 2 : 1));
    const size_t ring_terms = (size_t)m * (nb + pad_blocks) * 4 * (tern ? 1 : 2);
    const size_t ring_items = (size_t)((tiles + grid - 1) / grid) * steps;
    const size_t ring_part = 16 + ring_items * kRowsPerWave * m * (mode == kModeGateUp ? 2 : 1) * 4;
    return (size_t)steps * step_bytes + ring_terms + ring_part;
}

int launch_gemv(int mode, const tb_matrix *w0, const tb_matrix *w1, const int8_t *q,
                const float *dq, int m, float *out, int32_t *isum, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    GemvArgs a = {};
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
    a.codes_bytes = (uint32_t)codes_bytes(w0);
    // scales are read as aligned 4-byte words: when n * nb is odd the last word's upper
    // half lies past the array, inside the same aligned word (which cannot cross a page),
    // and is ignored
    a.scales_bytes = (uint32_t)((scales_bytes(w0) + 3) & ~(size_t)3);
    const int wpc = w0->fmt == TB_FMT_TERNARY2 ? 64 : 128;
    const int C = w0->k / wpc, nb = w0->k / kBlock;
    const long tiles = (w0->n + kRowsPerWave - 1) / kRowsPerWave;
    const int ring_grid = (int)(tiles < info.cus ? tiles : info.cus);
    const size_t terms = block_terms_bytes(w0->fmt, m, nb);
    const int steps = (C + kChunkLanes - 1) / kChunkLanes;
    const size_t step_bytes = (size_t)(w0->fmt == TB_FMT_TERNARY2 ? 1024 : 2048) * m;

    // batched rows: the matrix-core kernel, when its LDS plan fits (a lane's scale load
    // holds whole block pairs (ternary) or quads (sign) of one row)
    const bool tern = w0->fmt == TB_FMT_TERNARY2;
    // The block-sum export takes the matrix-core route from the gate/up threshold on (the
    // smallest M at which production runs the matrix-core integer core, which is the same
    // code in gate/up and one-matrix mode).
    if (nb % (tern ? 2 : 4) == 0 && m >= mfma_min_rows(tern, mode != kModeY)) {
        const size_t rows_cu = (size_t)((tiles + ring_grid - 1) / ring_grid) * kRowsPerWave;
        const size_t bps = tern ? 8 : 16;
        const size_t parts = rows_cu * steps * m * (mode == kModeGateUp ? 2 : 1) * 4;
#if TB_MFMA_PACK
        // two blocks per MFMA, for at most 8 rows
        const size_t pack_lds_bytes = m > 8 ? ~(size_t)0 :
            pack_lds(m, w0->fmt, w0->k, pack_threads(w0->fmt) / 64).part + parts;
        if (m <= 8 && pack_lds_bytes <= (size_t)info.lds_limit) {
            RingFn fn = tern ? (mode == kModeGateUp ? gemv_mfma_pack_pick_m<TB_FMT_TERNARY2, kModeGateUp>(m)
                                : mode == kModeY  ? gemv_mfma_pack_pick_m<TB_FMT_TERNARY2, kModeY>(m)
                                                  : gemv_mfma_pack_pick_m<TB_FMT_TERNARY2, kModeIsum>(m))
                             : (mode == kModeGateUp ? gemv_mfma_pack_pick_m<TB_FMT_SIGN1, kModeGateUp>(m)
                                : mode == kModeY  ? gemv_mfma_pack_pick_m<TB_FMT_SIGN1, kModeY>(m)
                                                  : gemv_mfma_pack_pick_m<TB_FMT_SIGN1, kModeIsum>(m));
            if (!fn)
                return TB_EINVAL;
            if ((rc = raise_lds(reinterpret_cast<const void *>(fn), pack_lds_bytes)))
                return rc;
            launch_ring(fn, ring_grid, pack_lds_bytes, stream, a, q, pack_threads(w0->fmt));
            return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
        }
#endif
        (void)bps;
        (void)step_bytes;
        const size_t mfma_lds = mfma_lds_bytes(w0->fmt, mode, w0->n, w0->k, m, ring_grid);
        if (mfma_lds <= (size_t)info.lds_limit) {
            GemvFn fn = tern ? (mode == kModeGateUp ? gemv_mfma_pick_m<TB_FMT_TERNARY2, kModeGateUp>(m)
                                : mode == kModeY  ? gemv_mfma_pick_m<TB_FMT_TERNARY2, kModeY>(m)
                                                  : gemv_mfma_pick_m<TB_FMT_TERNARY2, kModeIsum>(m))
                             : (mode == kModeGateUp ? gemv_mfma_pick_m<TB_FMT_SIGN1, kModeGateUp>(m)
                                : mode == kModeY  ? gemv_mfma_pick_m<TB_FMT_SIGN1, kModeY>(m)
                                                  : gemv_mfma_pick_m<TB_FMT_SIGN1, kModeIsum>(m));
            if (!fn)
                return TB_EINVAL;
            if ((rc = set_lds(fn, mfma_lds)))
                return rc;
            hipLaunchKernelGGL(fn, dim3(ring_grid), dim3(mfma_threads(w0->fmt)), mfma_lds, stream, a);
            return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
        }
    }

    if (m > 8)
        return TB_EUNSUPPORTED;   // the batch launcher only passes rows that fit
    // whole activation in LDS: the persistent ring kernel, one workgroup per CU
    const size_t ring_lds = ring_lds_bytes(w0, mode, m, ring_grid);
    // (both kernels fold every row in the same order, so the choice never changes a result)
    if (ring_lds <= (size_t)info.lds_limit) {
        RingFn fn = gemv_ring_kernel_pick(w0->fmt, mode, m);
        if (!fn)
            return TB_EINVAL;
        if ((rc = raise_lds(reinterpret_cast<const void *>(fn), ring_lds)))
            return rc;
        // one workgroup per CU (fewer only if there are fewer row tiles than CUs)
        a.slice_chunks = C;
        launch_ring(fn, ring_grid, ring_lds, stream, a, q);
        return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
    }
    // otherwise stage the activation in slices of S chunks (S a multiple of 16)
    int S = (C + 15) & ~15;
    while ((size_t)m * S * wpc + terms > (size_t)info.lds_limit) {
        if (S <= 16)
            return TB_EUNSUPPORTED;
        S = ((S / 2) + 15) & ~15;
    }
    const size_t lds = (size_t)m * S * wpc + terms;
    GemvFn fn = gemv_sliced_kernel_pick(w0->fmt, mode, m);
    if (!fn)
        return TB_EINVAL;
    if ((rc = set_lds(fn, lds)))
        return rc;
    a.slice_chunks = S;
    const int rows_per_wg = (kSlicedThreads / 64) * kRowsPerWave;
    const int grid = (w0->n + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kSlicedThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}


// gemv_ring_kernel with the rotation of x inside (ROTX), for the row counts it is built for
// Each 16-lane group of a workgroup rotates up to this many blocks (a workgroup of 1024
// lanes: m * k/128 <= 128). Separate-call FFN stream at 64 layers, µs per layer, with 1 / 2
// / 3 blocks per group: M=1 21.64 / 21.66 / 22.54 (the down stage's 136 blocks inside cost
// 1 µs more than the launch they save), M=2 26.14 / 25.43 / 25.42, M=3 30.51 / 30.00 /
// 29.97, M=4 32.98 / 32.99 / 34.15; two launches per layer before: 23.06, 25.90, 30.44, 32.92.
#ifndef TB_ROTX_MAX_ROUNDS
#define TB_ROTX_MAX_ROUNDS 2
#endif
#ifndef TB_ROTX_MAX_ROWS
#define TB_ROTX_MAX_ROWS 4
#endif
template <int FMT, int MODE>
RingFn gemv_ring_rotx_pick_m(int m)
{
    static_assert(TB_ROTX_MAX_ROWS >= 1 && TB_ROTX_MAX_ROWS <= 4, "built for 1..4 rows");
    switch (m) {
    case 1: return gemv_ring_kernel<1, FMT, MODE, true>;
    case 2: return TB_ROTX_MAX_ROWS >= 2 ? gemv_ring_kernel<2, FMT, MODE, true> : nullptr;
    case 3: return TB_ROTX_MAX_ROWS >= 3 ? gemv_ring_kernel<3, FMT, MODE, true> : nullptr;
    case 4: return TB_ROTX_MAX_ROWS >= 4 ? gemv_ring_kernel<4, FMT, MODE, true> : nullptr;
    default: return nullptr;
    }
}

// One launch that rotates and quantises x[m][k] inside the GEMV (mode y or gate/up), when
// the rows take the ring kernel (below the matrix-core thresholds, LDS plan fits, at most
// TB_ROTX_MAX_ROWS rows); TB_EUNSUPPORTED otherwise, and then nothing was launched.
// Workgroup 0 writes rotquant(x) to qx, dqx.
int launch_gemv_rotx(int mode, const tb_matrix *w0, const tb_matrix *w1, const float *x, int m,
                     int8_t *qx, float *dqx, float *out, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    const bool tern = w0->fmt == TB_FMT_TERNARY2;
    const int nb = w0->k / kBlock;
    if (m > TB_ROTX_MAX_ROWS || (long)m * nb > (long)TB_ROTX_MAX_ROUNDS * (kRingThreads / 16) ||
        (nb % (tern ? 2 : 4) == 0 && m >= mfma_min_rows(tern, mode != kModeY)))
        return TB_EUNSUPPORTED;
    const long tiles = (w0->n + kRowsPerWave - 1) / kRowsPerWave;
    const int grid = (int)(tiles < info.cus ? tiles : info.cus);
    const size_t lds = ring_lds_bytes(w0, mode, m, grid);
    if (lds > (size_t)info.lds_limit)
        return TB_EUNSUPPORTED;
    RingFn fn = tern ? (mode == kModeGateUp ? gemv_ring_rotx_pick_m<TB_FMT_TERNARY2, kModeGateUp>(m)
                                            : gemv_ring_rotx_pick_m<TB_FMT_TERNARY2, kModeY>(m))
                     : (mode == kModeGateUp ? gemv_ring_rotx_pick_m<TB_FMT_SIGN1, kModeGateUp>(m)
                                            : gemv_ring_rotx_pick_m<TB_FMT_SIGN1, kModeY>(m));
    if (!fn)
        return TB_EUNSUPPORTED;
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), lds)))
        return rc;
    GemvArgs a = {};
    a.codes0 = static_cast<const uint8_t *>(w0->codes);
    a.scales0 = w0->scales;
    a.codes1 = w1 ? static_cast<const uint8_t *>(w1->codes) : nullptr;
    a.scales1 = w1 ? w1->scales : nullptr;
    a.n = w0->n;
    a.k = w0->k;
    a.out = out;
    a.codes_bytes = (uint32_t)codes_bytes(w0);
    a.scales_bytes = (uint32_t)((scales_bytes(w0) + 3) & ~(size_t)3);
    a.slice_chunks = w0->k / (tern ? 64 : 128);
    a.x = x;
    a.qx = qx;
    a.dqx = dqx;
    a.unit = dq_unit();
    launch_ring(fn, grid, lds, stream, a, x);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

// y[m][n] = the step partials part[I][m][n] summed in step order (split_fold_kernel).
int launch_split_fold(const float *part, int I, int n, int m, float *y, hipStream_t stream)
{
    const int mn = m * n;
    hipLaunchKernelGGL(split_fold_kernel, dim3((mn + kFoldThreads - 1) / kFoldThreads),
                       dim3(kFoldThreads), 0, stream, part, I, n, mn, y);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

// The down stage split over k: gemv_mfma_pack_kernel<KS> on R row groups x I steps (R =
// floor(CUs / I), at least 1, at most the row tiles), which rotates its step's blocks of h
// and writes step partials to ws, then split_fold_kernel. TB_EUNSUPPORTED (nothing
// launched) where the packed kernel's LDS plan does not fit.
template <int FMT>
RingFn split_pick_m(int m)
{
    static_assert(TB_SPLIT_MIN_ROWS >= 4, "built from 4 rows");
    switch (m) {
    case 4: return gemv_mfma_pack_kernel<4, FMT, kModeY, true>;
    case 5: return gemv_mfma_pack_kernel<5, FMT, kModeY, true>;
    case 6: return gemv_mfma_pack_kernel<6, FMT, kModeY, true>;
    case 7: return gemv_mfma_pack_kernel<7, FMT, kModeY, true>;
    case 8: return gemv_mfma_pack_kernel<8, FMT, kModeY, true>;
    default: return nullptr;
    }
}
int split_steps(const tb_matrix *w) { return (w->k / (w->fmt == TB_FMT_TERNARY2 ? 64 : 128) + 15) / 16; }
size_t split_workspace_bytes(const tb_matrix *w, int m) { return (size_t)split_steps(w) * m * w->n * 4; }

int launch_down_split(const tb_matrix *w, const float *h, int m, int8_t *qh, float *dqh, float *y,
                      float *part, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    const bool tern = w->fmt == TB_FMT_TERNARY2;
    const int I = split_steps(w), nb = w->k / kBlock;
    const int T = (w->n + kRowsPerWave - 1) / kRowsPerWave;
    const int R = std::max(1, std::min(info.cus / I, T));
    if (nb % (tern ? 2 : 4) != 0)   // a lane's scale load holds whole block pairs / quads
        return TB_EUNSUPPORTED;
    const size_t rows_g = (size_t)((T + R - 1) / R) * kRowsPerWave + 16;   // + a 16-row tile's slack
    const size_t lds = pack_lds(m, w->fmt, (tern ? 8 : 16) * kBlock, pack_threads(w->fmt) / 64).part +
                       rows_g * m * 4;
    if (lds > (size_t)info.lds_limit)
        return TB_EUNSUPPORTED;
    RingFn fn = tern ? split_pick_m<TB_FMT_TERNARY2>(m) : split_pick_m<TB_FMT_SIGN1>(m);
    if (!fn)
        return TB_EUNSUPPORTED;
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), lds)))
        return rc;
    GemvArgs a = {};
    a.codes0 = static_cast<const uint8_t *>(w->codes);
    a.scales0 = w->scales;
    a.n = w->n;
    a.k = w->k;
    a.x = h;
    a.qx = qh;
    a.dqx = dqh;
    a.unit = dq_unit();
    a.groups = R;
    a.part = part;
    a.part_rows = m;
    a.codes_bytes = (uint32_t)codes_bytes(w);
    a.scales_bytes = (uint32_t)((scales_bytes(w) + 3) & ~(size_t)3);
    launch_ring(fn, split_grid(I * R, w->fmt), lds, stream, a, h, pack_threads(w->fmt));
    if (hipGetLastError() != hipSuccess)
        return TB_EHIP;
    return launch_split_fold(part, I, w->n, m, y, stream);
}

// The same split for batches of 9 ... 32 rows on gemv_mfma_kernel<KS> (one block per
// MFMA, all 16 B columns live). Ternary: one launch whose B operands hold up to 16 rows
// (one column group) or up to 32 (two, sharing each decoded A operand), so the down
// weights are read once per batch. Sign: balanced chunks of up to 16 rows (two column
// groups over its 16-block steps need more registers than 8 waves have: 120 bytes of
// spills per lane), each chunk one launch. Each workgroup stages one step of its rows
// (16 KB of codes at 16 ternary rows) where the unsplit 16-row kernel would stage all of
// k; the kernel is built for 16 or 32 rows and takes the row count at run time. Every
// launch writes its rows' step partials into the batch's [I][m][n] workspace; then one
// fold launch. TB_EUNSUPPORTED (nothing launched) where the LDS plan does not fit.
template <int FMT>
GemvFn split_wide_pick(int mcap)
{
    if constexpr (FMT == TB_FMT_TERNARY2)
        if (mcap > 16)
            return gemv_mfma_kernel<32, FMT, kModeY, true>;
    return mcap <= 16 ? gemv_mfma_kernel<16, FMT, kModeY, true> : nullptr;
}
int launch_down_split_wide(const tb_matrix *w, const float *h, int m, int8_t *qh, float *dqh,
                           float *y, float *part, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    if (m <= TB_MAX_ROWS || m > TB_MAX_BATCH_ROWS)
        return TB_EUNSUPPORTED;
    const bool tern = w->fmt == TB_FMT_TERNARY2;
    const int I = split_steps(w), k = w->k, nb = k / kBlock, bps = tern ? 8 : 16;
    const int T = (w->n + kRowsPerWave - 1) / kRowsPerWave;
    const int R = std::max(1, std::min(info.cus / I, T));
    if (nb % (tern ? 2 : 4) != 0)   // a lane's scale load holds whole block pairs / quads
        return TB_EUNSUPPORTED;
    const int mcap = (m <= 16 || !tern) ? 16 : 32;   // the kernel's rows (B columns)
    const int chunks = (m + mcap - 1) / mcap;
    const size_t rows_g = (size_t)((T + R - 1) / R) * kRowsPerWave;
    // (the kernel's carve-up: one step of codes, the step's block terms [2 steps][rows] (and
    // code sums for sign), the item counter, the step partials of the group's rows)
    const size_t lds = (size_t)(tern ? 1024 : 2048) * mcap + (size_t)2 * bps * mcap * 4 * (tern ? 1 : 2) +
                       16 + rows_g * mcap * 4;
    if (lds > (size_t)info.lds_limit)
        return TB_EUNSUPPORTED;
    GemvFn fn = tern ? split_wide_pick<TB_FMT_TERNARY2>(mcap) : split_wide_pick<TB_FMT_SIGN1>(mcap);
    if (!fn)
        return TB_EUNSUPPORTED;
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), lds)))
        return rc;
    for (int i = 0, r0 = 0; i < chunks; ++i) {
        const int mc = (m * (i + 1)) / chunks - (m * i) / chunks;
        GemvArgs a = {};
        a.codes0 = static_cast<const uint8_t *>(w->codes);
        a.scales0 = w->scales;
        a.n = w->n;
        a.k = k;
        a.x = h + (size_t)r0 * k;
        a.qx = qh + (size_t)r0 * k;
        a.dqx = dqh + (size_t)r0 * nb;
        a.unit = dq_unit();
        a.groups = R;
        a.part = part + (size_t)r0 * w->n;
        a.part_rows = m;
        a.act_rows = mc;
        a.codes_bytes = (uint32_t)codes_bytes(w);
        a.scales_bytes = (uint32_t)((scales_bytes(w) + 3) & ~(size_t)3);
        hipLaunchKernelGGL(fn, dim3(split_grid(I * R, w->fmt)), dim3(mfma_threads(w->fmt, mcap)), lds, stream,
                           a);
        if (hipGetLastError() != hipSuccess)
            return TB_EHIP;
        r0 += mc;
    }
    return launch_split_fold(part, I, w->n, m, y, stream);
}

// The lookup-table GEMV (block sums when isum is given) over row-interleaved sign weights,
// for 1 <= m <= 2 rows; one 16-wave workgroup per CU.
int launch_lut(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
               int32_t *isum, hipStream_t stream)
{
    if (m > tblut::kMaxRows)
        return TB_EUNSUPPORTED;
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    const int T = w->n / 4, nb = w->k / kBlock, I = (nb + 15) / 16;
    const int grid = T < info.cus ? T : info.cus;
    const size_t lds = (size_t)((T + grid - 1) / grid) * I * 4 * m * 4;
    if (lds > (size_t)info.lds_limit)
        return TB_EUNSUPPORTED;
    tblut::LutArgs a = {};
    a.codes = static_cast<const uint8_t *>(w->codes);
    a.scales = w->scales;
    a.n = w->n;
    a.k = w->k;
    a.q = q;
    a.dq = dq;
    a.out = y;
    a.isum = isum;
    a.codes_bytes = (uint32_t)codes_bytes(w);
    a.scales_bytes = (uint32_t)scales_bytes(w);
    using LutFn = void (*)(tblut::LutArgs);
    LutFn fn = isum ? (m == 1 ? tblut::gemv_lut_kernel<1, true> : tblut::gemv_lut_kernel<2, true>)
                    : (m == 1 ? tblut::gemv_lut_kernel<1, false> : tblut::gemv_lut_kernel<2, false>);
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), lds)))
        return rc;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(tblut::kThreads), lds, stream, a);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

// A batch of m (1..32) independent rows as balanced chunks: chunks of up to 16 rows on
// gemv_mfma_kernel (all 16 B columns live) where they fit the device's LDS, else of up to 8
// rows on the kernels of the 1..8-row calls. Every kernel folds a row the same way, so a
// row's outputs do not depend on the chunk it lands in.
// Ternary gate/up of 17 ... 32 rows in one launch: gemv_mfma_kernel<32, ..., KP>, two
// 16-column groups sharing each decoded weight operand, k staged in two phases (32 rows of
// the whole activation would not fit the LDS), so the weights are read once instead of once
// per 16-row chunk. TB_EUNSUPPORTED (nothing launched) where the LDS plan does not fit.
int launch_gateup_phased(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q, const float *dq,
                         int m, float *h, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
    if (wg->fmt != TB_FMT_TERNARY2 || m <= kMaxWideRows || m > TB_MAX_BATCH_ROWS)
        return TB_EUNSUPPORTED;
    const int k = wg->k, nb = k / kBlock;
    if (nb % 2 != 0)   // a lane's scale load holds whole block pairs
        return TB_EUNSUPPORTED;
    const int Ik = (k / 64 + kChunkLanes - 1) / kChunkLanes, Sp = (Ik + 1) / 2;
    const int NS = std::max(Sp, 1 + Ik - Sp);
    const long tiles = (wg->n + kRowsPerWave - 1) / kRowsPerWave;
    const int grid = (int)(tiles < info.cus ? tiles : info.cus);
    const size_t rows_cu = (size_t)((tiles + grid - 1) / grid) * kRowsPerWave;
    // (the kernel's carve-up: phase 0's codes, the block terms of all steps, the item
    // counter, the step partials [row][slot][32][gate, up])
    const size_t lds = (size_t)Sp * 1024 * 32 + (size_t)(nb + 8) * 32 * 4 + 16 + rows_cu * NS * 32 * 2 * 4;
    if (lds > (size_t)info.lds_limit)
        return TB_EUNSUPPORTED;
    GemvFn fn = gemv_mfma_kernel<32, TB_FMT_TERNARY2, kModeGateUp, false, true>;
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), lds)))
        return rc;
    GemvArgs a = {};
    a.codes0 = static_cast<const uint8_t *>(wg->codes);
    a.scales0 = wg->scales;
    a.codes1 = static_cast<const uint8_t *>(wu->codes);
    a.scales1 = wu->scales;
    a.n = wg->n;
    a.k = k;
    a.q = q;
    a.dq = dq;
    a.out = h;
    a.act_rows = m;
    a.codes_bytes = (uint32_t)codes_bytes(wg);
    a.scales_bytes = (uint32_t)((scales_bytes(wg) + 3) & ~(size_t)3);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(mfma_threads(TB_FMT_TERNARY2, 32)), lds, stream, a);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

int launch_gemv_batch(int mode, const tb_matrix *w0, const tb_matrix *w1, const int8_t *q,
                      const float *dq, int m, float *out, int32_t *isum, hipStream_t stream)
{
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc)
        return rc;
#if TB_GATEUP_PHASED
    if (mode == kModeGateUp && m > kMaxWideRows) {
        rc = launch_gateup_phased(w0, w1, q, dq, m, out, stream);
        if (rc != TB_EUNSUPPORTED)
            return rc;
    }
#endif
    int cmax = 8;
    for (int c = m < kMaxWideRows ? m : kMaxWideRows; c > 8; --c)
        if (wide_fits(info, mode, w0, c)) {
            cmax = c;
            break;
        }
    const int chunks = (m + cmax - 1) / cmax;
    const size_t k = (size_t)w0->k, n = (size_t)w0->n, nb = k / kBlock;
    for (int i = 0, r0 = 0; i < chunks; ++i) {
        const int mc = (m * (i + 1)) / chunks - (m * i) / chunks;
        rc = launch_gemv(mode, w0, w1, q + r0 * k, dq ? dq + r0 * nb : nullptr, mc,
                         out ? out + r0 * n : nullptr, isum ? isum + r0 * n * nb : nullptr, stream);
        if (rc)
            return rc;
        r0 += mc;
    }
    return TB_OK;
}

// ------------------------------------------------------------------------------------
// Fused FFN layers
// ------------------------------------------------------------------------------------
using LayersFn = void (*)(tbl::LArgs);

template <int FMT>
LayersFn layers_pick_m(int m)
{
    switch (m) {
    case 1: return tbl::ffn_layers_kernel<1, FMT>;
    case 2: return tbl::ffn_layers_kernel<2, FMT>;
    case 3: return tbl::ffn_layers_kernel<3, FMT>;
    case 4: return tbl::ffn_layers_kernel<4, FMT>;
    case 5: return tbl::ffn_layers_kernel<5, FMT>;
    case 6: return tbl::ffn_layers_kernel<6, FMT>;
    case 7: return tbl::ffn_layers_kernel<7, FMT>;
    case 8: return tbl::ffn_layers_kernel<8, FMT>;
    default: return nullptr;
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace: sync words, then the tagged arrays (8-byte entries).
struct WsLayout {
    size_t sync, hp, qp, dp, sp, yp, total;
};

WsLayout ws_layout(int m, int hidden, int inter)
{
    WsLayout w;
    const size_t nbi = (size_t)inter / kBlock;
    w.sync = 0;
    w.hp = align256((size_t)tbl::kSyncWords * 4);
    w.qp = align256(w.hp + (size_t)m * inter * 8);
    w.dp = align256(w.qp + (size_t)m * inter / 4 * 8);
    w.sp = align256(w.dp + (size_t)m * nbi * 8);
    w.yp = align256(w.sp + (size_t)m * nbi * 8);
    w.total = align256(w.yp + (size_t)m * hidden * 8);
    return w;
}

int check_ffn_shapes(const tb_ffn_weights *L, int n, int *hidden, int *inter, int *fmt)
{
    for (int i = 0; i < n; ++i) {
        int rc;
        if ((rc = check_matrix(&L[i].gate)) || (rc = check_matrix(&L[i].up)) ||
            (rc = check_matrix(&L[i].down)))
            return rc;
        const int H = L[i].gate.k, N = L[i].gate.n, F = L[i].gate.fmt;
        if (F == TB_FMT_SIGN1_RI4)
            return TB_EUNSUPPORTED;
        if (L[i].up.k != H || L[i].up.n != N || L[i].down.k != N || L[i].down.n != H ||
            L[i].up.fmt != F || L[i].down.fmt != F || N % kBlock)
            return TB_EINVAL;
        if (i == 0) {
            *hidden = H;
            *inter = N;
            *fmt = F;
        } else if (H != *hidden || N != *inter || F != *fmt) {
            return TB_EINVAL;
        }
    }
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
    case TB_EUNSUPPORTED: return "shape not supported by the library on this device";
    case TB_EHIP: return "HIP runtime error";
    case TB_ESCRATCH: return "input larger than the library's static scratch";
    default: return "unknown status";
    }
}

static int rotate_quant_impl(const float *x, int m, int k, int8_t *q, float *dq, void *stream,
                             int max_rows)
{
    if (check_rows(m, max_rows) || k < kBlock || k % kBlock || !x || !q || !dq)
        return TB_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(dq))
        return TB_EALIGN;
    const Range rx = range_of(x, (size_t)m * k * 4), rq = range_of(q, (size_t)m * k),
                rd = range_of(dq, (size_t)m * (k / kBlock) * 4);
    if (overlaps(rx, rq) || overlaps(rx, rd) || overlaps(rq, rd))
        return TB_EINVAL;
    return launch_rotquant(x, m, k, q, dq, static_cast<hipStream_t>(stream));
}

int tb_rotate_quant_i8(const float *x, int m, int k, int8_t *q, float *dq, void *stream)
{
    return rotate_quant_impl(x, m, k, q, dq, stream, TB_MAX_ROWS);
}

int tb_rotate_quant_i8_batch(const float *x, int m, int k, int8_t *q, float *dq, void *stream)
{
    return rotate_quant_impl(x, m, k, q, dq, stream, TB_MAX_BATCH_ROWS);
}

static int gemv_impl(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                     void *stream, bool batch)
{
    int rc = check_matrix(w);
    if (rc)
        return rc;
    if (check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS) || !y || !q || !dq)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(dq) || !aligned16(y))
        return TB_EALIGN;
    const Range ry = range_of(y, (size_t)m * w->n * 4);
    if (overlaps(ry, range_of(w->codes, codes_bytes(w))) ||
        overlaps(ry, range_of(w->scales, scales_bytes(w))) ||
        overlaps(ry, range_of(q, (size_t)m * w->k)) ||
        overlaps(ry, range_of(dq, (size_t)m * (w->k / kBlock) * 4)))
        return TB_EINVAL;
    if (w->fmt == TB_FMT_SIGN1_RI4)
        return launch_lut(w, q, dq, m, y, nullptr, static_cast<hipStream_t>(stream));
    return (batch ? launch_gemv_batch : launch_gemv)(kModeY, w, nullptr, q, dq, m, y, nullptr,
                                                     static_cast<hipStream_t>(stream));
}

int tb_gemv_ternary(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                    void *stream)
{
    return gemv_impl(w, q, dq, m, y, stream, false);
}

int tb_gemv_ternary_batch(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                          void *stream)
{
    return gemv_impl(w, q, dq, m, y, stream, true);
}

static int gateup_impl(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                       const float *dq, int m, float *h, void *stream, bool batch)
{
    int rc = check_matrix(wg);
    if (rc)
        return rc;
    if ((rc = check_matrix(wu)))
        return rc;
    if (wg->n != wu->n || wg->k != wu->k || wg->fmt != wu->fmt)
        return TB_EINVAL;
    if (wg->fmt == TB_FMT_SIGN1_RI4)
        return TB_EUNSUPPORTED;
    if (check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS) || !h || !q || !dq)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(dq) || !aligned16(h))
        return TB_EALIGN;
    const Range rh = range_of(h, (size_t)m * wg->n * 4);
    if (overlaps(rh, range_of(wg->codes, codes_bytes(wg))) ||
        overlaps(rh, range_of(wg->scales, scales_bytes(wg))) ||
        overlaps(rh, range_of(wu->codes, codes_bytes(wu))) ||
        overlaps(rh, range_of(wu->scales, scales_bytes(wu))) ||
        overlaps(rh, range_of(q, (size_t)m * wg->k)) ||
        overlaps(rh, range_of(dq, (size_t)m * (wg->k / kBlock) * 4)))
        return TB_EINVAL;
    return (batch ? launch_gemv_batch : launch_gemv)(kModeGateUp, wg, wu, q, dq, m, h, nullptr,
                                                     static_cast<hipStream_t>(stream));
}

int tb_ffn_gateup_silu(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                       const float *dq, int m, float *h, void *stream)
{
    return gateup_impl(wg, wu, q, dq, m, h, stream, false);
}

int tb_ffn_gateup_silu_batch(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                             const float *dq, int m, float *h, void *stream)
{
    return gateup_impl(wg, wu, q, dq, m, h, stream, true);
}

int tb_ffn_gateup_silu_x(const tb_matrix *wg, const tb_matrix *wu, const float *x, int m,
                         int8_t *qx, float *dqx, float *h, void *stream)
{
    int rc = check_matrix(wg);
    if (rc)
        return rc;
    if ((rc = check_matrix(wu)))
        return rc;
    if (wg->n != wu->n || wg->k != wu->k || wg->fmt != wu->fmt)
        return TB_EINVAL;
    if (wg->fmt == TB_FMT_SIGN1_RI4)
        return TB_EUNSUPPORTED;
    if (check_rows(m, TB_MAX_ROWS) || !x || !qx || !dqx || !h)
        return TB_EINVAL;
    if (!aligned16(x) || !aligned16(qx) || !aligned16(dqx) || !aligned16(h))
        return TB_EALIGN;
    const int k = wg->k;
    const Range rx = range_of(x, (size_t)m * k * 4), rq = range_of(qx, (size_t)m * k),
                rd = range_of(dqx, (size_t)m * (k / kBlock) * 4),
                rh = range_of(h, (size_t)m * wg->n * 4);
    const Range outs[3] = {rq, rd, rh};
    const Range ins[5] = {rx, range_of(wg->codes, codes_bytes(wg)), range_of(wg->scales, scales_bytes(wg)),
                          range_of(wu->codes, codes_bytes(wu)), range_of(wu->scales, scales_bytes(wu))};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return TB_EINVAL;
    if (overlaps(rq, rd) || overlaps(rq, rh) || overlaps(rd, rh))
        return TB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = launch_gemv_rotx(kModeGateUp, wg, wu, x, m, qx, dqx, h, s);
    if (rc != TB_EUNSUPPORTED)
        return rc;
    if ((rc = launch_rotquant(x, m, k, qx, dqx, s)))
        return rc;
    return launch_gemv(kModeGateUp, wg, wu, qx, dqx, m, h, nullptr, s);
}

static int down_impl(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                     float *y, void *stream, bool batch)
{
    int rc = check_matrix(wd);
    if (rc)
        return rc;
    if (check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS) || !h || !qh_ws || !dqh_ws || !y)
        return TB_EINVAL;
    if (wd->fmt == TB_FMT_SIGN1_RI4)
        return TB_EUNSUPPORTED;
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
    if (!batch) {
        rc = launch_gemv_rotx(kModeY, wd, nullptr, h, m, qh_ws, dqh_ws, y, s);
        if (rc != TB_EUNSUPPORTED)
            return rc;
    }
    if ((rc = launch_rotquant(h, m, k, qh_ws, dqh_ws, s)))
        return rc;
    return (batch ? launch_gemv_batch : launch_gemv)(kModeY, wd, nullptr, qh_ws, dqh_ws, m, y,
                                                     nullptr, s);
}

int tb_ffn_down(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                float *y, void *stream)
{
    return down_impl(wd, h, m, qh_ws, dqh_ws, y, stream, false);
}

int tb_gemv_ternary_x(const tb_matrix *w, const float *x, int m, int8_t *qx, float *dqx, float *y,
                      void *stream)
{
    return down_impl(w, x, m, qx, dqx, y, stream, false);
}

int tb_ffn_down_batch(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                      float *y, void *stream)
{
    return down_impl(wd, h, m, qh_ws, dqh_ws, y, stream, true);
}

int tb_ffn_down_noalloc(const tb_matrix *wd, const float *h, int m, float *y, void *stream)
{
    int rc = check_matrix(wd);
    if (rc)
        return rc;
    if (wd->fmt == TB_FMT_SIGN1_RI4)
        return TB_EUNSUPPORTED;
    if (check_rows(m) || !h || !y)
        return TB_EINVAL;
    if (!aligned16(h) || !aligned16(y))
        return TB_EALIGN;
    const int k = wd->k;
    const Range rh = range_of(h, (size_t)m * k * 4), ry = range_of(y, (size_t)m * wd->n * 4);
    if (overlaps(ry, rh) || overlaps(ry, range_of(wd->codes, codes_bytes(wd))) ||
        overlaps(ry, range_of(wd->scales, scales_bytes(wd))))
        return TB_EINVAL;
    // rotquant(h) codes, then its block scales, each 256-byte aligned, inside the scratch
    const size_t q_bytes = ((size_t)m * k + 255) & ~(size_t)255;
    if (q_bytes + (size_t)m * (k / kBlock) * 4 > kNoAllocScratchBytes)
        return TB_ESCRATCH;
    uint8_t *base = nullptr;
    if ((rc = scratch_address(&base)))
        return rc;
    int8_t *qh = reinterpret_cast<int8_t *>(base);
    float *dqh = reinterpret_cast<float *>(base + q_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = launch_rotquant(h, m, k, qh, dqh, s)))
        return rc;
    return launch_gemv(kModeY, wd, nullptr, qh, dqh, m, y, nullptr, s);
}

static size_t down_split_workspace(const tb_matrix *wd, int m, bool batch)
{
    if (check_matrix(wd) || wd->fmt == TB_FMT_SIGN1_RI4 ||
        check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS))
        return 0;
    return split_workspace_bytes(wd, m);
}

size_t tb_ffn_down_split_workspace_bytes(const tb_matrix *wd, int m)
{
    return down_split_workspace(wd, m, false);
}

size_t tb_ffn_down_split_batch_workspace_bytes(const tb_matrix *wd, int m)
{
    return down_split_workspace(wd, m, true);
}

static int down_split_impl(const tb_matrix *wd, const float *h, int m, int8_t *qh, float *dqh,
                           float *y, void *ws, size_t ws_bytes, void *stream, bool batch)
{
    int rc = check_matrix(wd);
    if (rc)
        return rc;
    if (wd->fmt == TB_FMT_SIGN1_RI4)
        return TB_EUNSUPPORTED;
    if (check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS) || !h || !qh || !dqh || !y || !ws)
        return TB_EINVAL;
    if (!aligned16(h) || !aligned16(qh) || !aligned16(dqh) || !aligned16(y) || !aligned16(ws))
        return TB_EALIGN;
    const size_t need = split_workspace_bytes(wd, m);
    if (ws_bytes < need)
        return TB_EINVAL;
    const int k = wd->k;
    const Range rh = range_of(h, (size_t)m * k * 4), rq = range_of(qh, (size_t)m * k),
                rd = range_of(dqh, (size_t)m * (k / kBlock) * 4),
                ry = range_of(y, (size_t)m * wd->n * 4), rw = range_of(ws, need),
                rc_ = range_of(wd->codes, codes_bytes(wd)),
                rs = range_of(wd->scales, scales_bytes(wd));
    const Range outs[4] = {rq, rd, ry, rw};
    const Range ins[3] = {rh, rc_, rs};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return TB_EINVAL;
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j]))
                return TB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool tern = wd->fmt == TB_FMT_TERNARY2;
    if (m > TB_MAX_ROWS) {
        if (k >= TB_SPLIT_MIN_K) {
            rc = launch_down_split_wide(wd, h, m, qh, dqh, y, static_cast<float *>(ws), s);
            if (rc != TB_EUNSUPPORTED)
                return rc;
        }
        return down_impl(wd, h, m, qh, dqh, y, stream, true);
    }
    if (m >= TB_SPLIT_MIN_ROWS && (m < mfma_min_rows(tern, false) || k >= TB_SPLIT_MIN_K)) {
        rc = launch_down_split(wd, h, m, qh, dqh, y, static_cast<float *>(ws), s);
        if (rc != TB_EUNSUPPORTED)
            return rc;
    }
    return down_impl(wd, h, m, qh, dqh, y, stream, false);
}

int tb_ffn_down_split(const tb_matrix *wd, const float *h, int m, int8_t *qh, float *dqh, float *y,
                      void *ws, size_t ws_bytes, void *stream)
{
    return down_split_impl(wd, h, m, qh, dqh, y, ws, ws_bytes, stream, false);
}

int tb_ffn_down_split_batch(const tb_matrix *wd, const float *h, int m, int8_t *qh, float *dqh,
                            float *y, void *ws, size_t ws_bytes, void *stream)
{
    return down_split_impl(wd, h, m, qh, dqh, y, ws, ws_bytes, stream, true);
}

static int block_sums_impl(const tb_matrix *w, const int8_t *q, int m, int32_t *isum, void *stream,
                           bool batch)
{
    int rc = check_matrix(w);
    if (rc)
        return rc;
    if (check_rows(m, batch ? TB_MAX_BATCH_ROWS : TB_MAX_ROWS) || !q || !isum)
        return TB_EINVAL;
    if (!aligned16(q) || !aligned16(isum))
        return TB_EALIGN;
    // the sums of one launch (at most 16 rows) are written with 32-bit buffer offsets
    if ((size_t)(m < kMaxWideRows ? m : kMaxWideRows) * w->n * (w->k / kBlock) * 4 >= ((size_t)1 << 31))
        return TB_EUNSUPPORTED;
    const Range ri = range_of(isum, (size_t)m * w->n * (w->k / kBlock) * 4);
    if (overlaps(ri, range_of(w->codes, codes_bytes(w))) ||
        overlaps(ri, range_of(w->scales, scales_bytes(w))) ||
        overlaps(ri, range_of(q, (size_t)m * w->k)))
        return TB_EINVAL;
    if (w->fmt == TB_FMT_SIGN1_RI4)
        return launch_lut(w, q, nullptr, m, nullptr, isum, static_cast<hipStream_t>(stream));
    return (batch ? launch_gemv_batch : launch_gemv)(kModeIsum, w, nullptr, q, nullptr, m, nullptr,
                                                     isum, static_cast<hipStream_t>(stream));
}

int tb_gemv_block_sums(const tb_matrix *w, const int8_t *q, int m, int32_t *isum, void *stream)
{
    return block_sums_impl(w, q, m, isum, stream, false);
}

int tb_gemv_block_sums_batch(const tb_matrix *w, const int8_t *q, int m, int32_t *isum,
                             void *stream)
{
    return block_sums_impl(w, q, m, isum, stream, true);
}

int tb_sign_interleave(const tb_matrix *w, void *codes_ri, uint16_t *scales_ri, void *stream)
{
    int rc = check_matrix(w);
    if (rc)
        return rc;
    if (w->fmt != TB_FMT_SIGN1 || w->n % 4 || !codes_ri || !scales_ri)
        return TB_EINVAL;
    if (!aligned16(codes_ri) || !aligned16(scales_ri))
        return TB_EALIGN;
    const Range rco = range_of(codes_ri, codes_bytes(w)), rso = range_of(scales_ri, scales_bytes(w));
    if (overlaps(rco, rso) || overlaps(rco, range_of(w->codes, codes_bytes(w))) ||
        overlaps(rco, range_of(w->scales, scales_bytes(w))) ||
        overlaps(rso, range_of(w->codes, codes_bytes(w))) ||
        overlaps(rso, range_of(w->scales, scales_bytes(w))))
        return TB_EINVAL;
    const int nb = w->k / kBlock;
    const size_t words = (size_t)(w->n / 4) * nb * 16;
    const int grid = (int)std::min<size_t>((words + 255) / 256, 65536);
    hipLaunchKernelGGL(tblut::sign_interleave_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(w->codes),
                       w->scales, w->n, nb, static_cast<uint32_t *>(codes_ri), scales_ri);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}


size_t tb_ffn_workspace_bytes(int m, int hidden, int inter)
{
    if (check_rows(m) || inter < kBlock || inter % kBlock || hidden < kBlock || hidden % kBlock)
        return 0;
    return ws_layout(m, hidden, inter).total;
}

int tb_ffn_workspace_init(void *ws, size_t ws_bytes, uint32_t spin_ticks, void *stream)
{
    if (!ws || ws_bytes < (size_t)tbl::kSyncWords * 4)
        return TB_EINVAL;
    if (!aligned16(ws))
        return TB_EALIGN;
    const size_t words = ws_bytes / 4;
    const int grid = (int)std::min<size_t>(1024, (words + 1023) / 1024);
    hipLaunchKernelGGL(tbl::layers_ws_init_kernel, dim3(grid), dim3(1024), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t *>(ws), words, spin_ticks);
    return hipGetLastError() == hipSuccess ? TB_OK : TB_EHIP;
}

int tb_ffn_workspace_error(const void *ws, int *error)
{
    if (!ws || !error)
        return TB_EINVAL;
    uint32_t v = 0;
    if (hipMemcpy(&v, static_cast<const uint32_t *>(ws) + tbl::kWErr, 4, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return TB_EHIP;
    *error = (int)v;
    return TB_OK;
}

int tb_ffn_layers(const tb_ffn_weights *layers, int num_layers, const float *x, int m,
                  unsigned flags, void *ws, size_t ws_bytes, float *y, void *stream)
{
    if (!layers || num_layers < 1 || !x || !y || !ws || check_rows(m) || (flags & ~TB_FFN_CHAIN))
        return TB_EINVAL;
    int H = 0, N = 0, F = 0;
    int rc = check_ffn_shapes(layers, num_layers, &H, &N, &F);
    if (rc)
        return rc;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws))
        return TB_EALIGN;
    const WsLayout wl = ws_layout(m, H, N);
    if (ws_bytes < wl.total)
        return TB_EINVAL;
    const bool chain = (flags & TB_FFN_CHAIN) != 0;
    const Range rx = range_of(x, (size_t)(chain ? 1 : num_layers) * m * H * 4),
                ry = range_of(y, (size_t)num_layers * m * H * 4), rw = range_of(ws, wl.total);
    if (overlaps(rx, ry) || overlaps(rx, rw) || overlaps(ry, rw))
        return TB_EINVAL;
    for (int i = 0; i < num_layers; ++i) {
        const tb_matrix *mats[3] = {&layers[i].gate, &layers[i].up, &layers[i].down};
        for (const tb_matrix *w : mats)
            if (overlaps(ry, range_of(w->codes, codes_bytes(w))) ||
                overlaps(ry, range_of(w->scales, scales_bytes(w))) ||
                overlaps(rw, range_of(w->codes, codes_bytes(w))) ||
                overlaps(rw, range_of(w->scales, scales_bytes(w))))
                return TB_EINVAL;
    }
    // tagged entries are addressed with 32-bit buffer offsets
    if (wl.total >= ((size_t)1 << 31))
        return TB_EUNSUPPORTED;
    DeviceInfo info;
    if ((rc = device_info(&info)))
        return rc;
    // one workgroup per CU, all resident at once
    const int G = info.cus;
    const tbl::LdsPlan plan = tbl::lds_plan(m, F, H, N, G);
    if (plan.total > info.lds_limit)
        return TB_EUNSUPPORTED;
    // item tags: tile < 2^13 and step < 2^10 per CU
    if ((N / kRowsPerWave + G - 1) / G >= (1 << 13) || (H / kRowsPerWave + G - 1) / G >= (1 << 13) ||
        N / (F == TB_FMT_TERNARY2 ? 64 : 128) / 16 >= (1 << 10))
        return TB_EUNSUPPORTED;
    LayersFn fn = F == TB_FMT_TERNARY2 ? layers_pick_m<TB_FMT_TERNARY2>(m) : layers_pick_m<TB_FMT_SIGN1>(m);
    if (!fn)
        return TB_EINVAL;
    if ((rc = raise_lds(reinterpret_cast<const void *>(fn), (size_t)plan.total)))
        return rc;

    uint8_t *wsb = static_cast<uint8_t *>(ws);
    tbl::LArgs a;
    a.H = H;
    a.N = N;
    a.sync = reinterpret_cast<uint32_t *>(wsb + wl.sync);
    a.hp = reinterpret_cast<uint64_t *>(wsb + wl.hp);
    a.qp = reinterpret_cast<uint64_t *>(wsb + wl.qp);
    a.dp = reinterpret_cast<uint64_t *>(wsb + wl.dp);
    a.sp = reinterpret_cast<uint64_t *>(wsb + wl.sp);
    a.yp = reinterpret_cast<uint64_t *>(wsb + wl.yp);
    a.gu_cb = (uint32_t)codes_bytes(&layers[0].gate);
    a.gu_sb = (uint32_t)((scales_bytes(&layers[0].gate) + 3) & ~(size_t)3);
    a.d_cb = (uint32_t)codes_bytes(&layers[0].down);
    a.d_sb = (uint32_t)((scales_bytes(&layers[0].down) + 3) & ~(size_t)3);
    a.unit = dq_unit();
    hipStream_t s = static_cast<hipStream_t>(stream);
    // at most kMaxLayers per launch; a chained sequence continues from the last y
    for (int start = 0; start < num_layers; start += tbl::kMaxLayers) {
        const int cnt = std::min(tbl::kMaxLayers, num_layers - start);
        a.L = cnt;
        for (int i = 0; i < tbl::kMaxLayers; ++i) {
            const tb_ffn_weights &w = layers[start + (i < cnt ? i : 0)];
            a.layer[i].codes[0] = static_cast<const uint8_t *>(w.gate.codes);
            a.layer[i].codes[1] = static_cast<const uint8_t *>(w.up.codes);
            a.layer[i].codes[2] = static_cast<const uint8_t *>(w.down.codes);
            a.layer[i].scales[0] = w.gate.scales;
            a.layer[i].scales[1] = w.up.scales;
            a.layer[i].scales[2] = w.down.scales;
        }
        a.chain = chain ? 1 : 0;
        a.x = chain ? (start == 0 ? x : y + (size_t)(start - 1) * m * H) : x + (size_t)start * m * H;
        a.y = y + (size_t)start * m * H;
        hipLaunchKernelGGL(fn, dim3(G), dim3(tbl::layers_threads(F, m)), plan.total, s, a);
        if (hipGetLastError() != hipSuccess)
            return TB_EHIP;
    }
    return TB_OK;
}

}  // extern "C"

// tb_fused.h -- the fused FFN kernel: one persistent launch runs L FFN layers (gfx950).
//
// One FFN layer, after "perf(bonsai): decode and small packed batches read the FFN from a
// ternary copy through a dp4a GEMV" (sparkinfer PR #1154, Summary and commit message):
// rotate + quantise x (one int8 copy shared by gate and up), gate/up GEMVs and the SiLU
// gate, rotate + quantise h, down GEMV. Every row is computed by the same device blocks
// as the separate entry points (tb_device.h), so a layer's outputs are bit-identical to
// tb_rotate_quant_i8 + tb_ffn_gateup_silu + tb_ffn_down on the same inputs, for every M.
//
// Why one launch: on MI355X a dependent kernel launch costs about 4 us of lost streaming
// (launch, ramp-up, tail), against 9.9 us for the whole layer's weights at the measured
// 7.2 TB/s. Here one workgroup per CU stays resident for all L layers and its weight ring
// keeps loading across the layer's three synchronisation points:
//   A  all h rows written           -> the h blocks can be rotated and quantised
//   B  all q_h blocks written       -> the down GEMV can stage q_h
//   C  all y rows of the layer done -> the next layer may start (arrived at the end of a
//      layer, waited for at the start of the next, so the wait overlaps the ring)
// Each point is a grid barrier on 16 counters (a workgroup arrives on counter
// blockIdx % 16; waiters read all 16), which spreads the atomics over 16 cache lines.
//
// Memory between workgroups of the launch (h, q_h, dq_h, sum q_h, chained y) is written
// with device-coherent stores (sc1) and read with device-coherent loads; before arriving
// at a barrier a workgroup waits for all its memory operations to complete.
//
// Every wait is bounded by a spin limit on the 100 MHz realtime counter. A wait that runs
// out sets a sticky error word in the workspace and every workgroup skips the rest of the
// work, so the grid always drains. Later launches on the same workspace exit at once until
// the workspace is initialised again.
#pragma once

#include "tb_device.h"

namespace tbk {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = 64 * kFusedWaves;
constexpr int kFusedDepth = 4;
constexpr int kMaxFusedLayers = 32;
constexpr int kFusedGroups = kFusedThreads / 16;   // 16-lane groups per workgroup

// Workspace sync words (uint32), each on its own 256-byte line.
constexpr int kSyncStride = 64;
constexpr int kSyncError = 0;
constexpr int kSyncExit = 1 * kSyncStride;
constexpr int kSyncSpin = 2 * kSyncStride;
constexpr int kSyncBar = 3 * kSyncStride;   // 16 barrier counters
constexpr int kBarCounters = 16;
constexpr int kSyncWords = (3 + kBarCounters) * kSyncStride;
constexpr uint32_t kDefaultSpinTicks = 10000000u;   // 100 ms of the 100 MHz clock
constexpr int kAuxCoherent = 16;                     // sc1: device-scope coherent access

struct FusedLayer {
    const uint8_t *codes[3];    // gate, up, down
    const uint16_t *scales[3];
};

struct FusedArgs {
    FusedLayer layer[kMaxFusedLayers];
    int L, hidden, inter, chain;
    const float *x;   // [L][M][hidden], or [M][hidden] when chained
    float *y;         // [L][M][hidden]
    uint32_t *sync;   // workspace: sync words
    float *h;         // workspace: [M][inter]
    int8_t *qh;       // workspace: [M][inter]
    float *dqh;       // workspace: [M][inter/128]
    int *qsumh;       // workspace: [M][inter/128]
    uint32_t gu_codes_bytes, gu_scales_bytes, d_codes_bytes, d_scales_bytes;
    float unit;
};

__device__ __forceinline__ uint32_t sync_load(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sync_add(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wave issued has completed (stores acknowledged).
__device__ __forceinline__ void drain_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint4 buffer_load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxCoherent);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Eight consecutive floats (32 bytes at byte offset off), device-coherent. The words go
// through scalar locals: a bit_cast applied directly to a vector element reads element 0.
__device__ __forceinline__ void load8_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[8])
{
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxCoherent);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kAuxCoherent);
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float(w[e]);
}
__device__ __forceinline__ void buffer_store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                      uint32_t v, int soffset)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, soffset, kAuxCoherent);
}

// Grid barrier instance `inst` (0, 1, 2, ... within the launch). Arrive: one atomic by
// thread 0 after the whole workgroup has drained its memory operations.
__device__ __forceinline__ void bar_arrive(uint32_t *sync)
{
    drain_memory();
    __syncthreads();
    if (threadIdx.x == 0)
        sync_add(sync + kSyncBar + (blockIdx.x % kBarCounters) * kSyncStride, 1u);
}

// Wait for instance `inst`: counter c must reach (inst + 1) * (number of workgroups that
// arrive on c). Lanes 0..15 of wave 0 read one counter each. Returns false on timeout or
// on an error raised by another workgroup (the caller then abandons the work).
__device__ bool bar_wait(uint32_t *sync, int inst, uint32_t spin_ticks, int *abort_lds)
{
    if (threadIdx.x < 64) {
        const int c = threadIdx.x & (kBarCounters - 1);
        const uint32_t G = gridDim.x;
        const uint32_t per = (G + kBarCounters - 1 - c) / kBarCounters;   // wgs with id % 16 == c
        const uint32_t target = (uint32_t)(inst + 1) * per;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            const uint32_t v = sync_load(sync + kSyncBar + c * kSyncStride);
            const bool ready = __all((int)(v - target) >= 0);
            if (ready)
                break;
            if (sync_load(sync + kSyncError) != 0u) {
                if (threadIdx.x == 0)
                    *abort_lds = 1;
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
                if (threadIdx.x == 0) {
                    sync_store(sync + kSyncError, 1u);
                    *abort_lds = 1;
                }
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    return *abort_lds == 0;
}

// Stage int8 activations already in LDS (natural order, [m][k]) into the step layout.
template <int M, int FMT>
__device__ __forceinline__ void stage_from_lds(uint8_t *act, const int8_t *qnat, int k)
{
    const int per_row = (FMT == TB_FMT_TERNARY2 ? k / 64 : k / 128) * 4;
    const int units = M * per_row;
    for (int u = threadIdx.x; u < units; u += kFusedThreads) {
        StageUnit<FMT> su;
        stage_unit_load_step<M, FMT, false>(su, qnat, k, u);
        stage_unit_store_step<M, FMT>(su, act, k, u);
    }
}

// Stage int8 activations written by other workgroups (global [m][k]) into the step layout.
// Each thread issues the loads of up to kStageBatch units before it stores any, so the
// staging costs about one memory round trip per batch instead of one per unit.
constexpr int kStageBatch = 4;
template <int M, int FMT>
__device__ __forceinline__ void stage_from_global_coherent(uint8_t *act, const int8_t *q, int k,
                                                           uint32_t q_bytes)
{
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(q, q_bytes);
    const int per_row = (FMT == TB_FMT_TERNARY2 ? k / 64 : k / 128) * 4;
    const int units = M * per_row;
    for (int u0 = threadIdx.x; u0 < units; u0 += kStageBatch * kFusedThreads) {
        StageUnit<FMT> su[kStageBatch];
#pragma unroll
        for (int i = 0; i < kStageBatch; ++i) {
            const int u = u0 + i * kFusedThreads;
            const int m = u / per_row, g = u % per_row;
            const int c = g >> 2, j = g & 3;
            const bool in = u < units;
            if (FMT == TB_FMT_TERNARY2) {
                su[i].lo = buffer_load16_coherent(r, in ? (uint32_t)(m * k + c * 64 + j * 16) : kOutOfRange);
            } else {
                const uint32_t off = in ? (uint32_t)(m * k + c * 128 + j * 32) : kOutOfRange;
                su[i].lo = buffer_load16_coherent(r, off);
                su[i].hi = buffer_load16_coherent(r, in ? off + 16 : kOutOfRange);
            }
        }
#pragma unroll
        for (int i = 0; i < kStageBatch; ++i) {
            const int u = u0 + i * kFusedThreads;
            if (u < units)
                stage_unit_store_step<M, FMT>(su[i], act, k, u);
        }
    }
}

// Rotate + quantise x ([M][H], read device-coherently) into LDS: q in natural order,
// dq and the code sums as block terms [b][m]. One 16-lane group per 128-block; a group
// loads up to kXBatch blocks before it computes any, so the loads share one round trip.
constexpr int kXBatch = 3;
template <int M>
__device__ __forceinline__ void rotquant_x_to_lds(__amdgpu_buffer_rsrc_t r_x, int H, float unit,
                                                  int8_t *qnat, float *dq_s, int *qs_s)
{
    const int nbh = H / kBlock, total = M * nbh;
    const int lane16 = threadIdx.x & 15;
    for (int p0 = threadIdx.x >> 4; p0 < total; p0 += kXBatch * kFusedGroups) {
        float v[kXBatch][8];
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
            const int p = p0 + i * kFusedGroups;
            const uint32_t off =
                p < total ? (uint32_t)(((p / nbh) * H + (p % nbh) * kBlock + lane16 * 8) * 4) : kOutOfRange;
            load8_coherent(r_x, off, v[i]);
        }
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
            const int p = p0 + i * kFusedGroups;
            if (p < total) {   // the same for the 16 lanes of a group
                const int m = p / nbh, b = p % nbh;
                uint32_t packed[2];
                float dq;
                int qsum;
                rotquant_regs(v[i], lane16, unit, packed, dq, qsum);
                *reinterpret_cast<uint2 *>(qnat + m * H + b * kBlock + lane16 * 8) =
                    make_uint2(packed[0], packed[1]);
                if (lane16 == 0) {
                    dq_s[b * M + m] = dq;
                    qs_s[b * M + m] = qsum;
                }
            }
        }
    }
}

template <int M, int FMT>
__global__ __launch_bounds__(kFusedThreads) void ffn_layers_kernel(FusedArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    using L_ = StepLayout<M, FMT>;
    constexpr int kWpc = Fmt<FMT>::kWeightsPerChunk;
    constexpr int kCpb = Fmt<FMT>::kChunksPerBlock;
    constexpr int kBps = kChunkLanes / kCpb;   // blocks per step
    constexpr int D = kFusedDepth;

    const int H = a.hidden, N = a.inter;
    const int nbh = H / kBlock, nbi = N / kBlock;
    // phase 0: gate/up (rows N, inputs H); phase 1: down (rows H, inputs N)
    const int C0 = H / kWpc, C1 = N / kWpc;
    const int I0 = (C0 + kChunkLanes - 1) / kChunkLanes, I1 = (C1 + kChunkLanes - 1) / kChunkLanes;
    const int T0 = N / kRowsPerWave, T1 = H / kRowsPerWave;
    const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15, rl = lane >> 4;
    // the wave index is the same in every lane; saying so lets the compiler keep the whole
    // item schedule (and the weight descriptors built from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, GW = G * kFusedWaves;
    const int t0 = blockIdx.x + G * wave;   // first tile of this wave (both phases)
    const int NT0 = t0 < T0 ? (T0 - t0 + GW - 1) / GW : 0;
    const int NT1 = t0 < T1 ? (T1 - t0 + GW - 1) / GW : 0;
    const int J0 = NT0 * I0, J1 = NT1 * I1;
    const int J0p = (J0 + D - 1) / D * D, J1p = (J1 + D - 1) / D * D;
    const uint32_t rb0b = (uint32_t)C0 * 16u, rb1b = (uint32_t)C1 * 16u;   // code bytes per row
    const uint32_t rag0 = (C0 % kChunkLanes != 0 && cl >= C0 % kChunkLanes) ? kOutOfRange : 0u;
    const uint32_t rag1 = (C1 % kChunkLanes != 0 && cl >= C1 % kChunkLanes) ? kOutOfRange : 0u;

    // ---- LDS: step layout | block terms [b][m] (+ one step of zero padding) | flags ------
    const int act_bytes = max(I1 * L_::kStepBytes, I0 * L_::kStepBytes + M * H);
    uint8_t *act = lds;
    int8_t *qnat = reinterpret_cast<int8_t *>(lds + I0 * L_::kStepBytes);   // phase-0 staging
    const int nbmax = max(nbh, nbi) + kBps;
    float *dq_s = reinterpret_cast<float *>(lds + act_bytes);
    int *qs_s = reinterpret_cast<int *>(dq_s + nbmax * M);
    int *abort_lds = qs_s + nbmax * M;

    uint32_t *sync = a.sync;
    if (tid == 0)
        *abort_lds = sync_load(sync + kSyncError) != 0u ? 1 : 0;
    const uint32_t spin_word = sync_load(sync + kSyncSpin);
    const uint32_t spin_ticks = spin_word ? spin_word : kDefaultSpinTicks;
    __syncthreads();
    bool alive = *abort_lds == 0;

    const __amdgpu_buffer_rsrc_t r_h = buffer_rsrc(a.h, (uint32_t)(M * N * 4));
    const __amdgpu_buffer_rsrc_t r_qh = buffer_rsrc(a.qh, (uint32_t)(M * N));
    const __amdgpu_buffer_rsrc_t r_dqh = buffer_rsrc(a.dqh, (uint32_t)(M * nbi * 4));
    const __amdgpu_buffer_rsrc_t r_qsh = buffer_rsrc(a.qsumh, (uint32_t)(M * nbi * 4));

    // ---- load side: (layer, phase, j) walks every layer's padded item lists in order ----
    int ll = 0, lp = 0, lj = 0, lstep = 0;
    uint32_t lrow = (uint32_t)(t0 * kRowsPerWave + rl), loff = 0, lsoff = 0;
    __amdgpu_buffer_rsrc_t rc0, rc1, rs0, rs1;
    auto set_phase = [&]() {
        lj = 0;
        lstep = 0;
        lrow = (uint32_t)(t0 * kRowsPerWave + rl);
        const uint32_t rowb = lp ? rb1b : rb0b;
        const uint32_t nb = (uint32_t)(lp ? nbi : nbh);
        loff = lrow * rowb + (uint32_t)cl * 16u;
        lsoff = (lrow * nb + (uint32_t)(cl / kCpb)) * 2u;
        const int li = ll < a.L ? ll : 0;
        if (lp == 0) {
            rc0 = buffer_rsrc(a.layer[li].codes[0], a.gu_codes_bytes);
            rs0 = buffer_rsrc(a.layer[li].scales[0], a.gu_scales_bytes);
            rc1 = buffer_rsrc(a.layer[li].codes[1], a.gu_codes_bytes);
            rs1 = buffer_rsrc(a.layer[li].scales[1], a.gu_scales_bytes);
        } else {
            rc0 = buffer_rsrc(a.layer[li].codes[2], a.d_codes_bytes);
            rs0 = buffer_rsrc(a.layer[li].scales[2], a.d_scales_bytes);
            rc1 = rc0;
            rs1 = rs0;
        }
    };
    set_phase();
    auto issue = [&](uint4 &w0, uint4 &w1, uint32_t &s0, uint32_t &s1) {
        const int I = lp ? I1 : I0, J = lp ? J1 : J0, Jp = lp ? J1p : J0p;
        const bool real = alive && ll < a.L && lj < J;
        const uint32_t extra = lstep == I - 1 ? (lp ? rag1 : rag0) : 0u;
        const uint32_t off = real ? loff + extra : kOutOfRange;
        const uint32_t soff = real ? (lsoff & ~3u) + extra : kOutOfRange;
        w0 = buffer_load16_nt(rc0, off);
        s0 = buffer_load_u32(rs0, soff);
        w1 = buffer_load16_nt(rc1, lp == 0 ? off : kOutOfRange);
        s1 = buffer_load_u32(rs1, lp == 0 ? soff : kOutOfRange);
        if (lj < J) {
            if (++lstep == I) {
                lstep = 0;
                lrow += (uint32_t)(GW * kRowsPerWave);
                const uint32_t rowb = lp ? rb1b : rb0b;
                const uint32_t nb = (uint32_t)(lp ? nbi : nbh);
                loff = lrow * rowb + (uint32_t)cl * 16u;
                lsoff = (lrow * nb + (uint32_t)(cl / kCpb)) * 2u;
            } else {
                loff += 16u * kChunkLanes;
                lsoff += 2u * kBps;
            }
        }
        if (++lj == Jp) {
            lp ^= 1;
            if (lp == 0)
                ++ll;
            set_phase();
        }
    };

    uint4 rw0[D], rw1[D];
    uint32_t rsc0[D], rsc1[D];
    // a phase with no items for this wave has Jp == 0: skip such phases before the prologue
    // and inside issue() (the while handles consecutive empty phases)
    auto skip_empty = [&]() {
        int guard = 0;
        while (ll < a.L && (lp ? J1p : J0p) == 0 && guard < 2 * kMaxFusedLayers + 2) {
            lp ^= 1;
            if (lp == 0)
                ++ll;
            set_phase();
            ++guard;
        }
    };
    skip_empty();
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue(rw0[d], rw1[d], rsc0[d], rsc1[d]);
        skip_empty();
    }

    int inst = 0;   // barrier instances used so far
    for (int l = 0; l < a.L; ++l) {
        // ---- P0: wait for the previous layer, rotate + quantise x into LDS -------------
        if (l > 0)
            alive = alive && bar_wait(sync, inst - 1, spin_ticks, abort_lds);
        if (alive) {
            const float *xl = a.chain && l > 0 ? a.y + (size_t)(l - 1) * M * H
                                               : a.x + (size_t)(a.chain ? 0 : l) * M * H;
            // read coherently: with chaining, x is the previous layer's y from other workgroups
            const __amdgpu_buffer_rsrc_t r_x = buffer_rsrc(xl, (uint32_t)(M * H * 4));
            rotquant_x_to_lds<M>(r_x, H, a.unit, qnat, dq_s, qs_s);
            for (int i = tid; i < kBps * M; i += kFusedThreads) {   // zero padding blocks
                dq_s[nbh * M + i] = 0.0f;
                qs_s[nbh * M + i] = 0;
            }
            __syncthreads();
            stage_from_lds<M, FMT>(act, qnat, H);
            __syncthreads();
        }

        // ---- P1: gate/up items, h rows to the workspace ---------------------------------
        float acc0[M], acc1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            acc0[m] = 0.0f;
            acc1[m] = 0.0f;
        }
        {
            int cj = 0, cstep = 0;
            uint32_t crow = (uint32_t)(t0 * kRowsPerWave + rl);
            const uint8_t *cact = act + cl * 16;
            int cblk = cl / kCpb;
            uint32_t cshift = ((crow * (uint32_t)nbh + (uint32_t)cblk) & 1u) * 16u;
            for (int j0 = 0; j0 < J0p; j0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const bool real = alive && cj < J0;
                    if (real) {
                        int is0[M], is1[M];
                        chunk_sums_step<M, FMT, true>(rw0[d], rw1[d], cact, is0, is1);
                        const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(rsc0[d], cshift, 16));
                        const float s1 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(rsc1[d], cshift, 16));
                        // the step partial: row tree of the lanes' terms, added in step order
                        float p0[M], p1[M];
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            int v0 = is0[m], v1 = is1[m];
                            if (FMT == TB_FMT_SIGN1) {
                                v0 = 2 * v0 - qs_s[cblk * M + m];
                                v1 = 2 * v1 - qs_s[cblk * M + m];
                            }
                            const float dqv = dq_s[cblk * M + m];
                            p0[m] = (s0 * dqv) * (float)v0;
                            p1[m] = (s1 * dqv) * (float)v1;
                        }
                        row_tree<M, FMT, true>(p0, p1);
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            acc0[m] += p0[m];
                            acc1[m] += p1[m];
                        }
                    }
                    issue(rw0[d], rw1[d], rsc0[d], rsc1[d]);
                    skip_empty();
                    if (real) {
                        if (++cstep == I0) {
                            const bool wr = cl == 0;
#pragma unroll
                            for (int m = 0; m < M; ++m) {
                                buffer_store_coherent(r_h, wr ? crow * 4u : kOutOfRange,
                                                      __builtin_bit_cast(uint32_t, silu_gate(acc0[m], acc1[m])),
                                                      m * N * 4);
                                acc0[m] = 0.0f;
                                acc1[m] = 0.0f;
                            }
                            cstep = 0;
                            crow += (uint32_t)(GW * kRowsPerWave);
                            cact = act + cl * 16;
                            cblk = cl / kCpb;
                            cshift = ((crow * (uint32_t)nbh + (uint32_t)cblk) & 1u) * 16u;
                        } else {
                            cact += L_::kStepBytes;
                            cblk += kBps;
                        }
                    }
                    ++cj;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        bar_arrive(sync);   // A
        ++inst;

        // ---- P2: rotate + quantise h, spread over all workgroups -------------------------
        alive = alive && bar_wait(sync, inst - 1, spin_ticks, abort_lds);
        if (alive) {
            for (int p = blockIdx.x + G * (tid >> 4); p < M * nbi; p += G * kFusedGroups) {
                const int m = p / nbi, b = p % nbi;
                const uint32_t off = (uint32_t)((m * N + b * kBlock + (lane & 15) * 8) * 4);
                float v[8];
                load8_coherent(r_h, off, v);
                uint32_t packed[2];
                float dq;
                int qsum;
                rotquant_regs(v, lane & 15, a.unit, packed, dq, qsum);
                const uint32_t qoff = (uint32_t)(m * N + b * kBlock + (lane & 15) * 8);
                buffer_store_coherent(r_qh, qoff, packed[0], 0);
                buffer_store_coherent(r_qh, qoff + 4, packed[1], 0);
                const bool w0 = (lane & 15) == 0;
                buffer_store_coherent(r_dqh, w0 ? (uint32_t)((m * nbi + b) * 4) : kOutOfRange,
                                      __builtin_bit_cast(uint32_t, dq), 0);
                buffer_store_coherent(r_qsh, w0 ? (uint32_t)((m * nbi + b) * 4) : kOutOfRange,
                                      (uint32_t)qsum, 0);
            }
        }
        bar_arrive(sync);   // B
        ++inst;

        // ---- P3: stage q_h, down items, y rows -----------------------------------------
        alive = alive && bar_wait(sync, inst - 1, spin_ticks, abort_lds);
        if (alive) {
            stage_from_global_coherent<M, FMT>(act, a.qh, N, (uint32_t)(M * N));
            for (int i = tid; i < nbmax * M; i += kFusedThreads) {
                const int b = i / M, m = i % M;
                const bool in = b < nbi;
                const uint32_t o = in ? (uint32_t)((m * nbi + b) * 4) : kOutOfRange;
                dq_s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_dqh, o, 0, kAuxCoherent));
                qs_s[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_qsh, o, 0, kAuxCoherent);
            }
            __syncthreads();
        }
        {
            float *yl = a.y + (size_t)l * M * H;
            const __amdgpu_buffer_rsrc_t r_y = buffer_rsrc(yl, (uint32_t)(M * H * 4));
            int cj = 0, cstep = 0;
            uint32_t crow = (uint32_t)(t0 * kRowsPerWave + rl);
            const uint8_t *cact = act + cl * 16;
            int cblk = cl / kCpb;
            uint32_t cshift = ((crow * (uint32_t)nbi + (uint32_t)cblk) & 1u) * 16u;
            for (int j0 = 0; j0 < J1p; j0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const bool real = alive && cj < J1;
                    if (real) {
                        int is0[M], is1[M];
                        chunk_sums_step<M, FMT, false>(rw0[d], rw1[d], cact, is0, is1);
                        const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(rsc0[d], cshift, 16));
                        // the step partial: row tree of the lanes' terms, added in step order
                        float p0[M], p1[M];
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            int v0 = is0[m];
                            if (FMT == TB_FMT_SIGN1)
                                v0 = 2 * v0 - qs_s[cblk * M + m];
                            p0[m] = (s0 * dq_s[cblk * M + m]) * (float)v0;
                            p1[m] = 0.0f;
                        }
                        row_tree<M, FMT, false>(p0, p1);
#pragma unroll
                        for (int m = 0; m < M; ++m)
                            acc0[m] += p0[m];
                    }
                    issue(rw0[d], rw1[d], rsc0[d], rsc1[d]);
                    skip_empty();
                    if (real) {
                        if (++cstep == I1) {
                            const bool wr = cl == 0;
#pragma unroll
                            for (int m = 0; m < M; ++m) {
                                buffer_store_coherent(r_y, wr ? crow * 4u : kOutOfRange,
                                                      __builtin_bit_cast(uint32_t, acc0[m]), m * H * 4);
                                acc0[m] = 0.0f;
                            }
                            cstep = 0;
                            crow += (uint32_t)(GW * kRowsPerWave);
                            cact = act + cl * 16;
                            cblk = cl / kCpb;
                            cshift = ((crow * (uint32_t)nbi + (uint32_t)cblk) & 1u) * 16u;
                        } else {
                            cact += L_::kStepBytes;
                            cblk += kBps;
                        }
                    }
                    ++cj;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        bar_arrive(sync);   // C (waited for at the start of the next layer)
        ++inst;
    }

    // ---- exit: the last workgroup out resets the counters for the next launch -----------
    drain_memory();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = sync_add(sync + kSyncExit, 1u);
        if (old == (uint32_t)G - 1u) {
            for (int c = 0; c < kBarCounters; ++c)
                sync_store(sync + kSyncBar + c * kSyncStride, 0u);
            sync_store(sync + kSyncExit, 0u);
        }
    }
}

// Zero the sync words and set the spin limit (a kernel, not a memset: safe in graphs).
__global__ void ffn_workspace_init_kernel(uint32_t *sync, uint32_t spin_ticks)
{
    for (int i = threadIdx.x; i < kSyncWords; i += blockDim.x)
        sync[i] = i == kSyncSpin ? spin_ticks : 0u;
}

}  // namespace tbk

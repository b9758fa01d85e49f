// tb_fused_lr.h -- the fused FFN kernel with dedicated loader waves (gfx950).
//
// Same computation, same device blocks and same outputs as ffn_layers_kernel (tb_fused.h):
// per layer rotate + quantise x, gate/up + SiLU gate, rotate + quantise h, down; every
// output bit-identical to the separate entry points. What changes is who loads the
// weights.
//
// In ffn_layers_kernel the waves that compute also stream the weights through a register
// ring. A wave waiting at a grid barrier issues nothing, and before it arrives it must
// wait for its outstanding weight loads too (one counter covers loads and stores), so the
// weight stream stops at every synchronisation point of the layer.
//
// Here a workgroup of 16 waves is split in two:
//   * 8 consumer waves run the layer exactly as before, but read their weights from LDS;
//   * 8 loader waves, one per consumer, walk that consumer's weight units (a unit is one
//     wave-wide item: 64 lanes x 16 code bytes + 64 scale words) and copy them from HBM,
//     through a register ring, into a per-consumer LDS ring of U units.
// A loader never takes part in a barrier, so the weight stream keeps running while its
// consumer waits, until that consumer's LDS ring is full. A consumer has no weight loads
// outstanding, so draining its stores before a barrier is cheap.
//
// Loader and consumer synchronise through two LDS counters per pair: units filled
// (written by the loader after the unit's bytes) and units consumed (written by the
// consumer after it has read the unit). LDS operations of one wave take effect in
// order, which is what makes "bytes, then counter" and "read, then counter" sufficient.
// Consumers synchronise among themselves with an LDS counter barrier (s_barrier would
// need the loader waves too). Every wait is bounded by the workspace's spin limit.
#pragma once

#include "tb_fused.h"

namespace tbk {

constexpr int kLrConsumers = 8;
constexpr int kLrThreads = 2 * 64 * kLrConsumers;   // 16 waves
constexpr int kUnitBytes = 1280;                    // 1024 code bytes + 256 scale-word bytes
constexpr int kLoaderDepth = 4;                     // units in flight per loader wave
constexpr int kMaxRingUnits = 16;
constexpr int kMinRingUnits = 4;
// LDS control words
constexpr int kCtlFilled = 0;      // [kLrConsumers] units written by each loader
constexpr int kCtlConsumed = 8;    // [kLrConsumers] units read by each consumer
constexpr int kCtlBar = 16;        // consumer barrier arrivals
constexpr int kCtlAbort = 17;      // nonzero: abandon the work
constexpr int kCtlWords = 32;

__device__ __forceinline__ int lds_ld(const int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

__device__ __forceinline__ void raise_error(uint32_t *sync, int *ctl)
{
    sync_store(sync + kSyncError, 1u);
    lds_st(ctl + kCtlAbort, 1);
}

// Barrier of the consumer waves only (LDS counter; `gen` counts this wave's barriers).
__device__ __forceinline__ void cbar(uint32_t *sync, int *ctl, int &gen, uint32_t spin_ticks)
{
    compiler_fence();
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctl + kCtlBar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int target = (++gen) * kLrConsumers;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 1; __builtin_amdgcn_readfirstlane(lds_ld(ctl + kCtlBar)) < target; ++it) {
        if ((it & 15) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
            raise_error(sync, ctl);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    compiler_fence();
}

// Grid barrier arrive / wait for the consumer waves (see bar_arrive / bar_wait).
__device__ __forceinline__ void lr_arrive(uint32_t *sync, int *ctl, int &gen, uint32_t spin_ticks)
{
    drain_memory();
    cbar(sync, ctl, gen, spin_ticks);
    if (threadIdx.x == 0)
        sync_add(sync + kSyncBar + (blockIdx.x % kBarCounters) * kSyncStride, 1u);
}

__device__ bool lr_wait(uint32_t *sync, int inst, uint32_t spin_ticks, int *ctl, int &gen)
{
    if (threadIdx.x < 64) {
        const int c = threadIdx.x & (kBarCounters - 1);
        const uint32_t G = gridDim.x;
        const uint32_t per = (G + kBarCounters - 1 - c) / kBarCounters;
        const uint32_t target = (uint32_t)(inst + 1) * per;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            const uint32_t v = sync_load(sync + kSyncBar + c * kSyncStride);
            if (__all((int)(v - target) >= 0))
                break;
            if (sync_load(sync + kSyncError) != 0u || lds_ld(ctl + kCtlAbort) != 0) {
                lds_st(ctl + kCtlAbort, 1);
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
                raise_error(sync, ctl);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    cbar(sync, ctl, gen, spin_ticks);
    return lds_ld(ctl + kCtlAbort) == 0;
}

// One consumer item in registers: the code words and scale words of gate and up (w1/s1
// unused for down). (Activations stay in LDS: holding the next step's activations too
// would need more than the 128 registers a 16-wave workgroup allows.)
template <int M, int FMT>
constexpr bool kPrefetchAct = false;

template <int M, int FMT, bool kAct = kPrefetchAct<M, FMT>>
struct LrItem {
    uint4 w0, w1;
    uint32_t s0, s1;
    uint4 av[StepLayout<M, FMT>::kPlanes][M];
};
template <int M, int FMT>
struct LrItem<M, FMT, false> {
    uint4 w0, w1;
    uint32_t s0, s1;
};

// LDS bytes before the rings (act, block terms, control words), 16-byte aligned.
__host__ __device__ constexpr int lr_ring_offset(int act_bytes, int nbmax, int m)
{
    return ((act_bytes + 2 * nbmax * m * 4 + kCtlWords * 4) + 15) & ~15;
}

template <int M, int FMT>
__global__ __launch_bounds__(kLrThreads) void ffn_layers_lr_kernel(FusedArgs a, int U)
{
    extern __shared__ __align__(16) uint8_t lds[];
    using L_ = StepLayout<M, FMT>;
    constexpr int kWpc = Fmt<FMT>::kWeightsPerChunk;
    constexpr int kCpb = Fmt<FMT>::kChunksPerBlock;
    constexpr int kBps = kChunkLanes / kCpb;   // blocks per step
    constexpr int D = kLoaderDepth;

    const int H = a.hidden, N = a.inter;
    const int nbh = H / kBlock, nbi = N / kBlock;
    // phase 0: gate/up (rows N, inputs H); phase 1: down (rows H, inputs N)
    const int C0 = H / kWpc, C1 = N / kWpc;
    const int I0 = (C0 + kChunkLanes - 1) / kChunkLanes, I1 = (C1 + kChunkLanes - 1) / kChunkLanes;
    const int T0 = N / kRowsPerWave, T1 = H / kRowsPerWave;
    const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15, rl = lane >> 4;
    // wave index: uniform, so the schedule below stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_loader = wave >= kLrConsumers;
    const int c = is_loader ? wave - kLrConsumers : wave;   // the consumer this wave is / serves
    const int G = gridDim.x, GW = G * kLrConsumers;
    const int t0 = blockIdx.x + G * c;   // the consumer's first row tile (both phases)
    const int NT0 = t0 < T0 ? (T0 - t0 + GW - 1) / GW : 0;
    const int NT1 = t0 < T1 ? (T1 - t0 + GW - 1) / GW : 0;
    const int J0 = NT0 * I0, J1 = NT1 * I1;   // items per phase (a gate/up item is 2 units)
    const uint32_t rb0b = (uint32_t)C0 * 16u, rb1b = (uint32_t)C1 * 16u;
    const uint32_t rag0 = (C0 % kChunkLanes != 0 && cl >= C0 % kChunkLanes) ? kOutOfRange : 0u;
    const uint32_t rag1 = (C1 % kChunkLanes != 0 && cl >= C1 % kChunkLanes) ? kOutOfRange : 0u;

    // ---- LDS: step layout | block terms | control words | rings ------------------------
    const int act_bytes = max(I1 * L_::kStepBytes, I0 * L_::kStepBytes + M * H);
    uint8_t *act = lds;
    int8_t *qnat = reinterpret_cast<int8_t *>(lds + I0 * L_::kStepBytes);
    const int nbmax = max(nbh, nbi) + kBps;
    float *dq_s = reinterpret_cast<float *>(lds + act_bytes);
    int *qs_s = reinterpret_cast<int *>(dq_s + nbmax * M);
    int *ctl = qs_s + nbmax * M;
    uint8_t *myring = lds + lr_ring_offset(act_bytes, nbmax, M) + c * U * kUnitBytes;

    uint32_t *sync = a.sync;
    if (tid < kCtlWords)
        ctl[tid] = 0;
    __syncthreads();
    if (tid == 0 && sync_load(sync + kSyncError) != 0u)
        lds_st(ctl + kCtlAbort, 1);
    const uint32_t spin_word = sync_load(sync + kSyncSpin);
    const uint32_t spin_ticks = spin_word ? spin_word : kDefaultSpinTicks;
    __syncthreads();   // the last barrier of all 16 waves

    // ================================ loader waves ====================================
    if (is_loader) {
        // The walk over the consumer's units, layer by layer: gate/up pairs of phase 0
        // (tile k, step st, matrix g), then the down units of phase 1. Only wave-uniform
        // state changes from unit to unit: a unit's load address is a per-lane constant
        // (row within the tile, chunk lane, ragged-tail marker) plus a uniform offset,
        // passed as the buffer load's scalar offset, so a unit costs no vector arithmetic.
        if (lds_ld(ctl + kCtlAbort) != 0)
            return;
        // the layer table is read in place from the kernel argument segment (indexing the
        // by-value parameter at run time inside these loops makes the compiler copy it to
        // scratch memory)
        const FusedArgs *ka = (const FusedArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        const int nl = ka->L;
        const uint32_t gcb = ka->gu_codes_bytes, gsb = ka->gu_scales_bytes;
        const uint32_t dcb = ka->d_codes_bytes, dsb = ka->d_scales_bytes;
        const int total = nl * (2 * J0 + J1);
        const uint32_t nbh2 = (uint32_t)nbh * 2u, nbi2 = (uint32_t)nbi * 2u;
        // per-lane offsets of the two phases; rag* moves a ragged-tail lane out of range
        const uint32_t lc0 = (uint32_t)rl * rb0b + (uint32_t)cl * 16u;
        const uint32_t lc1 = (uint32_t)rl * rb1b + (uint32_t)cl * 16u;
        const uint32_t ls0 = (((uint32_t)rl * nbh2) + (uint32_t)(cl / kCpb) * 2u) & ~3u;
        const uint32_t ls1 = (((uint32_t)rl * nbi2) + (uint32_t)(cl / kCpb) * 2u) & ~3u;
        // walk state (uniform)
        int wl = 0, wp = 0, wk = 0, wst = 0, wg = 0;
        uint32_t ucode = 0, uscale = 0;   // uniform byte offsets of the current unit
        int wlc = 0;   // layer whose pointers the loads use (wl clamped into range)
        auto set_layer = [&]() __attribute__((always_inline)) { wlc = wl < nl ? wl : 0; };
        auto tile_base = [&]() __attribute__((always_inline)) {
            const uint32_t row0 = (uint32_t)((t0 + wk * GW) * kRowsPerWave);
            if (wp == 0) {
                ucode = row0 * rb0b;
                uscale = row0 * nbh2;
            } else {
                ucode = row0 * rb1b;
                uscale = row0 * nbi2;
            }
        };
        // move to the first unit of the current (layer, phase), skipping empty phases
        auto enter_phase = [&]() __attribute__((always_inline)) {
            for (int guard = 0; guard < 2 * kMaxFusedLayers + 2 && wl < nl; ++guard) {
                if ((wp == 0 ? J0 : J1) > 0)
                    break;
                if (wp == 0) {
                    wp = 1;
                } else {
                    wp = 0;
                    ++wl;
                    set_layer();
                }
            }
            wk = 0;
            wst = 0;
            wg = 0;
            tile_base();
        };
        auto advance = [&]() __attribute__((always_inline)) {
            if (wp == 0 && wg == 0) {
                wg = 1;
                return;
            }
            wg = 0;
            const int I = wp == 0 ? I0 : I1;
            if (++wst < I) {
                ucode += 16u * kChunkLanes;
                uscale += 2u * kBps;
                return;
            }
            wst = 0;
            if (++wk < (wp == 0 ? NT0 : NT1)) {
                tile_base();
                return;
            }
            if (wp == 0) {
                wp = 1;
            } else {
                wp = 0;
                ++wl;
                set_layer();
            }
            enter_phase();
        };
        auto issue = [&](int v, uint4 &w, uint32_t &sw) __attribute__((always_inline)) {
            const bool real = v < total;
            const int g = wp == 0 ? wg : 2;
            const bool last = wst == (wp == 0 ? I0 : I1) - 1;
            const uint32_t extra = last ? (wp == 0 ? rag0 : rag1) : 0u;
            const uint32_t vc = real ? (wp == 0 ? lc0 : lc1) + extra : kOutOfRange;
            const uint32_t vs = real ? (wp == 0 ? ls0 : ls1) + extra : kOutOfRange;
            const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(ka->layer[wlc].codes[g], g < 2 ? gcb : dcb);
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(ka->layer[wlc].scales[g], g < 2 ? gsb : dsb);
            const u32x4 c4 = __builtin_amdgcn_raw_buffer_load_b128(rc, vc, (int)ucode, kAuxNonTemporal);
            w = make_uint4(c4.x, c4.y, c4.z, c4.w);
            sw = __builtin_amdgcn_raw_buffer_load_b32(rs, vs, (int)uscale, 0);
            if (real)
                advance();
        };
        set_layer();
        enter_phase();

        uint4 rw[D];
        uint32_t rs[D];
#pragma unroll
        for (int d = 0; d < D; ++d)
            issue(d, rw[d], rs[d]);
        int consumed_seen = 0, slot = 0;
        bool stop = false;
        for (int v0 = 0; v0 < total && !stop; v0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int v = v0 + d;
                if (v < total && !stop) {
                    // the unit goes to slot v % U, free once the consumer has read unit v - U
                    if (consumed_seen + U <= v) {
                        // the ring is full: the consumer needs hundreds of cycles per
                        // unit, so poll slowly (a busy poll takes issue slots from it)
                        const uint64_t ts = __builtin_amdgcn_s_memrealtime();
                        for (int it = 1;; ++it) {
                            consumed_seen = __builtin_amdgcn_readfirstlane(lds_ld(ctl + kCtlConsumed + c));
                            if (consumed_seen + U > v)
                                break;
                            if ((it & 15) == 0) {
                                if (lds_ld(ctl + kCtlAbort) != 0) {
                                    stop = true;
                                    break;
                                }
                                if (__builtin_amdgcn_s_memrealtime() - ts > spin_ticks) {
                                    raise_error(sync, ctl);
                                    stop = true;
                                    break;
                                }
                            }
                            __builtin_amdgcn_s_sleep(6);
                        }
                    }
                    if (!stop) {
                        uint8_t *dst = myring + slot * kUnitBytes;
                        *reinterpret_cast<uint4 *>(dst + lane * 16) = rw[d];
                        *reinterpret_cast<uint32_t *>(dst + 1024 + lane * 4) = rs[d];
                        compiler_fence();
                        if (lane == 0)
                            lds_st(ctl + kCtlFilled + c, v + 1);
                        if (++slot == U)
                            slot = 0;
                    }
                }
                issue(v + D, rw[d], rs[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }

    // ================================ consumer waves ==================================
    bool alive = lds_ld(ctl + kCtlAbort) == 0;
    int gen = 0;            // consumer barriers passed
    int ucons = 0;          // units read from the ring
    int filled_seen = 0;    // last value read of the loader's counter
    int cslot = 0;          // ring slot of the next unit
    auto wait_units = [&](int need) -> bool {
        if (filled_seen >= need)
            return true;
        const uint64_t ts = __builtin_amdgcn_s_memrealtime();
        for (int it = 1;; ++it) {
            filled_seen = __builtin_amdgcn_readfirstlane(lds_ld(ctl + kCtlFilled + c));
            if (filled_seen >= need)
                return true;
            if ((it & 15) == 0) {
                if (lds_ld(ctl + kCtlAbort) != 0)
                    return false;
                if (__builtin_amdgcn_s_memrealtime() - ts > spin_ticks) {
                    raise_error(sync, ctl);
                    return false;
                }
            }
            __builtin_amdgcn_s_sleep(1);
        }
    };
    auto read_unit = [&](uint4 &w, uint32_t &s) {
        const uint8_t *src = myring + cslot * kUnitBytes;
        w = *reinterpret_cast<const uint4 *>(src + lane * 16);
        s = *reinterpret_cast<const uint32_t *>(src + 1024 + lane * 4);
        if (++cslot == U)
            cslot = 0;
    };
    auto release = [&]() {
        compiler_fence();
        if (lane == 0)
            lds_st(ctl + kCtlConsumed + c, ucons);
    };

    const __amdgpu_buffer_rsrc_t r_h = buffer_rsrc(a.h, (uint32_t)(M * N * 4));
    const __amdgpu_buffer_rsrc_t r_qh = buffer_rsrc(a.qh, (uint32_t)(M * N));
    const __amdgpu_buffer_rsrc_t r_dqh = buffer_rsrc(a.dqh, (uint32_t)(M * nbi * 4));
    const __amdgpu_buffer_rsrc_t r_qsh = buffer_rsrc(a.qsumh, (uint32_t)(M * nbi * 4));

    int inst = 0;   // grid barrier instances used so far
    for (int l = 0; l < a.L; ++l) {
        // ---- P0: wait for the previous layer, rotate + quantise x into LDS -------------
        if (l > 0)
            alive = lr_wait(sync, inst - 1, spin_ticks, ctl, gen) && alive;
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
        }
        cbar(sync, ctl, gen, spin_ticks);
        if (alive)
            stage_from_lds<M, FMT>(act, qnat, H);
        cbar(sync, ctl, gen, spin_ticks);
        alive = alive && lds_ld(ctl + kCtlAbort) == 0;

        // ---- P1: gate/up items from the ring, h rows to the workspace -------------------
        float acc0[M], acc1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            acc0[m] = 0.0f;
            acc1[m] = 0.0f;
        }
        if (alive) {
            // items are read from the ring (and, for small M, their activations from LDS)
            // one item ahead of the one being computed; A and B alternate so no registers
            // are copied between items
            int fstep = 0;                           // step of the next item to fetch
            int cstep = 0;
            uint32_t crow = (uint32_t)(t0 * kRowsPerWave + rl);
            const uint8_t *cact = act + cl * 16;
            int cblk = cl / kCpb;
            uint32_t cshift = ((crow * (uint32_t)nbh + (uint32_t)cblk) & 1u) * 16u;
            auto fetch = [&](LrItem<M, FMT> &it, bool want) -> bool {
                if (!want)
                    return true;
                if (!wait_units(ucons + 2))
                    return false;
                read_unit(it.w0, it.s0);
                read_unit(it.w1, it.s1);
                ucons += 2;
                release();
                if constexpr (kPrefetchAct<M, FMT>)
                    load_act<M, FMT>(act + cl * 16 + fstep * L_::kStepBytes, it.av);
                if (++fstep == I0)
                    fstep = 0;
                return true;
            };
            auto compute = [&](const LrItem<M, FMT> &it) {
                int is0[M], is1[M];
                if constexpr (kPrefetchAct<M, FMT>)
                    chunk_sums_act<M, FMT, true>(it.w0, it.w1, it.av, is0, is1);
                else
                    chunk_sums_step<M, FMT, true>(it.w0, it.w1, cact, is0, is1);
                const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(it.s0, cshift, 16));
                const float s1 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(it.s1, cshift, 16));
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
            };
            LrItem<M, FMT> A, B;
            bool ok = fetch(A, J0 > 0);
            for (int j = 0; ok && j < J0;) {
                if (!(ok = fetch(B, j + 1 < J0)))
                    break;
                compute(A);
                if (++j == J0)
                    break;
                if (!(ok = fetch(A, j + 1 < J0)))
                    break;
                compute(B);
                ++j;
            }
            alive = ok;
        }
        lr_arrive(sync, ctl, gen, spin_ticks);   // A
        ++inst;

        // ---- P2: rotate + quantise h, spread over all workgroups -------------------------
        alive = lr_wait(sync, inst - 1, spin_ticks, ctl, gen) && alive;
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
        lr_arrive(sync, ctl, gen, spin_ticks);   // B
        ++inst;

        // ---- P3: stage q_h, down items from the ring, y rows ---------------------------
        alive = lr_wait(sync, inst - 1, spin_ticks, ctl, gen) && alive;
        if (alive) {
            stage_from_global_coherent<M, FMT>(act, a.qh, N, (uint32_t)(M * N));
            for (int i = tid; i < nbmax * M; i += kFusedThreads) {
                const int b = i / M, m = i % M;
                const bool in = b < nbi;
                const uint32_t o = in ? (uint32_t)((m * nbi + b) * 4) : kOutOfRange;
                dq_s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_dqh, o, 0, kAuxCoherent));
                qs_s[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_qsh, o, 0, kAuxCoherent);
            }
        }
        cbar(sync, ctl, gen, spin_ticks);
        alive = alive && lds_ld(ctl + kCtlAbort) == 0;
        if (alive) {
            float *yl = a.y + (size_t)l * M * H;
            const __amdgpu_buffer_rsrc_t r_y = buffer_rsrc(yl, (uint32_t)(M * H * 4));
            int fstep = 0;
            int cstep = 0;
            uint32_t crow = (uint32_t)(t0 * kRowsPerWave + rl);
            const uint8_t *cact = act + cl * 16;
            int cblk = cl / kCpb;
            uint32_t cshift = ((crow * (uint32_t)nbi + (uint32_t)cblk) & 1u) * 16u;
            auto fetch = [&](LrItem<M, FMT> &it, bool want) -> bool {
                if (!want)
                    return true;
                if (!wait_units(ucons + 1))
                    return false;
                read_unit(it.w0, it.s0);
                ucons += 1;
                release();
                if constexpr (kPrefetchAct<M, FMT>)
                    load_act<M, FMT>(act + cl * 16 + fstep * L_::kStepBytes, it.av);
                if (++fstep == I1)
                    fstep = 0;
                return true;
            };
            auto compute = [&](const LrItem<M, FMT> &it) {
                int is0[M], is1[M];
                if constexpr (kPrefetchAct<M, FMT>)
                    chunk_sums_act<M, FMT, false>(it.w0, it.w0, it.av, is0, is1);
                else
                    chunk_sums_step<M, FMT, false>(it.w0, it.w0, cact, is0, is1);
                const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(it.s0, cshift, 16));
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
            };
            LrItem<M, FMT> A, B;
            bool ok = fetch(A, J1 > 0);
            for (int j = 0; ok && j < J1;) {
                if (!(ok = fetch(B, j + 1 < J1)))
                    break;
                compute(A);
                if (++j == J1)
                    break;
                if (!(ok = fetch(A, j + 1 < J1)))
                    break;
                compute(B);
                ++j;
            }
            alive = ok;
        }
        lr_arrive(sync, ctl, gen, spin_ticks);   // C (waited for at the start of the next layer)
        ++inst;
    }

    // ---- exit: the last workgroup out resets the counters for the next launch -----------
    drain_memory();
    cbar(sync, ctl, gen, spin_ticks);
    if (tid == 0) {
        const uint32_t old = sync_add(sync + kSyncExit, 1u);
        if (old == (uint32_t)G - 1u) {
            for (int k = 0; k < kBarCounters; ++k)
                sync_store(sync + kSyncBar + k * kSyncStride, 0u);
            sync_store(sync + kSyncExit, 0u);
        }
    }
}

}  // namespace tbk

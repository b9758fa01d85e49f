// tb_layers.h -- tb_ffn_layers: whole FFN layers in one persistent launch (gfx950).
//
// One FFN layer, after "perf(bonsai): decode and small packed batches read the FFN from a
// ternary copy through a dp4a GEMV" (sparkinfer PR #1154, Summary and commit message):
// rotate + quantise x (one int8 copy shared by gate and up), gate/up GEMVs and the SiLU
// gate, rotate + quantise h, down GEMV. Every row is folded exactly as by the separate
// entry points (same device blocks, same order: row tree per step, step partials summed
// in step order), so a layer's outputs are bit-identical to tb_rotate_quant_i8 +
// tb_ffn_gateup_silu + tb_ffn_down on the same inputs, for every M.
//
// Why one launch: a dependent kernel launch costs a ramp of 2-4 us before its weight
// stream reaches full rate, against about 10 us for the whole layer's 71 MB at the
// measured 7 TB/s. Here one workgroup per CU (16 waves; 12 or 8 for sign batches) stays resident for all layers:
//   * Work. Each CU owns an equal share of the gate/up row tiles and of the down row tiles
//     (4 rows each), the same shares every layer. An item is one step of a gate/up tile
//     (gate and up, 2 KB per wave) or two steps of a down tile (2 KB). The CU's items of
//     all layers form one stream; its waves take items from an LDS counter, so the
//     register ring of each wave (kDepth items) runs across phase and layer boundaries
//     and keeps loading while the CU waits for data from other CUs.
//   * Dependencies without barriers. Data that crosses CUs (h, rotquant(h), y) is stored
//     as 8-byte entries {value, tag}, tag = launch epoch * 32 + layer + 1, with 8-byte
//     device-coherent atomic stores. A consumer reads the entries device-coherently and
//     waits until every tag it needs is current; a producer never waits for its own
//     stores. (With one vmcnt counter for loads and stores, a producer that waited for its
//     stores before raising a flag would also wait for all of its weight prefetches.)
//   * Per layer: gate/up items; the CU sums its h rows (step partials in LDS) and stores
//     them tagged; it rotates and quantises its share of the h blocks as soon as their
//     rows are current and stores the codes tagged; it stages all of rotquant(h) once
//     current; down items; it stores its y rows (output, and tagged); the next layer
//     starts once every y row of this layer is current (strict layer order).
// Every wait is bounded by a spin limit on the 100 MHz real-time clock. A wait that runs
// out sets a sticky error word; the launch then runs to its end without waiting (outputs
// undefined), and later launches on the workspace do nothing until it is initialised.
#pragma once

#include "tb_device.h"

namespace tbl {

using namespace tbk;

// Waves per workgroup: 16 for ternary and for sign at one row; for sign, whose decode holds
// more registers, 12 for 2 to 5 rows and 8 from 6 (at 16 waves, 128 VGPRs each, its kernels
// spilled from 2 rows on, 328 bytes per lane at 8; at 12 waves, from 6 rows on). Sign
// layers, us per layer: M=8 96.7 -> 69.3; M=1 on 12 waves 25.0 against 23.6 on 16.
__host__ __device__ constexpr int layers_waves(int fmt, int m)
{
    return (fmt == TB_FMT_SIGN1 && m > 1) ? (m >= 6 ? 8 : 12) : 16;
}
__host__ __device__ constexpr int layers_threads(int fmt, int m) { return 64 * layers_waves(fmt, m); }
#ifndef TBL_DEPTH_TERN
#define TBL_DEPTH_TERN 2
#endif
constexpr int kDepthTern = TBL_DEPTH_TERN;   // ring items per wave (ternary; the sign decode
constexpr int kDepthSign = 2;                // needs more registers)
constexpr int kMaxLayers = 32;       // layers per launch (tags: epoch * 32 + layer + 1)
constexpr int kAuxSc1 = 16;          // device-coherent access
constexpr uint32_t kSpinDefault = 10000000u;   // 100 ms

// Workspace sync words (uint32), each on its own 256-byte line.
constexpr int kLine = 64;
constexpr int kWErr = 0, kWSpin = kLine, kWExit = 2 * kLine, kWEpoch = 3 * kLine;
constexpr int kMaxGrid = 1024;
// then two arrays of kMaxGrid tagged entries: a workgroup's rotquant(h) blocks stored,
// its y rows stored (hints that tell consumers when to read; the data's own tags decide)
constexpr int kWQDone = 4 * kLine, kWYDone = kWQDone + 2 * kMaxGrid;
constexpr int kSyncWords = kWYDone + 2 * kMaxGrid;
constexpr int kCtlBytes = 256;       // LDS control block

struct LLayer {
    const uint8_t *codes[3];   // gate, up, down
    const uint16_t *scales[3];
};

struct LArgs {
    LLayer layer[kMaxLayers];
    const float *x;   // [L][M][H], or [M][H] when chained
    float *y;         // [L][M][H]
    uint32_t *sync;
    uint64_t *hp;     // [M][N]    h, tagged
    uint64_t *qp;     // [M][N/4]  rotquant(h) codes, 4 per entry, tagged
    uint64_t *dp;     // [M][N/128] its scales, tagged
    uint64_t *sp;     // [M][N/128] its per-block code sums (sign format), tagged
    uint64_t *yp;     // [M][H]    y, tagged
    int L, H, N, chain;
    uint32_t gu_cb, gu_sb, d_cb, d_sb;   // bytes of codes / scales (scales rounded up to 4)
    float unit;
};

// LDS carve-up, shared with the host. The activation region holds the current phase's
// step-major activation; the step partials of a phase sit right after that phase's
// activation (gate/up partials inside the larger down activation region, which is free
// during gate/up), then the block terms.
struct LdsPlan {
    int act, part_gu, part_d, dq, qs, total;
};
__host__ __device__ inline LdsPlan lds_plan(int M, int fmt, int H, int N, int G)
{
    const int wpc = fmt == TB_FMT_TERNARY2 ? 64 : 128;
    const int sb = (fmt == TB_FMT_TERNARY2 ? 1024 : 2048) * M;
    const int I1 = (H / wpc + 15) / 16, I2 = (N / wpc + 15) / 16;
    const int T1 = N / 4, T2 = H / 4;
    const int nt1 = (T1 + G - 1) / G, nt2 = (T2 + G - 1) / G;
    const int bps = fmt == TB_FMT_TERNARY2 ? 8 : 16;
    const int nbmax = (H > N ? H : N) / 128;
    LdsPlan p;
    p.act = kCtlBytes;
    p.part_gu = p.act + I1 * sb;
    p.part_d = p.act + I2 * sb;
    const int end_gu = p.part_gu + nt1 * I1 * 4 * M * 2 * 4;
    const int end_d = p.part_d + nt2 * I2 * 4 * M * 4;
    p.dq = (end_gu > end_d ? end_gu : end_d);
    p.qs = p.dq + (nbmax + bps) * M * 4;
    p.total = p.qs + (fmt == TB_FMT_SIGN1 ? (nbmax + bps) * M * 4 : 0);
    return p;
}

__device__ __forceinline__ void st_tag(uint64_t *p, uint32_t v, uint32_t tag)
{
    __hip_atomic_store(p, (uint64_t)tag << 32 | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_sync(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sync(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two tagged entries (16 bytes, one load): .x value 0, .y tag 0, .z value 1, .w tag 1.
__device__ __forceinline__ u32x4 ld_tag2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxSc1);
}
// One tagged entry (8 bytes, one load): .x value, .y tag.
__device__ __forceinline__ u32x2 ld_tag1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxSc1);
}

// a / b for 0 <= a < 2^22, 0 < b, with rb = 1.0f / b: the float quotient is within one of
// the true one, and one correction step fixes it.
__device__ __forceinline__ int div_small(int a, int b, float rb)
{
    int q = (int)((float)a * rb);
    if (q * b > a)
        --q;
    else if ((q + 1) * b <= a)
        ++q;
    return q;
}

template <int M, int FMT>
__global__ __launch_bounds__(layers_threads(FMT, M), 1) void ffn_layers_kernel(LArgs a)
{
    constexpr int kWaves = layers_waves(FMT, M), kThreads = layers_threads(FMT, M);
    extern __shared__ __align__(16) uint8_t lds[];
    using SL = StepLayout<M, FMT>;
    constexpr int kWpc = Fmt<FMT>::kWeightsPerChunk;
    constexpr int kCpb = Fmt<FMT>::kChunksPerBlock;
    constexpr int kBps = kChunkLanes / kCpb;   // blocks per step
    constexpr int kGroups = kThreads / 16;
    constexpr int kDepth = FMT == TB_FMT_TERNARY2 ? kDepthTern : kDepthSign;

    const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15, rl = lane >> 4;
    const int l16 = tid & 15, grp = tid >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, c = blockIdx.x;
    const int H = a.H, N = a.N, L = a.L;
    const int nbH = H / kBlock, nbN = N / kBlock;
    const int C1 = H / kWpc, C2 = N / kWpc;                   // chunks per gate/up, down row
    const int I1 = (C1 + 15) / 16, I2 = (C2 + 15) / 16;       // steps per row
    const int P2 = (I2 + 1) / 2;                              // down items per tile
    const int T1 = N / kRowsPerWave, T2 = H / kRowsPerWave;
    const int tA1 = part_lo(T1, G, c), nt1 = part_lo(T1, G, c + 1) - tA1;
    const int tA2 = part_lo(T2, G, c), nt2 = part_lo(T2, G, c + 1) - tA2;
    const int J1 = nt1 * I1, J2 = nt2 * P2, JL = J1 + J2;
    const int total = L * JL;
    const float rJL = 1.0f / (float)(JL > 0 ? JL : 1), rI1 = 1.0f / (float)I1, rP2 = 1.0f / (float)P2;
    const uint32_t RB1 = (uint32_t)C1 * 16u, RB2 = (uint32_t)C2 * 16u;   // row bytes
    const LdsPlan plan = lds_plan(M, FMT, H, N, G);
    uint8_t *act = lds + plan.act;
    float *part_gu = reinterpret_cast<float *>(lds + plan.part_gu);
    float *part_d = reinterpret_cast<float *>(lds + plan.part_d);
    float *dq_s = reinterpret_cast<float *>(lds + plan.dq);
    int *qs_s = reinterpret_cast<int *>(lds + plan.qs);
    int *ctl = reinterpret_cast<int *>(lds);   // [0] item counter, [1] abort
    uint32_t *sync = a.sync;

    if (tid == 0) {
        ctl[0] = kWaves;   // wave w starts with item w
        ctl[1] = ld_sync(sync + kWErr) != 0u ? 1 : 0;
    }
    __syncthreads();
    const bool dead = ctl[1] != 0;   // the sticky error was set before this launch
    const uint32_t tag0 = ld_sync(sync + kWEpoch) * (uint32_t)kMaxLayers + 1u;   // tag of layer 0
    const uint32_t spin_w = ld_sync(sync + kWSpin);
    const uint64_t spin = spin_w ? spin_w : kSpinDefault;

    // ---- bounded waits ------------------------------------------------------------------
    // ok(t0): false once the launch is aborted, or when the spin limit has run out (which
    // aborts it). Other workgroups' errors are seen through the error word.
    auto aborted = [&]() -> bool {
        return __hip_atomic_load(ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
    };
    auto keep_waiting = [&](uint64_t t0, int it) -> bool {
        if (aborted())
            return false;
        if ((it & 15) == 15 && ld_sync(sync + kWErr) != 0u) {
            __hip_atomic_store(ctl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > spin) {
            st_sync(sync + kWErr, 1u);
            __hip_atomic_store(ctl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
        return true;
    };

    // Wave 0 waits until done entry w is current for every workgroup w (16-byte loads, two
    // entries each, all issued before any is checked); then every thread passes the barrier.
    auto wait_done = [&](int word, uint32_t tg, uint64_t t0) {
        if (tid < 64) {
            const __amdgpu_buffer_rsrc_t rdn = buffer_rsrc(sync + word, (uint32_t)(G * 8));
            for (int it = 0;; ++it) {
                bool ok = true;
                for (int i = lane; i < (G + 1) / 2; i += 64 * 4) {
                    u32x4 e[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[r] = ld_tag2(rdn, i + 64 * r < (G + 1) / 2 ? (uint32_t)(i + 64 * r) * 16u : kOutOfRange);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int w0 = 2 * (i + 64 * r);
                        if (w0 < G)
                            ok = ok && e[r].y == tg;
                        if (w0 + 1 < G)
                            ok = ok && e[r].w == tg;
                    }
                }
                if (__all(ok) || !keep_waiting(t0, it))
                    break;
            }
        }
        __syncthreads();
    };
    auto mark_done = [&](int word, uint32_t tg) {
        __syncthreads();   // every thread of the workgroup has issued its data stores
        if (tid == 0)
            st_tag(reinterpret_cast<uint64_t *>(sync + word) + c, 0u, tg);
    };

    // ---- phase transitions (all threads) ------------------------------------------------
    // Stage rotquant of layer l's input into the activation region. For l > 0 this waits
    // until every y row of layer l - 1 is current (strict layer order); chained, those
    // rows are the input.
    auto stage_x = [&](int l) {
        const bool from_y = l > 0 && a.chain;
        const uint32_t tprev = tag0 + (uint32_t)l - 1u;
        const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(a.yp, (uint32_t)(M * H * 8));
        const float *xl = a.chain ? a.x : a.x + (size_t)l * M * H;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        // input blocks: the first round is loaded before the order check below
        constexpr int kXR = 1;
        float xv[kXR][8];
        if (!from_y) {
#pragma unroll
            for (int r = 0; r < kXR; ++r) {
                const int z = grp + r * kGroups;
                if (z < M * nbH) {
                    const float *src = xl + (size_t)(z / nbH) * H + (z % nbH) * kBlock + l16 * 8;
                    const float4 lo = *reinterpret_cast<const float4 *>(src);
                    const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
                    xv[r][0] = lo.x; xv[r][1] = lo.y; xv[r][2] = lo.z; xv[r][3] = lo.w;
                    xv[r][4] = hi.x; xv[r][5] = hi.y; xv[r][6] = hi.z; xv[r][7] = hi.w;
                }
            }
        }
        // strict layer order: every workgroup has stored its y rows of layer l - 1
        if (l > 0)
            wait_done(kWYDone, tprev, t0);
        auto block = [&](float (&v)[8], int z) {
            const int m = z / nbH, b = z % nbH;
            uint32_t pk[2];
            float dq;
            int qsum;
            rotquant_regs(v, l16, a.unit, pk, dq, qsum);
            store_block_step<M, FMT>(act, m, b, l16, pk);
            if (l16 == 0) {
                dq_s[b * M + m] = dq;
                if (FMT == TB_FMT_SIGN1)
                    qs_s[b * M + m] = qsum;
            }
        };
        if (from_y) {
            for (int z = grp; z < M * nbH; z += kGroups) {
                const int m = z / nbH, b = z % nbH;
                const uint32_t off = (uint32_t)((m * H + b * kBlock + l16 * 8) * 8);
                u32x4 e[4];
                for (int it = 0;; ++it) {
                    bool ok = true;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        e[q] = ld_tag2(ry, off + 16u * q);
                        ok = ok && e[q].y == tprev && e[q].w == tprev;
                    }
                    if (ok || !keep_waiting(t0, it))
                        break;
                }
                float v[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[2 * q] = __uint_as_float(e[q].x);
                    v[2 * q + 1] = __uint_as_float(e[q].z);
                }
                block(v, z);
            }
        } else {
#pragma unroll
            for (int r = 0; r < kXR; ++r)
                if (grp + r * kGroups < M * nbH)
                    block(xv[r], grp + r * kGroups);
            for (int z = grp + kXR * kGroups; z < M * nbH; z += kGroups) {
                const float *src = xl + (size_t)(z / nbH) * H + (z % nbH) * kBlock + l16 * 8;
                const float4 lo = *reinterpret_cast<const float4 *>(src);
                const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
                float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                block(v, z);
            }
        }
        for (int i = nbH * M + tid; i < (nbH + kBps) * M; i += kThreads) {
            dq_s[i] = 0.0f;
            if (FMT == TB_FMT_SIGN1)
                qs_s[i] = 0;
        }
    };

    // Gate/up of layer l done: store this CU's h rows, rotate + quantise its share of the
    // h blocks, stage all of rotquant(h).
    auto gateup_to_down = [&](int l) {
        const uint32_t tg = tag0 + (uint32_t)l;
        for (int i = tid; i < nt1 * kRowsPerWave * M; i += kThreads) {
            const int tl = i / (kRowsPerWave * M), r = (i / M) % kRowsPerWave, m = i % M;
            const float *ps = part_gu + ((size_t)(tl * I1 * kRowsPerWave + r) * M + m) * 2;
            float g = 0.0f, u = 0.0f;
            for (int s = 0; s < I1; ++s) {
                g += ps[(size_t)s * kRowsPerWave * M * 2];
                u += ps[(size_t)s * kRowsPerWave * M * 2 + 1];
            }
            const int row = (tA1 + tl) * kRowsPerWave + r;
            st_tag(a.hp + (size_t)m * N + row, __float_as_uint(silu_gate(g, u)), tg);
        }
        // this CU's h blocks
        const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(a.hp, (uint32_t)(M * N * 8));
        const int zA = part_lo(M * nbN, G, c), zB = part_lo(M * nbN, G, c + 1);
        uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (int z = zA + grp; z < zB; z += kGroups) {
            const int m = z / nbN, b = z % nbN;
            const uint32_t off = (uint32_t)((m * N + b * kBlock + l16 * 8) * 8);
            u32x4 e[4];
            for (int it = 0;; ++it) {
                bool ok = true;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    e[q] = ld_tag2(rh, off + 16u * q);
                    ok = ok && e[q].y == tg && e[q].w == tg;
                }
                if (ok || !keep_waiting(t0, it))
                    break;
            }
            float v[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] = __uint_as_float(e[q].x);
                v[2 * q + 1] = __uint_as_float(e[q].z);
            }
            uint32_t pk[2];
            float dq;
            int qsum;
            rotquant_regs(v, l16, a.unit, pk, dq, qsum);
            uint64_t *qd = a.qp + (size_t)(m * N + b * kBlock + l16 * 8) / 4;
            st_tag(qd, pk[0], tg);
            st_tag(qd + 1, pk[1], tg);
            if (l16 == 0) {
                st_tag(a.dp + m * nbN + b, __float_as_uint(dq), tg);
                if (FMT == TB_FMT_SIGN1)
                    st_tag(a.sp + m * nbN + b, (uint32_t)qsum, tg);
            }
        }
        mark_done(kWQDone, tg);
        wait_done(kWQDone, tg, __builtin_amdgcn_s_memrealtime());
        // stage all of rotquant(h): units of 16 codes (ternary) or 32 (sign), kR units per
        // thread and round, the block terms in the first round; every load of a round is
        // issued before any tag is checked
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.qp, (uint32_t)(M * N * 2));
        const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(a.dp, (uint32_t)(M * nbN * 8));
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.sp, (uint32_t)(M * nbN * 8));
        constexpr int kE = FMT == TB_FMT_TERNARY2 ? 2 : 4;   // 16-byte loads per unit
        constexpr int kR = 1;
        const int per_row = C2 * 4, units = M * per_row, nterm = (nbN + kBps) * M;
        t0 = __builtin_amdgcn_s_memrealtime();
        for (int u0 = tid; u0 - tid < units || u0 == tid; u0 += kR * kThreads) {
            const bool first = u0 == tid;
            u32x4 e[kR][kE];
            u32x2 dv[2], sv[2];
            for (int it = 0;; ++it) {
                bool ok = true;
#pragma unroll
                for (int r = 0; r < kR; ++r) {
                    const int u = u0 + r * kThreads;
                    int m, g2;
                    unit_split<M>(u, per_row, m, g2);
                    const uint32_t off = u < units ? (uint32_t)((m * N + (g2 >> 2) * kWpc + (g2 & 3) * (kWpc / 4)) * 2)
                                                   : kOutOfRange;
#pragma unroll
                    for (int q = 0; q < kE; ++q)
                        e[r][q] = ld_tag2(rq, off + 16u * q);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int i = tid + t * kThreads, b = i / M, m = i % M;
                    const uint32_t off = (first && i < nterm && b < nbN) ? (uint32_t)((m * nbN + b) * 8) : kOutOfRange;
                    dv[t] = ld_tag1(rd, off);
                    sv[t] = FMT == TB_FMT_SIGN1 ? ld_tag1(rs, off) : u32x2{0u, 0u};
                    if (off != kOutOfRange)
                        ok = ok && dv[t].y == tg && (FMT != TB_FMT_SIGN1 || sv[t].y == tg);
                }
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    if (u0 + r * kThreads < units)
#pragma unroll
                        for (int q = 0; q < kE; ++q)
                            ok = ok && e[r][q].y == tg && e[r][q].w == tg;
                if (ok || !keep_waiting(t0, it))
                    break;
            }
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const int u = u0 + r * kThreads;
                if (u >= units)
                    continue;
                StageUnit<FMT> su;
                su.lo = make_uint4(e[r][0].x, e[r][0].z, e[r][1].x, e[r][1].z);
                if (FMT == TB_FMT_SIGN1)
                    su.hi = make_uint4(e[r][kE - 2].x, e[r][kE - 2].z, e[r][kE - 1].x, e[r][kE - 1].z);
                int m, g2;
                unit_split<M>(u, per_row, m, g2);
                stage_unit_store_step<M, FMT>(su, act, m, g2);
            }
            if (first) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int i = tid + t * kThreads, b = i / M;
                    if (i < nterm) {
                        dq_s[i] = b < nbN ? __uint_as_float(dv[t].x) : 0.0f;
                        if (FMT == TB_FMT_SIGN1)
                            qs_s[i] = b < nbN ? (int)sv[t].x : 0;
                    }
                }
            }
        }
        // block terms past the first round (intermediate sizes above 32768)
        for (int i = tid + 2 * kThreads; i < nterm; i += kThreads) {
            const int b = i / M, m = i % M;
            u32x2 d = u32x2{0u, tg}, e = u32x2{0u, tg};
            for (int it = 0; b < nbN; ++it) {
                d = ld_tag1(rd, (uint32_t)((m * nbN + b) * 8));
                if (FMT == TB_FMT_SIGN1)
                    e = ld_tag1(rs, (uint32_t)((m * nbN + b) * 8));
                if ((d.y == tg && e.y == tg) || !keep_waiting(t0, it))
                    break;
            }
            dq_s[i] = b < nbN ? __uint_as_float(d.x) : 0.0f;
            if (FMT == TB_FMT_SIGN1)
                qs_s[i] = b < nbN ? (int)e.x : 0;
        }
    };

    // Down of layer l done: this CU's y rows, to the output and tagged (the next layer's
    // start condition, and its input when chained).
    auto down_end = [&](int l) {
        const uint32_t tg = tag0 + (uint32_t)l;
        float *yl = a.y + (size_t)l * M * H;
        for (int i = tid; i < nt2 * kRowsPerWave * M; i += kThreads) {
            const int tl = i / (kRowsPerWave * M), r = (i / M) % kRowsPerWave, m = i % M;
            const float *ps = part_d + (size_t)(tl * I2 * kRowsPerWave + r) * M + m;
            float yv = 0.0f;
            for (int s = 0; s < I2; ++s)
                yv += ps[(size_t)s * kRowsPerWave * M];
            const int row = (tA2 + tl) * kRowsPerWave + r;
            yl[(size_t)m * H + row] = yv;
            st_tag(a.yp + (size_t)m * H + row, __float_as_uint(yv), tg);
        }
        mark_done(kWYDone, tg);
    };

    // ---- the item stream ---------------------------------------------------------------
    // Slot tag: layer << 24 | phase << 23 | tile << 10 | step (gate/up) or step pair (down);
    // the phase index of a slot is tag >> 23 = 2 * layer + (down ? 1 : 0). -1: empty.
    const uint32_t ragged1 = (C1 % 16 != 0 && cl >= C1 % 16) ? kOutOfRange : 0u;
    const uint32_t ragged2 = (C2 % 16 != 0 && cl >= C2 % 16) ? kOutOfRange : 0u;
    int pending = wave;   // the next item, taken one issue ahead
    uint4 rb0[kDepth], rb1[kDepth];
    uint32_t rs0[kDepth], rs1[kDepth];
    int rit[kDepth];
    auto issue = [&](uint4 &w0, uint4 &w1, uint32_t &s0, uint32_t &s1, int &it) {
        const int idx = __builtin_amdgcn_readfirstlane(pending);
        uint32_t o0 = kOutOfRange, o1 = kOutOfRange, so0 = kOutOfRange, so1 = kOutOfRange;
        const uint8_t *p0 = a.layer[0].codes[0], *p1 = p0;
        const uint16_t *q0 = a.layer[0].scales[0], *q1 = q0;
        uint32_t cb = a.gu_cb, sb = a.gu_sb;
        it = -1;
        if (idx < total) {
            const int l = div_small(idx, JL, rJL);
            const int r = idx - l * JL;
            if (r < J1) {
                const int tile = div_small(r, I1, rI1), step = r - tile * I1;
                it = l << 24 | tile << 10 | step;
                const uint32_t row = (uint32_t)((tA1 + tile) * kRowsPerWave + rl);
                const uint32_t ex = step == I1 - 1 ? ragged1 : 0u;
                o0 = (row * RB1 + (uint32_t)cl * 16u + (uint32_t)step * 256u) | ex;
                o1 = o0;
                so0 = (((row * (uint32_t)nbH + (uint32_t)(step * kBps + cl / kCpb)) * 2u) & ~3u) | ex;
                so1 = so0;
                p0 = a.layer[l].codes[0];
                p1 = a.layer[l].codes[1];
                q0 = a.layer[l].scales[0];
                q1 = a.layer[l].scales[1];
            } else {
                const int r2 = r - J1;
                const int tile = div_small(r2, P2, rP2), pr = r2 - tile * P2;
                it = l << 24 | 1 << 23 | tile << 10 | pr;
                const uint32_t row = (uint32_t)((tA2 + tile) * kRowsPerWave + rl);
                const int st0 = 2 * pr, st1 = 2 * pr + 1;
                const uint32_t e0 = st0 == I2 - 1 ? ragged2 : 0u, e1 = st1 == I2 - 1 ? ragged2 : 0u;
                const uint32_t base = row * RB2 + (uint32_t)cl * 16u;
                const uint32_t sbase = row * (uint32_t)nbN + (uint32_t)(cl / kCpb);
                o0 = (base + (uint32_t)st0 * 256u) | e0;
                so0 = (((sbase + (uint32_t)(st0 * kBps)) * 2u) & ~3u) | e0;
                if (st1 < I2) {
                    o1 = (base + (uint32_t)st1 * 256u) | e1;
                    so1 = (((sbase + (uint32_t)(st1 * kBps)) * 2u) & ~3u) | e1;
                }
                p0 = p1 = a.layer[l].codes[2];
                q0 = q1 = a.layer[l].scales[2];
                cb = a.d_cb;
                sb = a.d_sb;
            }
            int v = 0;
            if (lane == 0)
                v = atomicAdd(ctl, 1);
            pending = v;
        }
        w0 = buffer_load16_nt(buffer_rsrc(p0, cb), o0);
        w1 = buffer_load16_nt(buffer_rsrc(p1, cb), o1);
        s0 = buffer_load_u32(buffer_rsrc(q0, sb), so0);
        s1 = buffer_load_u32(buffer_rsrc(q1, sb), so1);
    };

    const uint8_t *lds_lane = act + cl * 16;
    const int blk_lane = cl / kCpb;
    // one step of one row tile: the lanes' terms, the row tree, the step partial to LDS
    auto step_terms = [&](const uint4 &w0, const uint4 &w1, uint32_t sw0, uint32_t sw1, int step,
                          uint32_t row, int nb, float *dst, bool two) {
        int is0[M], is1[M];
        if (two)
            chunk_sums_step<M, FMT, true, false>(w0, w1, lds_lane + (size_t)step * SL::kStepBytes, is0, is1);
        else
            chunk_sums_step<M, FMT, false, false>(w0, w0, lds_lane + (size_t)step * SL::kStepBytes, is0, is1);
        const int blk = step * kBps + blk_lane;
        const uint32_t cshift = ((row * (uint32_t)nb + (uint32_t)blk_lane) & 1u) * 16u;
        const float s0 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(sw0, cshift, 16));
        const float s1 = half_bits_to_float((uint16_t)__builtin_amdgcn_ubfe(sw1, cshift, 16));
        float p0[M], p1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            int v0 = is0[m], v1 = is1[m];
            if (FMT == TB_FMT_SIGN1) {
                v0 = 2 * v0 - qs_s[blk * M + m];
                v1 = 2 * v1 - qs_s[blk * M + m];
            }
            const float dqv = dq_s[blk * M + m];
            p0[m] = (s0 * dqv) * (float)v0;
            p1[m] = two ? (s1 * dqv) * (float)v1 : 0.0f;
        }
        if (two)
            row_tree<M, FMT, true>(p0, p1);
        else
            row_tree<M, FMT, false>(p0, p1);
        if (cl == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (two) {
                    dst[2 * m] = p0[m];
                    dst[2 * m + 1] = p1[m];
                } else {
                    dst[m] = p0[m];
                }
            }
        }
    };
    auto consume = [&](const uint4 &w0, const uint4 &w1, uint32_t sw0, uint32_t sw1, int it) {
        const int tile = (it >> 10) & 0x1fff, st = it & 0x3ff;
        if (((it >> 23) & 1) == 0) {
            const uint32_t row = (uint32_t)((tA1 + tile) * kRowsPerWave + rl);
            step_terms(w0, w1, sw0, sw1, st, row, nbH,
                       part_gu + ((size_t)(tile * I1 + st) * kRowsPerWave + rl) * M * 2, true);
        } else {
            const uint32_t row = (uint32_t)((tA2 + tile) * kRowsPerWave + rl);
            const int s0 = 2 * st;
            step_terms(w0, w0, sw0, sw0, s0, row, nbN,
                       part_d + ((size_t)(tile * I2 + s0) * kRowsPerWave + rl) * M, false);
            if (s0 + 1 < I2)
                step_terms(w1, w1, sw1, sw1, s0 + 1, row, nbN,
                           part_d + ((size_t)(tile * I2 + s0 + 1) * kRowsPerWave + rl) * M, false);
        }
    };

    // ---- run ------------------------------------------------------------------------------
    if (!dead) {
        stage_x(0);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(rb0[d], rb1[d], rs0[d], rs1[d], rit[d]);
        __syncthreads();
        int cur = 0;   // the phase whose activation is staged
        for (;;) {
            int brk = -1;
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                if (brk < 0) {
                    const int it = rit[d];
                    const int ph = it < 0 ? 0x7fffffff : (it >> 23);
                    if (ph > cur) {
                        brk = d;
                    } else {
                        consume(rb0[d], rb1[d], rs0[d], rs1[d], it);
                        issue(rb0[d], rb1[d], rs0[d], rs1[d], rit[d]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (brk < 0)
                continue;
            // every wave's next item is of a later phase: this CU's items of phase cur are done
            __syncthreads();
            const int l = cur >> 1;
            if ((cur & 1) == 0) {
                gateup_to_down(l);
            } else {
                down_end(l);
                if (l + 1 < L)
                    stage_x(l + 1);
            }
            __syncthreads();
            if (++cur == 2 * L)
                break;
            // rotate the ring so that slot 0 holds the next item
            switch (brk) {
#define TBL_ROT(K)                                                                               \
    case K: {                                                                                    \
        uint4 t0[kDepth], t1[kDepth];                                                            \
        uint32_t u0[kDepth], u1[kDepth];                                                         \
        int ti[kDepth];                                                                          \
        _Pragma("unroll") for (int d = 0; d < kDepth; ++d) {                                     \
            t0[d] = rb0[(d + K) % kDepth];                                                       \
            t1[d] = rb1[(d + K) % kDepth];                                                       \
            u0[d] = rs0[(d + K) % kDepth];                                                       \
            u1[d] = rs1[(d + K) % kDepth];                                                       \
            ti[d] = rit[(d + K) % kDepth];                                                       \
        }                                                                                        \
        _Pragma("unroll") for (int d = 0; d < kDepth; ++d) {                                     \
            rb0[d] = t0[d];                                                                      \
            rb1[d] = t1[d];                                                                      \
            rs0[d] = u0[d];                                                                      \
            rs1[d] = u1[d];                                                                      \
            rit[d] = ti[d];                                                                      \
        }                                                                                        \
        break;                                                                                   \
    }
                TBL_ROT(1) TBL_ROT(2)
#undef TBL_ROT
            default:
                break;
            }
        }
    }

    // ---- exit: the last workgroup out advances the epoch --------------------------------
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(sync + kWExit, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1u == (uint32_t)G) {
            st_sync(sync + kWExit, 0u);
            st_sync(sync + kWEpoch, ld_sync(sync + kWEpoch) + 1u);
        }
    }
}

// Initialise a workspace: every word zero (no tag is current: tags start at 1), the spin
// limit word set.
__global__ void layers_ws_init_kernel(uint32_t *ws, size_t words, uint32_t spin_ticks)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        ws[i] = i == (size_t)kWSpin ? spin_ticks : 0u;
}

}  // namespace tbl

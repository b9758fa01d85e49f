// tb_device.h -- device building blocks of the ternary-weight int8 FFN kernels (gfx950).
//
// Included by tb.hip only. Every block here is shared by all entry points, so that
// one weight row is computed the same way whichever kernel runs it. The fold order of a
// row is fixed by its shape alone: in step i lane cl holds chunk 16 i + cl; the step's
// partial is the fixed 16-lane row tree of the lanes' terms (scale * dq) * isum; the row's
// output is the sum of its step partials in step order, starting from +0. Neither the
// row count M, nor the kernel, nor which wave ran which step changes it. That is what
// makes a batched row bit-identical to the same row run alone, the property the pages
// claim for their batched kernel ("perf(bonsai): decode and small packed batches read the
// FFN from a ternary copy through a dp4a GEMV", sparkinfer PR #1154, commit message).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "tb.h"

// sign weights at one row: bit planes masked in place (1), or shifted to bit 0 (0)
#ifndef TB_SIGN_MASK
#define TB_SIGN_MASK 1
#endif

namespace tbk {

constexpr int kBlock = 128;
constexpr int kChunkLanes = 16;   // lanes that share one weight row
constexpr int kRowsPerWave = 4;   // 64 lanes / 16

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int FMT>
struct Fmt;
template <>
struct Fmt<TB_FMT_TERNARY2> {
    static constexpr int kWeightsPerChunk = 64;   // 16 bytes of 2-bit codes, half a block
    static constexpr int kChunksPerBlock = 2;
};
template <>
struct Fmt<TB_FMT_SIGN1> {
    static constexpr int kWeightsPerChunk = 128;  // 16 bytes of sign bits, one block
    static constexpr int kChunksPerBlock = 1;
};

// First index of part i when n items are split into p near-equal contiguous parts.
__device__ __forceinline__ int part_lo(int n, int p, int i) { return (int)(((long long)n * i) / p); }
// The part that holds item t (0 <= t < n): the largest i with part_lo(n, p, i) <= t.
__device__ __forceinline__ int part_of(int n, int p, int t)
{
    return (int)((((long long)t + 1) * p - 1) / n);
}

__device__ __forceinline__ uint32_t byte_at(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Weights are read exactly once per call: stream them past the caches.
__device__ __forceinline__ uint4 load_nt(const uint8_t *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer descriptors (gfx9 layout: stride 0, num_records in bytes, 32-bit data format).
// A load whose offset is past num_records returns zeros and touches no memory: the
// streaming loops use that instead of branches, so every slot issues the same loads and
// the compiler can keep many of them in flight.
constexpr uint32_t kBufWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;   // callers keep num_records below this
constexpr int kAuxNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             (int)kBufWord3);
}

// soffset: a wave-uniform byte offset added to off. Only off is range-checked, so a lane
// that must read zeros sets off to kOutOfRange; every other lane's off + soffset must lie
// inside the buffer.
__device__ __forceinline__ uint4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                  int soffset = 0)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soffset, kAuxNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The same without the non-temporal hint: for reads whose cache line is read again by a
// neighbouring load (the matrix-core kernel reads each 128-byte line in two halves).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, int soffset)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soffset, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint16_t buffer_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// The 4-byte word holding the 2-byte value at byte offset off (off & ~3). A 32-bit ring
// entry needs no zero-extension, which the compiler would otherwise place at the loop
// latch, where it waits for every outstanding load.
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   int soffset = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soffset, 0);
}

// soffset: a wave-uniform byte offset added to off (not part of the range check).
__device__ __forceinline__ void buffer_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v,
                                                 int soffset = 0)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, soffset, 0);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float silu_gate(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// Swap-adjacent-lanes add: lanes 2i and 2i+1 both get their sum (exact integers).
__device__ __forceinline__ int pair_add(int v)
{
    return v + __builtin_amdgcn_update_dpp(0, v, 0xB1 /* quad_perm [1,0,3,2] */, 0xF, 0xF, false);
}

// The value of lane L ^ s of the lane's 16-lane DPP row (s = 1, 2, 4 or 8, a constant
// once loops are unrolled), moved by DPP instead of an LDS permute. Every lane of the row
// must be active.
__device__ __forceinline__ int row_xor(int v, int s)
{
    switch (s) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1 /* quad_perm [1,0,3,2] */, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E /* quad_perm [2,3,0,1] */, 0xF, 0xF, false);
    case 4: {
        // L ^ 7 (row_half_mirror), then ^ 3 (quad_perm [3,2,1,0])
        const int t = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
        return __builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false);
    }
    default: return __builtin_amdgcn_update_dpp(0, v, 0x128 /* row_ror:8 */, 0xF, 0xF, false);
    }
}
__device__ __forceinline__ float row_xor(float v, int s) { return __int_as_float(row_xor(__float_as_int(v), s)); }
__device__ __forceinline__ uint32_t row_xor(uint32_t v, int s) { return (uint32_t)row_xor((int)v, s); }

// The value of lane t (0..3, a constant once unrolled) of the lane's quad.
__device__ __forceinline__ uint32_t quad_lane(uint32_t v, int t)
{
    switch (t) {
    case 0: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xFF, 0xF, 0xF, false);
    }
}

// Ternary decode of one 32-bit code word (16 weights) into four int8x4 words; word j
// holds weights {j, j+4, j+8, j+12}. Selector bytes 0..3 index the table 0x00FF0100 ->
// {0, +1, -1, 0}. For the field masked in place at bits 2..3 the selector is 4c:
// 0 -> byte 0 of S1 (0), 4 -> byte 0 of S0 (+1), 8 -> sign of bit 15 of S1 (0xFF = -1),
// 12 -> 0. Nine VALU operations, shared by all rows of the batch.
__device__ __forceinline__ void decode_ternary(uint32_t w, uint32_t &d0, uint32_t &d1,
                                               uint32_t &d2, uint32_t &d3)
{
    const uint32_t w4 = w >> 4;
    d0 = __builtin_amdgcn_perm(0u, 0x00FF0100u, w & 0x03030303u);
    d1 = __builtin_amdgcn_perm(1u, 0x00008000u, w & 0x0C0C0C0Cu);
    d2 = __builtin_amdgcn_perm(0u, 0x00FF0100u, w4 & 0x03030303u);
    d3 = __builtin_amdgcn_perm(1u, 0x00008000u, w4 & 0x0C0C0C0Cu);
}

// ------------------------------------------------------------------------------------
// Rotate + quantise one 128-block with a 16-lane group. Lane L holds elements
// 8L .. 8L+7. Butterfly spans 1, 2, 4 are inside the lane; spans 8, 16, 32, 64 pair lane L
// with L ^ 1, 2, 4, 8. Ascending order, each (a, b) -> (a + b, a - b) in fp32. Then
// amax = max |u|; if amax != 0, q = rint(u * (127 / amax)) (IEEE division, ties to
// even) and dq = amax * unit; else q = 0 and dq = 0. Writes 8 q bytes per lane, and dq
// from lane 0 of the group.
// ------------------------------------------------------------------------------------
// Register core of the rotate-quantise step, for a 16-lane group holding one block:
// v[8] = elements 8L .. 8L+7 of the block in lane L. Returns the lane's 8 codes packed
// little-endian in packed[2], the block's dq, and the block's sum of codes (group total,
// for the sign format's isum = 2 * dot - sum(q)).
__device__ __forceinline__ void rotquant_regs(float (&v)[8], int lane16, float unit,
                                              uint32_t (&packed)[2], float &dq, int &qsum)
{
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
            const float other = row_xor(v[e], s);
            v[e] = upper ? (other - v[e]) : (v[e] + other);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
    for (int s = 1; s < 16; s <<= 1)
        amax = fmaxf(amax, row_xor(amax, s));

    packed[0] = 0u;
    packed[1] = 0u;
    int sum = 0;
    if (amax != 0.0f) {
        const float inv = 127.0f / amax;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float r = rintf(v[e] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const int qi = (int)r;
            sum += qi;
            packed[e >> 2] |= (uint32_t)(uint8_t)(int8_t)qi << (8 * (e & 3));
        }
    }
#pragma unroll
    for (int s = 1; s < 16; s <<= 1)
        sum += row_xor(sum, s);
    dq = amax != 0.0f ? amax * unit : 0.0f;
    qsum = sum;
}

// Rotate + quantise one 128-block with a 16-lane group (see rotquant_regs), from global
// memory to global memory.
template <bool kCoherentIO>
__device__ __forceinline__ void rotquant16(const float *src, int8_t *qdst, float *dqdst,
                                           int lane16, float unit)
{
    float v[8];
    if (kCoherentIO) {
        // data written by other workgroups of the same launch: read it device-coherently
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = __hip_atomic_load(src + lane16 * 8 + e, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const float4 lo = *reinterpret_cast<const float4 *>(src + lane16 * 8);
        const float4 hi = *reinterpret_cast<const float4 *>(src + lane16 * 8 + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
    uint32_t packed[2];
    float dq;
    int qsum;
    rotquant_regs(v, lane16, unit, packed, dq, qsum);
    uint32_t *qw = reinterpret_cast<uint32_t *>(qdst + lane16 * 8);
    if (kCoherentIO) {
        __hip_atomic_store(qw, packed[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(qw + 1, packed[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane16 == 0)
            __hip_atomic_store(dqdst, dq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *reinterpret_cast<uint2 *>(qw) = make_uint2(packed[0], packed[1]);
        if (lane16 == 0)
            *dqdst = dq;
    }
}

// ------------------------------------------------------------------------------------
// Activation staging. q[M][k] (global) -> LDS, chunks [c0, c0 + sc) into slots [0, sc).
// Ternary: per row m, S slots of 64 activations laid out [code word j][slot] as 16-byte
//   groups, each group the 4x4 byte transpose of 16 consecutive activations, to match
//   decode_ternary's word order.
// Sign: per row m, S slots of 128 activations laid out [dword d][half h][slot]; word j of
//   (d, h) holds activations {32d + 4h + j + 8p : p = 0..3}, to match (w >> j) & 0x01010101.
// Lanes of a row read consecutive slots, so ds_read_b128 sees no bank conflicts.
// COHERENT: q was written by other workgroups of the same launch.
// ------------------------------------------------------------------------------------
template <bool COHERENT>
__device__ __forceinline__ uint4 load16(const int8_t *p)
{
    if (COHERENT) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(p);
        uint4 r;
        r.x = __hip_atomic_load(w + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        r.y = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        r.z = __hip_atomic_load(w + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        r.w = __hip_atomic_load(w + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return r;
    }
    return *reinterpret_cast<const uint4 *>(p);
}

// One staging unit: 16 activations (ternary: one code word's worth) or 32 (sign: one
// dword of sign bits). stage_unit_load reads it, stage_unit_store writes it transposed.
template <int FMT>
struct StageUnit {
    uint4 lo, hi;
};

// A staging unit is (row m, chunk c, part j): 4 parts per chunk (16 activations ternary,
// 32 sign), numbered unit = m * per_row + 4 c + j with per_row = 4 * chunks per row.
// unit_split returns m and g = 4 c + j without an integer division (m < M <= 8 rows):
// a runtime division costs tens of VALU instructions, and staging runs it for every unit.
template <int M>
__device__ __forceinline__ void unit_split(int unit, int per_row, int &m, int &g)
{
    m = 0;
#pragma unroll
    for (int i = 1; i < M; ++i)
        m += unit >= i * per_row ? 1 : 0;
    g = unit - m * per_row;
}

template <int FMT, bool COHERENT>
__device__ __forceinline__ void stage_unit_load(StageUnit<FMT> &u, const int8_t *q, int k, int c0,
                                                int m, int g)
{
    const int c = g >> 2, j = g & 3;
    if (FMT == TB_FMT_TERNARY2) {
        u.lo = load16<COHERENT>(q + (size_t)m * k + (size_t)(c0 + c) * 64 + j * 16);
    } else {
        const int8_t *src = q + (size_t)m * k + (size_t)(c0 + c) * 128 + j * 32;
        u.lo = load16<COHERENT>(src);
        u.hi = load16<COHERENT>(src + 16);
    }
}

template <int FMT>
__device__ __forceinline__ void stage_unit_store(const StageUnit<FMT> &u, uint8_t *act, int S,
                                                 int m, int g)
{
    const int c = g >> 2, j = g & 3;
    if (FMT == TB_FMT_TERNARY2) {
        const uint4 r = u.lo;
        uint4 o;
        o.x = byte_at(r.x, 0) | byte_at(r.y, 0) << 8 | byte_at(r.z, 0) << 16 | byte_at(r.w, 0) << 24;
        o.y = byte_at(r.x, 1) | byte_at(r.y, 1) << 8 | byte_at(r.z, 1) << 16 | byte_at(r.w, 1) << 24;
        o.z = byte_at(r.x, 2) | byte_at(r.y, 2) << 8 | byte_at(r.z, 2) << 16 | byte_at(r.w, 2) << 24;
        o.w = byte_at(r.x, 3) | byte_at(r.y, 3) << 8 | byte_at(r.z, 3) << 16 | byte_at(r.w, 3) << 24;
        *reinterpret_cast<uint4 *>(act + (size_t)m * S * 64 + ((size_t)j * S + c) * 16) = o;
    } else {
        const uint32_t r[8] = {u.lo.x, u.lo.y, u.lo.z, u.lo.w, u.hi.x, u.hi.y, u.hi.z, u.hi.w};
        // word i holds (q[i], q[8+i], q[16+i], q[24+i]); q[8p+i] is byte i&3 of r[2p+i/4]
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = byte_at(r[0 + (i >> 2)], i & 3) | byte_at(r[2 + (i >> 2)], i & 3) << 8 |
                   byte_at(r[4 + (i >> 2)], i & 3) << 16 | byte_at(r[6 + (i >> 2)], i & 3) << 24;
        uint8_t *dst = act + (size_t)m * S * 128;
        *reinterpret_cast<uint4 *>(dst + ((size_t)(j * 2 + 0) * S + c) * 16) =
            make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(dst + ((size_t)(j * 2 + 1) * S + c) * 16) =
            make_uint4(o[4], o[5], o[6], o[7]);
    }
}

template <int M, int FMT, bool COHERENT>
__device__ __forceinline__ void stage_act(uint8_t *act, int S, const int8_t *q, int k, int c0,
                                          int sc, int tid, int nthreads)
{
    const int units = M * sc * 4;
    for (int u = tid; u < units; u += nthreads) {
        StageUnit<FMT> su;
        int m, g;
        unit_split<M>(u, sc * 4, m, g);
        stage_unit_load<FMT, COHERENT>(su, q, k, c0, m, g);
        stage_unit_store<FMT>(su, act, S, m, g);
    }
}

// ------------------------------------------------------------------------------------
// Step-major activation layout, used by the streaming kernels. Chunk c of row m sits in
// step c / 16, lane slot c % 16. All 16 chunks of a step, for all M rows, are one
// contiguous block of kStepBytes:
//   ternary: [code word j][row m][slot] x 16 bytes   (kStepBytes = 1024 * M)
//   sign:    [dword d][half h][row m][slot] x 16 bytes (kStepBytes = 2048 * M)
// A lane's reads within one step are therefore at compile-time offsets from a single
// base address (lane slot * 16 + step * kStepBytes), and the 16 lanes of a row read 256
// consecutive bytes: no bank conflicts.
// ------------------------------------------------------------------------------------
template <int M, int FMT>
struct StepLayout {
    static constexpr int kPlanes = FMT == TB_FMT_TERNARY2 ? 4 : 8;   // 16-byte groups per chunk
    static constexpr int kStepBytes = kPlanes * M * 256;
    __device__ static constexpr int offset(int plane, int m) { return (plane * M + m) * 256; }
};

template <int M, int FMT, bool COHERENT>
__device__ __forceinline__ void stage_unit_load_step(StageUnit<FMT> &u, const int8_t *q, int k,
                                                     int m, int g)
{
    const int c = g >> 2, j = g & 3;
    if (FMT == TB_FMT_TERNARY2) {
        u.lo = load16<COHERENT>(q + (size_t)m * k + (size_t)c * 64 + j * 16);
    } else {
        const int8_t *src = q + (size_t)m * k + (size_t)c * 128 + j * 32;
        u.lo = load16<COHERENT>(src);
        u.hi = load16<COHERENT>(src + 16);
    }
}

template <int M, int FMT>
__device__ __forceinline__ void stage_unit_store_step(const StageUnit<FMT> &u, uint8_t *act, int m,
                                                      int g)
{
    using L = StepLayout<M, FMT>;
    const int c = g >> 2, j = g & 3;
    uint8_t *base = act + (size_t)(c >> 4) * L::kStepBytes + (c & 15) * 16;
    if (FMT == TB_FMT_TERNARY2) {
        const uint4 r = u.lo;
        uint4 o;
        o.x = byte_at(r.x, 0) | byte_at(r.y, 0) << 8 | byte_at(r.z, 0) << 16 | byte_at(r.w, 0) << 24;
        o.y = byte_at(r.x, 1) | byte_at(r.y, 1) << 8 | byte_at(r.z, 1) << 16 | byte_at(r.w, 1) << 24;
        o.z = byte_at(r.x, 2) | byte_at(r.y, 2) << 8 | byte_at(r.z, 2) << 16 | byte_at(r.w, 2) << 24;
        o.w = byte_at(r.x, 3) | byte_at(r.y, 3) << 8 | byte_at(r.z, 3) << 16 | byte_at(r.w, 3) << 24;
        *reinterpret_cast<uint4 *>(base + L::offset(j, m)) = o;
    } else {
        const uint32_t r[8] = {u.lo.x, u.lo.y, u.lo.z, u.lo.w, u.hi.x, u.hi.y, u.hi.z, u.hi.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = byte_at(r[0 + (i >> 2)], i & 3) | byte_at(r[2 + (i >> 2)], i & 3) << 8 |
                   byte_at(r[4 + (i >> 2)], i & 3) << 16 | byte_at(r[6 + (i >> 2)], i & 3) << 24;
        *reinterpret_cast<uint4 *>(base + L::offset(j * 2 + 0, m)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(base + L::offset(j * 2 + 1, m)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

// The same 16-byte groups in the layout of the matrix-core kernel, staged in slot order:
// unit (g, m) with g = 4 c + j (chunk c, part j) goes to slot g * M + m (ternary: one
// 16-byte group), or to slots (2 g + h) * M + m, h = 0, 1 (sign: its two groups). Per step
// that is [chunk][code word][row m] (ternary) or [chunk][dword][half][row m] (sign), so
// the 16 lanes of an MFMA B operand, which hold the M rows of one group, read consecutive
// 16-byte slots (no bank conflicts).
template <int M, int FMT>
__device__ __forceinline__ void stage_unit_store_mfma(const StageUnit<FMT> &u, uint8_t *act, int m,
                                                      int g)
{
    if (FMT == TB_FMT_TERNARY2) {
        const uint4 r = u.lo;
        uint4 o;
        o.x = byte_at(r.x, 0) | byte_at(r.y, 0) << 8 | byte_at(r.z, 0) << 16 | byte_at(r.w, 0) << 24;
        o.y = byte_at(r.x, 1) | byte_at(r.y, 1) << 8 | byte_at(r.z, 1) << 16 | byte_at(r.w, 1) << 24;
        o.z = byte_at(r.x, 2) | byte_at(r.y, 2) << 8 | byte_at(r.z, 2) << 16 | byte_at(r.w, 2) << 24;
        o.w = byte_at(r.x, 3) | byte_at(r.y, 3) << 8 | byte_at(r.z, 3) << 16 | byte_at(r.w, 3) << 24;
        *reinterpret_cast<uint4 *>(act + ((size_t)g * M + m) * 16) = o;
    } else {
        const uint32_t r[8] = {u.lo.x, u.lo.y, u.lo.z, u.lo.w, u.hi.x, u.hi.y, u.hi.z, u.hi.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = byte_at(r[0 + (i >> 2)], i & 3) | byte_at(r[2 + (i >> 2)], i & 3) << 8 |
                   byte_at(r[4 + (i >> 2)], i & 3) << 16 | byte_at(r[6 + (i >> 2)], i & 3) << 24;
        *reinterpret_cast<uint4 *>(act + ((size_t)(2 * g) * M + m) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(act + ((size_t)(2 * g + 1) * M + m) * 16) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

// One rotated-quantised block into the step-major layout. The 16-lane group holds block b
// of row m; lane L has codes 8L .. 8L+7 packed little-endian in pk[0], pk[1] (the
// registers rotquant_regs returns). Lanes exchange codes so that each writes 8 bytes of
// the layout that stage_unit_store_step writes from global memory.
template <int M, int FMT>
__device__ __forceinline__ void store_block_step(uint8_t *act, int m, int b, int lane16,
                                                 const uint32_t (&pk)[2])
{
    using L = StepLayout<M, FMT>;
    uint32_t o[2];
    int c, plane, half;
    if (FMT == TB_FMT_TERNARY2) {
        // 16-code group g = lane16 / 2 is code word g % 4 of chunk 2b + g / 4; its even lane
        // has codes 0..7, the odd lane 8..15. Word e of the group is codes {e, e+4, e+8,
        // e+12}; the even lane writes words 0, 1, the odd lane words 2, 3.
        const uint32_t q0 = row_xor(pk[0], 1), q1 = row_xor(pk[1], 1);
        const bool odd = lane16 & 1;
        const uint32_t lo0 = odd ? q0 : pk[0], lo1 = odd ? q1 : pk[1];
        const uint32_t hi0 = odd ? pk[0] : q0, hi1 = odd ? pk[1] : q1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int e = (odd ? 2 : 0) + t;
            o[t] = byte_at(lo0, e) | byte_at(lo1, e) << 8 | byte_at(hi0, e) << 16 | byte_at(hi1, e) << 24;
        }
        const int g = lane16 >> 1;
        c = 2 * b + (g >> 2);
        plane = g & 3;
        half = lane16 & 1;
    } else {
        // 32-code unit u = lane16 / 4: lane i = lane16 % 4 of it has codes 8i .. 8i+7. Word w
        // (0..7) of the unit is codes {w, w+8, w+16, w+24}: words 0..3 go to plane 2u,
        // words 4..7 to plane 2u + 1. Lane i writes words 2i, 2i + 1.
        const int i = lane16 & 3;
        uint32_t src[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t w0 = quad_lane(pk[0], t), w1 = quad_lane(pk[1], t);
            src[t] = (i >> 1) ? w1 : w0;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int e = (2 * i + t) & 3;
            o[t] = byte_at(src[0], e) | byte_at(src[1], e) << 8 | byte_at(src[2], e) << 16 |
                   byte_at(src[3], e) << 24;
        }
        c = b;
        plane = 2 * (lane16 >> 2) + (i >> 1);
        half = i & 1;
    }
    *reinterpret_cast<uint2 *>(act + (size_t)(c >> 4) * L::kStepBytes + (c & 15) * 16 +
                               L::offset(plane, m) + half * 8) = make_uint2(o[0], o[1]);
}

// One rotated-quantised block into the matrix-core layout of one step (the slots that
// stage_unit_store_mfma writes from global memory): block b of the step, row m; the
// 16-lane group holds the block as rotquant_regs returns it (lane L: codes 8L .. 8L+7).
// The lanes exchange codes exactly as in store_block_step; only the slot differs.
template <int M, int FMT>
__device__ __forceinline__ void store_block_mfma(uint8_t *act, int m, int b, int lane16,
                                                 const uint32_t (&pk)[2])
{
    uint32_t o[2];
    size_t slot;
    int half;
    if (FMT == TB_FMT_TERNARY2) {
        // unit u = lane16 / 2 of the block is unit g = 8 b + u of the step (chunk 2b + u / 4,
        // part u % 4); its even lane writes words 0, 1 of the slot, the odd lane 2, 3
        const uint32_t q0 = row_xor(pk[0], 1), q1 = row_xor(pk[1], 1);
        const bool odd = lane16 & 1;
        const uint32_t lo0 = odd ? q0 : pk[0], lo1 = odd ? q1 : pk[1];
        const uint32_t hi0 = odd ? pk[0] : q0, hi1 = odd ? pk[1] : q1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int e = (odd ? 2 : 0) + t;
            o[t] = byte_at(lo0, e) | byte_at(lo1, e) << 8 | byte_at(hi0, e) << 16 | byte_at(hi1, e) << 24;
        }
        slot = (size_t)(8 * b + (lane16 >> 1)) * M + m;
        half = lane16 & 1;
    } else {
        // unit u = lane16 / 4 is unit g = 4 b + u; lane i = lane16 % 4 writes words 2i, 2i+1
        // of the unit's eight: slot 2g (words 0..3) or 2g + 1 (words 4..7)
        const int i = lane16 & 3;
        uint32_t src[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t w0 = quad_lane(pk[0], t), w1 = quad_lane(pk[1], t);
            src[t] = (i >> 1) ? w1 : w0;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int e = (2 * i + t) & 3;
            o[t] = byte_at(src[0], e) | byte_at(src[1], e) << 8 | byte_at(src[2], e) << 16 |
                   byte_at(src[3], e) << 24;
        }
        slot = (size_t)(2 * (4 * b + (lane16 >> 2)) + (i >> 1)) * M + m;
        half = i & 1;
    }
    *reinterpret_cast<uint2 *>(act + slot * 16 + half * 8) = make_uint2(o[0], o[1]);
}

// Integer sums of one chunk against all M rows, step-major layout; `lds` is this lane's
// slot address in the current step. Same arithmetic as chunk_sums. MASK: sign weights at
// one row take the masked bit planes below (more registers: the fused kernel, which holds
// a whole ring across phases, spilled 76 bytes per lane with them).
template <int M, int FMT, bool TWO, bool MASK = true>
__device__ __forceinline__ void chunk_sums_step(const uint4 &w0, const uint4 &w1, const uint8_t *lds,
                                                int (&is0)[M], int (&is1)[M])
{
    using L = StepLayout<M, FMT>;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        is0[m] = 0;
        is1[m] = 0;
    }
    const uint32_t cw0[4] = {w0.x, w0.y, w0.z, w0.w};
    const uint32_t cw1[4] = {w1.x, w1.y, w1.z, w1.w};
    if (FMT == TB_FMT_TERNARY2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t d0, d1, d2, d3, e0 = 0, e1 = 0, e2 = 0, e3 = 0;
            decode_ternary(cw0[j], d0, d1, d2, d3);
            if (TWO)
                decode_ternary(cw1[j], e0, e1, e2, e3);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 av = *reinterpret_cast<const uint4 *>(lds + L::offset(j, m));
                is0[m] = dot4(d0, av.x, is0[m]);
                is0[m] = dot4(d1, av.y, is0[m]);
                is0[m] = dot4(d2, av.z, is0[m]);
                is0[m] = dot4(d3, av.w, is0[m]);
                if (TWO) {
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
            if (TWO)
                is1[m] = pair_add(is1[m]);
        }
    } else if (TB_SIGN_MASK && MASK && M == 1) {
        // Bit k of every byte masked in place: the bytes are 0 or 2^k (k = 7: 0x80, i.e.
        // -128 as a signed byte), so the dot product of plane bit k is 2^k D_k (k = 7:
        // -128 D_7) with D_k the exact sum over that bit's weights. One AND per dot product
        // instead of a shift and an AND; the eight scaled sums are joined exactly at the end:
        // 128 sum_k D_k = sum_{k<7} acc_k 2^(7 - k) - acc_7 (at most 8 * 128 * 16 * 127 in
        // magnitude), a multiple of 128, then an arithmetic shift by 7. Measured at M = 1
        // (32 sign layers, us per call): gate/up 10.80 -> 10.65, down 9.63 -> 9.47; at M = 2
        // the sixteen accumulators per row made it slower (13.18 -> 13.30, 10.78 -> 11.10).
        int a0[8][M], a1[8][M];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                a0[kk][m] = 0;
                a1[kk][m] = 0;
            }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int d = p >> 1, h = p & 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kk = 4 * h + j;
                const uint32_t mask = 0x01010101u << kk;
                const uint32_t c0 = cw0[d] & mask, c1 = TWO ? (cw1[d] & mask) : 0u;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint4 av = *reinterpret_cast<const uint4 *>(lds + L::offset(p, m));
                    const uint32_t aj = j == 0 ? av.x : j == 1 ? av.y : j == 2 ? av.z : av.w;
                    a0[kk][m] = dot4(c0, aj, a0[kk][m]);
                    if (TWO)
                        a1[kk][m] = dot4(c1, aj, a1[kk][m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            int t0 = -a0[7][m], t1 = -a1[7][m];
#pragma unroll
            for (int kk = 0; kk < 7; ++kk) {
                t0 += a0[kk][m] * (1 << (7 - kk));
                if (TWO)
                    t1 += a1[kk][m] * (1 << (7 - kk));
            }
            is0[m] = t0 >> 7;
            if (TWO)
                is1[m] = t1 >> 7;
        }
    } else {
        // Planes are taken one at a time with the next plane's reads in flight: left free,
        // the scheduler hoists the reads of all 8 planes (32 M registers), which spills
        // from M = 5 on.
        uint4 nxt[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            nxt[m] = *reinterpret_cast<const uint4 *>(lds + L::offset(0, m));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int d = p >> 1, h = p & 1;
            uint4 cur[M];
#pragma unroll
            for (int m = 0; m < M; ++m)
                cur[m] = nxt[m];
            if (p < 7) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    nxt[m] = *reinterpret_cast<const uint4 *>(lds + L::offset(p + 1, m));
            }
            uint32_t b0[4], b1[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b0[j] = (cw0[d] >> (4 * h + j)) & 0x01010101u;
                if (TWO)
                    b1[j] = (cw1[d] >> (4 * h + j)) & 0x01010101u;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 av = cur[m];
                is0[m] = dot4(b0[0], av.x, is0[m]);
                is0[m] = dot4(b0[1], av.y, is0[m]);
                is0[m] = dot4(b0[2], av.z, is0[m]);
                is0[m] = dot4(b0[3], av.w, is0[m]);
                if (TWO) {
                    is1[m] = dot4(b1[0], av.x, is1[m]);
                    is1[m] = dot4(b1[1], av.y, is1[m]);
                    is1[m] = dot4(b1[2], av.z, is1[m]);
                    is1[m] = dot4(b1[3], av.w, is1[m]);
                }
            }
            if (M >= 4) {
                // Pin this plane's dot products before the barrier: they are pure
                // operations, which the IR passes may otherwise sink below every plane (as
                // they did in the block-sum export, keeping all 8 planes' reads live).
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    asm volatile("" : "+v"(is0[m]));
                    if (TWO)
                        asm volatile("" : "+v"(is1[m]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// dq[M][nb] -> LDS; for the sign format also sum(q) per block -> LDS (int).
template <int M, int FMT, bool COHERENT>
__device__ __forceinline__ void stage_block_terms(float *dq_s, int *qsum_s, const float *dq,
                                                  const int8_t *q, int nb, bool need_dq, int tid,
                                                  int nthreads)
{
    if (need_dq)
        for (int i = tid; i < M * nb; i += nthreads)
            dq_s[i] = COHERENT ? __hip_atomic_load(dq + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : dq[i];
    if (FMT == TB_FMT_SIGN1) {
        for (int i = tid; i < M * nb; i += nthreads) {
            const int8_t *src = q + (size_t)i * kBlock;   // [m][b] blocks are contiguous
            int s = 0;
            for (int j = 0; j < kBlock; j += 16) {
                const uint4 g = load16<COHERENT>(src + j);
                s = dot4(g.x, 0x01010101u, s);
                s = dot4(g.y, 0x01010101u, s);
                s = dot4(g.z, 0x01010101u, s);
                s = dot4(g.w, 0x01010101u, s);
            }
            qsum_s[i] = s;
        }
    }
}

// ------------------------------------------------------------------------------------
// Integer sums of one 16-byte chunk against all M staged rows. TWO: a second matrix
// (up) shares the activation reads. Ternary: each lane holds half a block, and the
// partner's half is added with one DPP op, so both lanes hold the block sum. Sign: the
// dot of the 0/1 bits; the caller applies isum = 2 * dot - sum(q).
// slot: the chunk's LDS slot (any valid slot when the lane has no chunk; its codes are 0).
// ------------------------------------------------------------------------------------
template <int M, int FMT, bool TWO>
__device__ __forceinline__ void chunk_sums(const uint4 &w0, const uint4 &w1, const uint8_t *act,
                                           int S, int slot, int (&is0)[M], int (&is1)[M])
{
#pragma unroll
    for (int m = 0; m < M; ++m) {
        is0[m] = 0;
        is1[m] = 0;
    }
    const uint32_t cw0[4] = {w0.x, w0.y, w0.z, w0.w};
    const uint32_t cw1[4] = {w1.x, w1.y, w1.z, w1.w};
    if (FMT == TB_FMT_TERNARY2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t d0, d1, d2, d3, e0 = 0, e1 = 0, e2 = 0, e3 = 0;
            decode_ternary(cw0[j], d0, d1, d2, d3);
            if (TWO)
                decode_ternary(cw1[j], e0, e1, e2, e3);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 av =
                    *reinterpret_cast<const uint4 *>(act + (size_t)m * S * 64 + ((size_t)j * S + slot) * 16);
                is0[m] = dot4(d0, av.x, is0[m]);
                is0[m] = dot4(d1, av.y, is0[m]);
                is0[m] = dot4(d2, av.z, is0[m]);
                is0[m] = dot4(d3, av.w, is0[m]);
                if (TWO) {
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
            if (TWO)
                is1[m] = pair_add(is1[m]);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t b0[4], b1[4] = {0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    b0[j] = (cw0[d] >> (4 * h + j)) & 0x01010101u;
                    if (TWO)
                        b1[j] = (cw1[d] >> (4 * h + j)) & 0x01010101u;
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint4 av = *reinterpret_cast<const uint4 *>(
                        act + (size_t)m * S * 128 + ((size_t)(d * 2 + h) * S + slot) * 16);
                    is0[m] = dot4(b0[0], av.x, is0[m]);
                    is0[m] = dot4(b0[1], av.y, is0[m]);
                    is0[m] = dot4(b0[2], av.z, is0[m]);
                    is0[m] = dot4(b0[3], av.w, is0[m]);
                    if (TWO) {
                        is1[m] = dot4(b1[0], av.x, is1[m]);
                        is1[m] = dot4(b1[1], av.y, is1[m]);
                        is1[m] = dot4(b1[2], av.z, is1[m]);
                        is1[m] = dot4(b1[3], av.w, is1[m]);
                    }
                }
            }
        }
    }
}

// Lane (i + off) mod 16 of the same 16-lane row (DPP row rotate). Lane 0 of a row, the
// only lane whose tree result is used, reads lane off; a rotate has no out-of-row lanes,
// so the compiler folds it into the add (v_add_f32_dpp) at every level.
__device__ __forceinline__ float row_down(float v, int off)
{
    int r;
    switch (off) {
    case 1: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false); break;
    }
    return __int_as_float(r);
}

// Fixed tree over the 16 lanes of a row; lane 0 of the row ends with the total. Each
// level adds the value of lane L - off (row_ror reads the lane off places below, mod 16),
// so for ternary (odd lanes hold copies) lane 0 gets
// ((a0 + a14) + (a12 + a10)) + ((a8 + a6) + (a4 + a2)), and for sign the same pattern
// over all 16 lanes with offsets 1, 2, 4, 8. DPP row rotates: no LDS traffic.
template <int M, int FMT, bool TWO>
__device__ __forceinline__ void row_tree(float (&acc0)[M], float (&acc1)[M])
{
#pragma unroll
    for (int off = FMT == TB_FMT_TERNARY2 ? 2 : 1; off < kChunkLanes; off <<= 1) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            acc0[m] += row_down(acc0[m], off);
            if (TWO)
                acc1[m] += row_down(acc1[m], off);
        }
    }
    // Keep the last level here: callers use the totals in lane 0 only, and an add sunk
    // into that branch could no longer take its DPP operand directly.
#pragma unroll
    for (int m = 0; m < M; ++m) {
        asm volatile("" : "+v"(acc0[m]));
        if (TWO)
            asm volatile("" : "+v"(acc1[m]));
    }
}

}  // namespace tbk

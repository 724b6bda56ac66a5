// moe_device.h -- device helpers shared by the libmoe kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Storage types: bfloat16 travels as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bfloat16, round to nearest, ties to even: gfx950's
// v_cvt_pk_bf16_f32 (one instruction for two values; a NaN stays a NaN).
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(moe_f32x2{lo, hi}, moe_bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Weighted routed rows y of bfloat16 layers, in 16-bit block floating point.
// A row of d values is stored as d signed 16-bit mantissas followed by d/8
// exponent bytes, padded to a multiple of 16 bytes (y16_pitch(d)).  Group g,
// elements 8g..8g+7, shares exponent byte X: element i is m_i * 2^(X - 141).
// X is the biased binary32 exponent of the group's largest magnitude M (at
// least 1; 0 when the group is all zeros), so M * 2^(141 - X) lies in
// [2^14, 2^15) and every m_i = round-to-nearest-even(v_i * 2^(141 - X))
// (+2^15 clamped to 2^15 - 1) is off by at most 2^-15 M.  Against bfloat16
// (an error of up to 2^-9 of each element) this keeps the rows as good as
// binary32 for the layer's output tolerance, at about 2.1 bytes per element
// instead of 4.
__host__ __device__ constexpr int64_t y16_pitch(int d) {
    return (2 * (int64_t)d + d / 8 + 15) / 16 * 16;
}

__device__ __forceinline__ uint32_t y16_exponent(float amax) {
    const uint32_t f = (__float_as_uint(amax) >> 23) & 0xFFu;
    return amax == 0.0f ? 0u : (f > 1u ? f : 1u);
}
__device__ __forceinline__ int32_t y16_q(float v, uint32_t x) {
    return (int32_t)fminf(__builtin_rintf(ldexpf(v, 141 - (int)x)), 32767.0f);
}
// Two elements as one packed pair of 16-bit mantissas (element a low).
__device__ __forceinline__ uint32_t y16_pack2(float a, float b, uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(y16_q(a, x), y16_q(b, x)));
}
__device__ __forceinline__ float y16_value(uint32_t m16, uint32_t x) {
    return ldexpf((float)(int32_t)(int16_t)(uint16_t)m16, (int)x - 141);
}
__device__ __forceinline__ float absmax4(float a, float b, float c, float e) {
    return fmaxf(fmaxf(fabsf(a), fabsf(b)), fmaxf(fabsf(c), fabsf(e)));
}
// One element per lane, a group's eight elements in eight consecutive lanes
// (8q .. 8q+7, consecutive columns): the group's exponent byte.  Every lane
// of the wave must execute it.
__device__ __forceinline__ uint32_t y16_octet_exponent(float v) {
    float a = fabsf(v);
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    a = fmaxf(a, __shfl_xor(a, 4, 64));
    return y16_exponent(a);
}
// The element at col of row from its lane, with its octet's exponent x (the
// lane holding the group's first column writes the exponent byte).
__device__ __forceinline__ void y16_store1(uint8_t *row, int d, int col, float v, uint32_t x) {
    *reinterpret_cast<uint16_t *>(row + 2 * (int64_t)col) =
        (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_i16(y16_q(v, x), 0)) & 0xFFFFu);
    if ((col & 7) == 0) row[2 * (int64_t)d + col / 8] = (uint8_t)x;
}

// Eight consecutive elements widened to binary32 (exact).
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    uint4 q = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Eight MXFP4 E2M1 codes (one dword, element 2j in the low nibble of byte j)
// times 2^(X-127), exactly, as bf16 in element order.
// v_cvt_scalef32_pk_bf16_fp4 reads only the exponent field of its binary32
// scale operand, so scale byte X is passed as the bits X << 23.
__device__ __forceinline__ bf16x8 mx4_decode8(uint32_t w, float scale) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ float mx4_scale(uint32_t x) { return __uint_as_float(x << 23); }

__device__ __forceinline__ float to_f32(uint16_t b) { return bf16_to_f32(b); }
__device__ __forceinline__ float to_f32(float f) { return f; }

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Block -> (m, n) tile for a GEMM grid of nm x nn tiles launched as a 1-D
// grid of 8 * ceil(nm * nn / 8) blocks (gm >= 0) or 8 * ceil(nm / 8) * nn
// blocks (gm < 0).  Workgroups are dispatched to the 8
// XCDs round robin, so block b runs on XCD b % 8; logical tile ids are made
// contiguous per XCD, and within an XCD consecutive ids sweep gm M-tiles
// before advancing N, so the blocks that run together on one XCD share both
// their A rows and their B columns through that XCD's L2.  gm == 0 instead
// takes the plain order with N fastest.  Returns false for padding blocks.
__device__ __forceinline__ bool raster_tile(int nm, int nn, int gm, int &m, int &n) {
    const int nblocks = nm * nn;
    const int b = blockIdx.x;
    if (gm < 0) {
        // M-tile m runs on XCD m % 8 and its N-tiles are 8 block ids apart:
        // they share the tile's A rows through one L2, while consecutive
        // M-tiles still alternate over the XCDs (grid of 8 * ceil(nm / 8) * nn)
        const int x = b & 7, q = b >> 3;
        n = q % nn;
        m = 8 * (q / nn) + x;
        return m < nm;
    }
    if (gm == 0) {
        if (b >= nblocks) return false;
        m = b / nn;
        n = b - m * nn;
        return true;
    }
    const int per = (nblocks + 7) / 8;
    const int L = (b & 7) * per + (b >> 3);
    if (L >= nblocks) return false;
    const int span = gm * nn;
    const int group = L / span, idx = L - group * span;
    const int rows = min(gm, nm - group * gm);  // M-tiles in this (possibly short) group
    m = group * gm + idx % rows;
    n = idx / rows;
    return true;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

}  // namespace moe

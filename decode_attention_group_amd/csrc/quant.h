// Affine group quantization of one 64-value group, shared by the append kernel
// and the fused decode step so that both write the same codes bit for bit
// (page 78 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, gemma4-e4b.ts
// Gemma4Layer.kv: widths 4 and 8, group 64; the pages give no formula, this
// library's is):
//   bias  = min(group) rounded down to bf16 (-0 read as +0)
//   scale = ((max(group) - bias) / (2^bits - 1)) rounded up to bf16
//   code  = clamp(rint((x - bias) / scale), 0, 2^bits - 1)   (0 when scale == 0)
// each step a single IEEE fp32 operation (no contraction).
#pragma once

#include "kvq_device.h"

namespace kvq {

// Largest bf16 value <= x (x finite): clearing the low 16 bits moves toward
// zero, which is downward only for x >= 0; a negative x steps one bf16 unit
// further from zero instead.
__device__ __forceinline__ float bf16_round_down(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0xFFFFu) == 0u) return x;
    const uint32_t t = u & 0xFFFF0000u;
    return __uint_as_float((u & 0x80000000u) ? t + 0x10000u : t);
}

// Smallest bf16 value >= x (x finite, here always >= 0).
__device__ __forceinline__ float bf16_round_up(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0xFFFFu) == 0u) return x;
    const uint32_t t = u & 0xFFFF0000u;
    return __uint_as_float((u & 0x80000000u) ? t : t + 0x10000u);
}

// Codes of this lane's 8 values.  Eight consecutive lanes hold one group and
// must all be active; the group's min and max meet through three butterfly
// shuffles.  top = 2^bits - 1.
__device__ __forceinline__ void quantize_group8(const float (&v)[8], int top, uint32_t (&q)[8],
                                                float& scale, float& bias)
{
#pragma clang fp contract(off)
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    mn = mn + 0.0f;                       // -0 reads as +0
    mx = mx + 0.0f;
    bias = bf16_round_down(mn);
    const float step = (mx - bias) / (float)top;
    scale = bf16_round_up(step);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float r = 0.0f;
        if (scale != 0.0f) {
            r = __builtin_rintf((v[e] - bias) / scale);
            r = fminf(fmaxf(r, 0.0f), (float)top);
        }
        q[e] = (uint32_t)r;
    }
}

// Scale|bias word of a group: bf16 scale in bits 0..15, bf16 bias in 16..31.
__device__ __forceinline__ uint32_t sb_word(float scale, float bias)
{
    return (__float_as_uint(scale) >> 16) | (__float_as_uint(bias) & 0xFFFF0000u);
}

// Codes of 8 consecutive values (chunk ch of a slot) into a token-major K row:
// 8-bit codes fill two words, 4-bit codes one, element e at bits [bits*e', ...)
// of its word (little-endian).
__device__ __forceinline__ void store_k_chunk(uint32_t* row, int ch, int bits, const uint32_t (&q)[8])
{
    if (bits == 8) {
        uint2 w;
        w.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        w.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        *reinterpret_cast<uint2*>(row + ch * 2) = w;
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= q[e] << (4 * e);
        row[ch] = w;
    }
}

}  // namespace kvq

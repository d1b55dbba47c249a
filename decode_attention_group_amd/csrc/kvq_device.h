// Device helpers for the gfx950 kernels: vector types, code -> fp16 conversion,
// MFMA wrappers and wave-level reductions.  Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Tag a pointer as global memory.  Pointers read from a kernel-argument array
// at a run-time index lose their address space; accesses through them would be
// flat_* instructions, which count against the LDS wait counter as well and
// so serialize LDS reads behind in-flight global loads.
template <class T>
__device__ __forceinline__ T* as_global(T* p)
{
    using GT = __attribute__((address_space(1))) T;
    return (T*)reinterpret_cast<GT*>(reinterpret_cast<uintptr_t>(p));
}

// Work item of workgroup `bid` of `n`: workgroups are dealt to the 8 XCDs in
// turn, so this gives each XCD a run of consecutive items (items that read the
// same keys then share that XCD's L2).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_item(int bid, int n)
{
    const int x = bid % kXcds, k = bid / kXcds;
    const int q = n / kXcds, r = n % kXcds;
    return x * q + min(x, r) + k;
}

// Slot of a position already reduced to [0, 2R): one conditional subtraction.
__device__ __forceinline__ int wrap_slot(int slot, int R) { return slot >= R ? slot - R : slot; }

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp16 pair holding two 8-bit codes exactly.  v_perm_b32 builds the bytes
// {code_a, 0x64, code_b, 0x64}: the fp16 values 1024 + code, exact because
// fp16 has a 10-bit fraction; subtracting 1024 leaves the codes themselves.
// `sel` picks the code bytes: 0x04010400 -> bytes 0,1; 0x04030402 -> bytes 2,3.
// (v_perm_b32 D = bytes of {src0:src1}; selector 0..3 = src1 bytes, 4..7 = src0.)
__device__ __forceinline__ f16x2 u8pair_to_f16x2(uint32_t w, uint32_t sel)
{
    const uint32_t m = __builtin_amdgcn_perm(0x64646464u, w, sel);
    f16x2 h = __builtin_bit_cast(f16x2, m);
    return h - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
}

// fp16 pair holding nibbles i and i+4 of w (i in 0..3) exactly, the same way.
__device__ __forceinline__ f16x2 u4pair_to_f16x2(uint32_t w, int i)
{
    const uint32_t m = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
    f16x2 h = __builtin_bit_cast(f16x2, m);
    return h - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
}

// 16 8-bit codes (4 words) -> two MFMA operands of 8 fp16 each, in element order.
__device__ __forceinline__ void codes8x16_to_f16(const u32x4 w, f16x8 &a0, f16x8 &a1)
{
    f16x2 p0 = u8pair_to_f16x2(w.x, 0x04010400u), p1 = u8pair_to_f16x2(w.x, 0x04030402u);
    f16x2 p2 = u8pair_to_f16x2(w.y, 0x04010400u), p3 = u8pair_to_f16x2(w.y, 0x04030402u);
    f16x2 p4 = u8pair_to_f16x2(w.z, 0x04010400u), p5 = u8pair_to_f16x2(w.z, 0x04030402u);
    f16x2 p6 = u8pair_to_f16x2(w.w, 0x04010400u), p7 = u8pair_to_f16x2(w.w, 0x04030402u);
    a0 = (f16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    a1 = (f16x8){p4.x, p4.y, p5.x, p5.y, p6.x, p6.y, p7.x, p7.y};
}

// 16 8-bit codes (4 words) -> two operands of fp16 values 1024 + code (one
// v_perm_b32 per pair, no subtraction); the caller cancels the offset.
__device__ __forceinline__ void codes8x16_to_f16_off(const u32x4 w, f16x8 &a0, f16x8 &a1)
{
    const uint32_t lo = 0x04010400u, hi = 0x04030402u, c = 0x64646464u;
    const u32x4 x0 = {__builtin_amdgcn_perm(c, w.x, lo), __builtin_amdgcn_perm(c, w.x, hi),
                      __builtin_amdgcn_perm(c, w.y, lo), __builtin_amdgcn_perm(c, w.y, hi)};
    const u32x4 x1 = {__builtin_amdgcn_perm(c, w.z, lo), __builtin_amdgcn_perm(c, w.z, hi),
                      __builtin_amdgcn_perm(c, w.w, lo), __builtin_amdgcn_perm(c, w.w, hi)};
    a0 = __builtin_bit_cast(f16x8, x0);
    a1 = __builtin_bit_cast(f16x8, x1);
}

// 8 4-bit codes (1 word) -> fp16 values 1024 + code, element order {0,4,1,5,2,6,3,7}.
__device__ __forceinline__ f16x8 codes4x8_to_f16_off(uint32_t w)
{
    const u32x4 x = {(w & 0x000F000Fu) | 0x64006400u, ((w >> 4) & 0x000F000Fu) | 0x64006400u,
                     ((w >> 8) & 0x000F000Fu) | 0x64006400u, ((w >> 12) & 0x000F000Fu) | 0x64006400u};
    return __builtin_bit_cast(f16x8, x);
}

// 8 8-bit codes (2 words) -> one operand of 8 fp16, element order.
__device__ __forceinline__ f16x8 codes8x8_to_f16(const u32x2 w)
{
    f16x2 p0 = u8pair_to_f16x2(w.x, 0x04010400u), p1 = u8pair_to_f16x2(w.x, 0x04030402u);
    f16x2 p2 = u8pair_to_f16x2(w.y, 0x04010400u), p3 = u8pair_to_f16x2(w.y, 0x04030402u);
    return (f16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 8 4-bit codes (1 word) -> one operand of 8 fp16 in the element order
// {0,4,1,5,2,6,3,7} (the order the nibble pairs come out in).
__device__ __forceinline__ f16x8 codes4x8_to_f16(uint32_t w)
{
    f16x2 p0 = u4pair_to_f16x2(w, 0), p1 = u4pair_to_f16x2(w, 1);
    f16x2 p2 = u4pair_to_f16x2(w, 2), p3 = u4pair_to_f16x2(w, 3);
    return (f16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Element e of an 8-wide 4-bit operand holds code index kNib[e].
__device__ __forceinline__ constexpr int nib_order(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }

// 16x16x32 MFMA, fp16 / bf16 inputs, fp32 accumulate.  Lane l supplies A row
// (l%16) and B column (l%16) with 8 K-values each; lanes l, l+16, l+32, l+48
// together cover K = 32.  The result lane l holds C[4*(l/16) + i][l%16], i < 4.
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reductions across the four 16-lane row groups (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap permutes: v_permlane16_swap(v, v) leaves lane l
// holding v_l and v_(l^16) in its two results, v_permlane32_swap(v, v) v_l
// and v_(l^32).  VALU only, no LDS round trip.  The pairs are combined as
// (l, l^16) first, then (l, l^32): every lane of the four gets the same value.
__device__ __forceinline__ float max_with_l16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_across_groups(float v)
{
    v = max_with_l16(v);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_groups(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace kvq

// Measurement probes for gfx950: the ceilings that the attention kernels are
// compared with besides the chip's published peaks.
//   stream_read_kernel: reads a buffer once with 128-bit loads (optionally
//     non-temporal), grid-stride, four loads in flight per thread per
//     iteration; the bytes read over the time is the attainable HBM read rate.
//   mfma_loop_kernel: back-to-back bf16 MFMAs on register operands, several
//     independent accumulators per wave so the matrix pipe never waits on a
//     result; the FLOPs over the time is the attainable dense bf16 rate.
// Neither reads or writes anything but its own buffers; each writes one word
// per thread only under a condition the data never meets (it keeps the work
// from being optimized away).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq_probes.h"

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kNever = 0x9E3779B9u;

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n_vec,
                                                          uint32_t* __restrict__ sink)
{
    constexpr int kUnroll = 4;
    const size_t stride = (size_t)gridDim.x * 256 * kUnroll;
    size_t i = (size_t)blockIdx.x * 256 * kUnroll + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * 256 < n_vec; i += stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = NT ? __builtin_nontemporal_load(src + i + u * 256) : src[i + u * 256];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n_vec; i += 256) acc ^= src[i];
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == kNever) sink[blockIdx.x * 256 + threadIdx.x] = r;
}

// Each workgroup reads its own contiguous segment (as a split of a KV read does),
// four 16-byte loads in flight per thread per iteration.
template <bool NT>
__global__ __launch_bounds__(256) void segment_read_kernel(const u32x4* __restrict__ src, size_t seg_vec,
                                                           uint32_t* __restrict__ sink)
{
    constexpr int kUnroll = 4;
    const u32x4* base = src + (size_t)blockIdx.x * seg_vec;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = threadIdx.x;
    for (; i + (kUnroll - 1) * 256 < seg_vec; i += 256 * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = NT ? __builtin_nontemporal_load(base + i + u * 256) : base[i + u * 256];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < seg_vec; i += 256) acc ^= base[i];
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == kNever) sink[blockIdx.x * 256 + threadIdx.x] = r;
}

// SHAPE 0: v_mfma_f32_16x16x32_bf16 (16384 FLOP each), 8 accumulators per wave;
// SHAPE 1: v_mfma_f32_32x32x16_bf16 (32768 FLOP each), 4 accumulators per wave.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
    }
    float total = 0.0f;
    if constexpr (SHAPE == 0) {
        f32x4 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) total += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    } else {
        f32x16 c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) c[j][e] = 0.0f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) total += c[j][e];
    }
    if (__float_as_uint(total) == kNever) sink[blockIdx.x * 256 + threadIdx.x] = total;
}

}  // namespace

KVQ_API int kvq_probe_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t nontemporal,
                                  uint32_t* sink, hipStream_t stream)
{
    if (!src || !sink || blocks < 1 || (reinterpret_cast<uintptr_t>(src) & 15) || bytes % 16) return 1;
    const size_t n_vec = bytes / 16;
    if (nontemporal)
        stream_read_kernel<true><<<blocks, 256, 0, stream>>>(static_cast<const u32x4*>(src), n_vec, sink);
    else
        stream_read_kernel<false><<<blocks, 256, 0, stream>>>(static_cast<const u32x4*>(src), n_vec, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

KVQ_API int kvq_probe_segment_read(const void* src, size_t segment_bytes, int32_t blocks, int32_t nontemporal,
                                   uint32_t* sink, hipStream_t stream)
{
    if (!src || !sink || blocks < 1 || (reinterpret_cast<uintptr_t>(src) & 15) || segment_bytes % 16) return 1;
    const size_t seg_vec = segment_bytes / 16;
    if (nontemporal)
        segment_read_kernel<true><<<blocks, 256, 0, stream>>>(static_cast<const u32x4*>(src), seg_vec, sink);
    else
        segment_read_kernel<false><<<blocks, 256, 0, stream>>>(static_cast<const u32x4*>(src), seg_vec, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

KVQ_API int kvq_probe_mfma_bf16(int32_t shape, int32_t iters, int32_t blocks, float* sink, hipStream_t stream)
{
    if (!sink || blocks < 1 || iters < 1 || (shape != 0 && shape != 1)) return 1;
    if (shape == 0) mfma_loop_kernel<0><<<blocks, 256, 0, stream>>>(iters, sink);
    else mfma_loop_kernel<1><<<blocks, 256, 0, stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

KVQ_API double kvq_probe_mfma_flops_per_iter(int32_t shape, int32_t blocks)
{
    const double per = shape == 0 ? 8.0 * 2 * 16 * 16 * 32 : 4.0 * 2 * 32 * 32 * 16;
    return per * 4.0 /* waves per block */ * blocks;
}

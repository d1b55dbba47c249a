// Quantize-and-append: fp32 keys/values -> affine group-64 codes written at
// ring slots (page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff,
// model.ts attentionTraining: cache.appendWindow before the read; page 78,
// gemma4-e4b.ts Gemma4Layer.kv: 4- or 8-bit affine codes, group 64).
//
// One workgroup owns one 8-slot block of one (sequence, KV head) cache, for K
// or for V, so the blocked V words of that block are read-merged-written by a
// single workgroup: no two workgroups of a call touch the same word.
// Eight consecutive lanes quantize one 64-value group (8 values each).
#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant.h"

namespace kvq {

#pragma clang fp contract(off)

typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One workgroup's block: (bx, h, bz) as the single-cache grid (blocks, H, 2B)
// numbers them.  tok: 8 ints of LDS; vq: 8 x D bytes of LDS.
template <int D>
__device__ __forceinline__ void append_body(const AppendParams& p, int bx, int h, int bz, lds_i32* tok,
                                            lds_u8* vq)
{
    constexpr int G = D / 64;
    constexpr int CH = D / 8;                 // 8-value chunks per slot
    // tok[j]: token written into slot j of the block, or -1; vcode: the block's
    // V codes, slot-major
    auto vcode = [&](int j, int d) -> lds_u8& { return vq[j * D + d]; };

    const int b = bz >> 1;
    const bool is_v = bz & 1;
    const int H = p.H, R = p.R, T = p.T;
    const int bits = is_v ? p.v_bits : p.k_bits;
    const float* __restrict__ x = is_v ? p.v : p.k;
    uint32_t* __restrict__ codes = is_v ? p.v_codes : p.k_codes;
    uint32_t* __restrict__ sb = is_v ? p.v_sb : p.k_sb;
    const int nblk = R / 8;
    const int64_t bh = (int64_t)b * H + h;

    const int64_t p_lo = (int64_t)p.pos0[b] + p.t_first;
    const int first_slot = (int)(((p_lo % R) + R) % R);   // in [0, R) even for a bad pos0
    const int blk = (first_slot / 8 + bx) % nblk;
    if (threadIdx.x < 8) {
        const int slot = blk * 8 + threadIdx.x;
        const int off = (slot - first_slot + R) % R;
        tok[threadIdx.x] = off < p.n_written ? p.t_first + off : -1;
    }
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) any |= tok[j] >= 0;
    if (!any) return;

    const int top = (1 << bits) - 1;
    for (int task = threadIdx.x; task < 8 * CH; task += blockDim.x) {
        const int j = task / CH;              // slot within the block
        const int ch = task % CH;             // values [8*ch, 8*ch + 8)
        const int t = tok[j];
        if (t < 0) continue;                  // whole 8-lane groups skip together
        const float* src = x + ((bh * T + t) * D + ch * 8);
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 c = *reinterpret_cast<const float4*>(src + 4);
        float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        uint32_t q[8];
        float scale, bias;
        quantize_group8(v, top, q, scale, bias);
        const int slot = blk * 8 + j;
        if ((ch & 7) == 0)
            sb[(bh * R + slot) * G + (ch >> 3)] = sb_word(scale, bias);
        if (!is_v) {
            store_k_chunk(codes + (bh * R + slot) * (int64_t)(D * bits / 32), ch, bits, q);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vcode(j, ch * 8 + e) = (uint8_t)q[e];
        }
    }
    if (!is_v) return;
    __syncthreads();

    // Merge the block's new V codes into its words: for each d, the 8 slots'
    // codes sit in bits/4 words, slot t at bits [bits*t, bits*(t+1)).
    bool all = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) all &= tok[j] >= 0;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        uint32_t* w = codes + ((bh * nblk + blk) * D + d) * (bits / 4);
        if (bits == 4) {
            uint32_t acc = all ? 0u : w[0];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (tok[j] >= 0) acc = (acc & ~(0xFu << (4 * j))) | ((uint32_t)vcode(j, d) << (4 * j));
            w[0] = acc;
        } else {
            uint32_t lo = all ? 0u : w[0], hi = all ? 0u : w[1];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (tok[j] >= 0) lo = (lo & ~(0xFFu << (8 * j))) | ((uint32_t)vcode(j, d) << (8 * j));
#pragma unroll
            for (int j = 4; j < 8; ++j)
                if (tok[j] >= 0) hi = (hi & ~(0xFFu << (8 * (j - 4)))) | ((uint32_t)vcode(j, d) << (8 * (j - 4)));
            w[0] = lo;
            w[1] = hi;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p)
{
    __shared__ int tok[8];
    __shared__ uint8_t vcode[8 * D];
    append_body<D>(p, blockIdx.x, blockIdx.y, blockIdx.z, (lds_i32*)tok, (lds_u8*)vcode);
}

// Several caches' appends in one launch (a decode step of a donor and a full
// layer): block ranges in order of the caches, each numbered as its own grid.
__global__ __launch_bounds__(256) void append_kernel_multi(AppendMulti P)
{
    __shared__ int tok[8];
    __shared__ uint8_t vcode[8 * 512];
    int i = 0;
    while (i + 1 < P.n && (int)blockIdx.x >= P.block_begin[i + 1]) ++i;
    const AppendParams& p = P.a[i];
    int local = (int)blockIdx.x - P.block_begin[i];
    const int bx = local % P.n_cand[i];
    local /= P.n_cand[i];
    const int h = local % p.H, bz = local / p.H;
    lds_i32* t = (lds_i32*)tok;
    lds_u8* v = (lds_u8*)vcode;
    switch (p.D) {
    case 64: append_body<64>(p, bx, h, bz, t, v); break;
    case 128: append_body<128>(p, bx, h, bz, t, v); break;
    case 192: append_body<192>(p, bx, h, bz, t, v); break;
    case 256: append_body<256>(p, bx, h, bz, t, v); break;
    case 320: append_body<320>(p, bx, h, bz, t, v); break;
    case 384: append_body<384>(p, bx, h, bz, t, v); break;
    case 448: append_body<448>(p, bx, h, bz, t, v); break;
    case 512: append_body<512>(p, bx, h, bz, t, v); break;
    default: break;
    }
}

hipError_t launch_append_multi(const AppendMulti& p, hipStream_t stream)
{
    const int blocks = p.block_begin[p.n];
    if (blocks <= 0) return hipSuccess;
    append_kernel_multi<<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, int n_cand, hipStream_t stream)
{
    const dim3 grid(n_cand, p.H, 2 * p.B);
    switch (p.D) {
    case 64: append_kernel<64><<<grid, 256, 0, stream>>>(p); break;
    case 128: append_kernel<128><<<grid, 256, 0, stream>>>(p); break;
    case 192: append_kernel<192><<<grid, 256, 0, stream>>>(p); break;
    case 256: append_kernel<256><<<grid, 256, 0, stream>>>(p); break;
    case 320: append_kernel<320><<<grid, 256, 0, stream>>>(p); break;
    case 384: append_kernel<384><<<grid, 256, 0, stream>>>(p); break;
    case 448: append_kernel<448><<<grid, 256, 0, stream>>>(p); break;
    case 512: append_kernel<512><<<grid, 256, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq

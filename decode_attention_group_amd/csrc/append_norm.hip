// Normalize, rotate and append in one kernel (page 80 of the @mlx-bun/inference
// 0.0.0-stage -> 1.0.0 diff, gemma4/model.ts attentionTraining: the keys go
// through kNorm and then the rotary embedding at their cache positions, the
// values through vNorm, and both are then appended to the cache; the header
// notes give the value norm no learned scale and let the rotation cover only
// part of head_dim).
//
//   RMS factor  r   = fp32(1 / sqrt(ss / D + eps)), ss the sum of the row's
//                     squares in fp64 over a pairwise tree (the row padded with
//                     zeros to a power of two, neighbours (2i, 2i+1) added at
//                     each level), the quotient and root in fp64
//   keys        y_d = fp32(fp32(x_d * r) * w_d); then, for j < n/2 with the
//                     caller's table at the token's position (c, s):
//                     y_j <- fp32(fp32(y_j c) - fp32(y_{j+n/2} s)),
//                     y_{j+n/2} <- fp32(fp32(y_{j+n/2} c) + fp32(y_j s))
//   values      y_d = fp32(x_d * r)
// and the rows are then quantized (or rounded to bf16) exactly as the plain
// append does.  Every fp32 step is one IEEE operation (no contraction).
//
// Launch: as the plain append, one workgroup per 8-slot block of one (sequence,
// KV head) cache, K or V.  Pass 1 gives each row a power-of-two group of lanes
// (8 values a lane, padding lanes hold zeros), so the fp64 tree above is the
// lane's own 8-value tree followed by xor butterflies inside the group; the
// normed rows go to LDS.  Pass 2 rotates from LDS (the partner column may sit
// in any lane), quantizes each 64-value group on 8 lanes and stores.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant.h"

namespace kvq {

#pragma clang fp contract(off)

template <int D>
__global__ __launch_bounds__(256) void append_norm_kernel(NormAppendParams P)
{
    const AppendParams& p = P.a;
    constexpr int G = D / 64;
    constexpr int CH = D / 8;                 // 8-value chunks per row
    constexpr int LP = CH <= 8 ? 8 : CH <= 16 ? 16 : CH <= 32 ? 32 : 64;   // pass-1 lanes per row
    __shared__ int tok[8];
    __shared__ float yrow[8][D];              // normed rows of the block, slot-major
    __shared__ uint8_t vcode[8][D];

    const int b = blockIdx.z >> 1;
    const bool is_v = blockIdx.z & 1;
    const int h = blockIdx.y;
    const int H = p.H, R = p.R, T = p.T;
    const int bits = is_v ? p.v_bits : p.k_bits;
    const float* __restrict__ x = is_v ? p.v : p.k;
    float* __restrict__ out = is_v ? P.v_out : P.k_out;
    uint32_t* __restrict__ codes = is_v ? p.v_codes : p.k_codes;
    uint32_t* __restrict__ sb = is_v ? p.v_sb : p.k_sb;
    const float* __restrict__ w = is_v ? nullptr : P.k_weight;
    const int nblk = R / 8;
    const int64_t bh = (int64_t)b * H + h;

    const int64_t p_lo = (int64_t)p.pos0[b] + p.t_first;
    const int first_slot = (int)(((p_lo % R) + R) % R);
    const int blk = (first_slot / 8 + (int)blockIdx.x) % nblk;
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

    // pass 1: RMS factor and the normed (weighted) row
    for (int task = threadIdx.x; task < 8 * LP; task += blockDim.x) {
        const int j = task / LP, l = task % LP;
        const int t = tok[j];
        if (t < 0) continue;                  // whole lane groups skip together
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (l < CH) {
            const float* src = x + ((bh * T + t) * D + l * 8);
            const float4 a = *reinterpret_cast<const float4*>(src);
            const float4 c = *reinterpret_cast<const float4*>(src + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        }
        double sq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sq[e] = (double)v[e] * (double)v[e];
        double s = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
#pragma unroll
        for (int m = 1; m < LP; m <<= 1) s += __shfl_xor(s, m);
        const float f = (float)(1.0 / __builtin_sqrt(s / (double)D + (double)P.eps));
        if (l < CH) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = v[e] * f;
                yrow[j][l * 8 + e] = w ? y * w[l * 8 + e] : y;
            }
        }
    }
    __syncthreads();

    // pass 2: rotation (keys), then the append of the block's rows
    const int half = is_v ? 0 : P.rope_half;
    const int top = (1 << bits) - 1;
    for (int task = threadIdx.x; task < 8 * CH; task += blockDim.x) {
        const int j = task / CH;
        const int ch = task % CH;
        const int t = tok[j];
        if (t < 0) continue;                  // whole 8-lane groups skip together
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = yrow[j][ch * 8 + e];
        if (half > 0 && ch * 8 < 2 * half) {
            int64_t pos = (int64_t)p.pos0[b] + t;
            pos = pos < 0 ? 0 : (pos >= P.rope_positions ? P.rope_positions - 1 : pos);
            const float* cs = P.rope_cos + pos * half;
            const float* sn = P.rope_sin + pos * half;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = ch * 8 + e;
                if (d < half) {
                    const float a = v[e], bb = yrow[j][d + half];
                    const float ac = a * cs[d], bs = bb * sn[d];
                    v[e] = ac - bs;
                } else if (d < 2 * half) {
                    const float a = yrow[j][d - half], bb = v[e];
                    const float bc = bb * cs[d - half], as = a * sn[d - half];
                    v[e] = bc + as;
                }
            }
        }
        if (out) {
            float* dst = out + ((bh * T + t) * D + ch * 8);
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
        const int slot = blk * 8 + j;
        if (bits == 16) {                     // bf16 cache: round and store
            if (!is_v) {
                uint4 wd;
                wd.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
                wd.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
                wd.z = (uint32_t)f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
                wd.w = (uint32_t)f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
                *reinterpret_cast<uint4*>(codes + (bh * R + slot) * (int64_t)(D / 2) + ch * 4) = wd;
            } else {
                uint16_t* vd = reinterpret_cast<uint16_t*>(codes) + ((bh * nblk + blk) * D + ch * 8) * 8 + j;
#pragma unroll
                for (int e = 0; e < 8; ++e) vd[e * 8] = f32_to_bf16_rne(v[e]);
            }
            continue;
        }
        uint32_t q[8];
        float scale, bias;
        quantize_group8(v, top, q, scale, bias);
        if ((ch & 7) == 0)
            sb[(bh * R + slot) * G + (ch >> 3)] = sb_word(scale, bias);
        if (!is_v) {
            store_k_chunk(codes + (bh * R + slot) * (int64_t)(D * bits / 32), ch, bits, q);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vcode[j][ch * 8 + e] = (uint8_t)q[e];
        }
    }
    if (!is_v || bits == 16) return;
    __syncthreads();

    // Merge the block's new V codes into its words (as the plain append does).
    bool all = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) all &= tok[j] >= 0;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        uint32_t* wp = codes + ((bh * nblk + blk) * D + d) * (bits / 4);
        if (bits == 4) {
            uint32_t acc = all ? 0u : wp[0];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (tok[j] >= 0) acc = (acc & ~(0xFu << (4 * j))) | ((uint32_t)vcode[j][d] << (4 * j));
            wp[0] = acc;
        } else {
            uint32_t lo = all ? 0u : wp[0], hi = all ? 0u : wp[1];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (tok[j] >= 0) lo = (lo & ~(0xFFu << (8 * j))) | ((uint32_t)vcode[j][d] << (8 * j));
#pragma unroll
            for (int j = 4; j < 8; ++j)
                if (tok[j] >= 0) hi = (hi & ~(0xFFu << (8 * (j - 4)))) | ((uint32_t)vcode[j][d] << (8 * (j - 4)));
            wp[0] = lo;
            wp[1] = hi;
        }
    }
}

hipError_t launch_append_norm(const NormAppendParams& P, int n_cand, hipStream_t stream)
{
    const dim3 grid(n_cand, P.a.H, 2 * P.a.B);
    switch (P.a.D) {
    case 64: append_norm_kernel<64><<<grid, 256, 0, stream>>>(P); break;
    case 128: append_norm_kernel<128><<<grid, 256, 0, stream>>>(P); break;
    case 192: append_norm_kernel<192><<<grid, 256, 0, stream>>>(P); break;
    case 256: append_norm_kernel<256><<<grid, 256, 0, stream>>>(P); break;
    case 320: append_norm_kernel<320><<<grid, 256, 0, stream>>>(P); break;
    case 384: append_norm_kernel<384><<<grid, 256, 0, stream>>>(P); break;
    case 448: append_norm_kernel<448><<<grid, 256, 0, stream>>>(P); break;
    case 512: append_norm_kernel<512><<<grid, 256, 0, stream>>>(P); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq

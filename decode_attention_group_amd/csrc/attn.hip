// Split-KV flash attention over an affine group-quantized cache, gfx950:
// the launches of the plain reads (one descriptor, or several of one
// configuration), of the multi-configuration read and of the combine.  The
// device code is in attn_impl.h; the fused decode step of a single
// descriptor launches from attn_step.hip.
#include "attn_impl.h"

namespace kvq {

// One launch over descriptors of different configurations: the Gemma 4 decode
// step reads a head_dim 256 sliding donor and a head_dim 512 full donor.
__global__ __launch_bounds__(256) void attn_kernel_multi(AttnParams P)
{
    // One LDS block sized for head_dim 512; the head_dim 256 bodies use a prefix of it.
    static_assert(sizeof(AttnSmem<256, true>) <= sizeof(AttnSmem<512, true>), "LDS reuse");
    __shared__ AttnSmem<512, true> sm;
    AttnSmem<256, true>& sm256 =
        *(AttnSmem<256, true>*)(__attribute__((address_space(3))) AttnSmem<256, true>*)(&sm);
    const int bid = blockIdx.x;
    const int di = find_desc(P, bid);
    const AttnDesc& d = P.d[di];
    const int idx = bid - d.item_begin;
    switch (d.cfg) {
    case cfg_of(256, 4, 4): attn_body<256, 4, 4, kTokFold>(d, idx, sm256); break;
    case cfg_of(256, 4, 8): attn_body<256, 4, 8, kTokFold>(d, idx, sm256); break;
    case cfg_of(256, 8, 4): attn_body<256, 8, 4, kTokFold>(d, idx, sm256); break;
    case cfg_of(256, 8, 8): attn_body<256, 8, 8, kTokFold>(d, idx, sm256); break;
    case cfg_of(512, 4, 4): attn_body<512, 4, 4, kTokFold>(d, idx, sm); break;
    case cfg_of(512, 4, 8): attn_body<512, 4, 8, kTokFold>(d, idx, sm); break;
    case cfg_of(512, 8, 4): attn_body<512, 8, 4, kTokFold>(d, idx, sm); break;
    case cfg_of(512, 8, 8): attn_body<512, 8, 8, kTokFold>(d, idx, sm); break;
    default: break;
    }
}

// One workgroup per (descriptor, sequence and KV head, row, 64-column chunk):
// out = sum_s w_s o_s / sum_s w_s l_s, w_s = 2^(m_s - max m).  The 256 threads
// are 16 column quads x 16 split lanes.  Each split lane issues the loads of all
// its splits first, then folds them with a running max, so the partials are
// read in one round trip; the 16 lanes' results meet in LDS.  Splits that saw
// no key (m_s = -inf) contribute nothing.  A descriptor with part_h holds o_s / l_s
// as fp16, which is multiplied back by l_s.
constexpr int kCombCols = 64;
constexpr int kCombLanes = 16;
constexpr int kCombMaxPer = kMaxSplits / kCombLanes;

__global__ __launch_bounds__(256) void combine_kernel(AttnParams P)
{
    __shared__ f32x4 red_o[kCombLanes][16];
    __shared__ float red_m[kCombLanes], red_l[kCombLanes];
    const int bid = blockIdx.x;
    int di = -1;
    for (int i = 0; i < P.n_desc; ++i)
        if (P.d[i].S > 1 && bid >= P.d[i].comb_begin) di = i;
    if (di < 0) return;
    const AttnDesc& d = P.d[di];
    const int S = d.S, D = d.D;
    const int nch = D / kCombCols;
    int ir = bid - d.comb_begin;
    const int ch = ir % nch;
    ir /= nch;
    const int grow = ir % d.n_rows;          // row of the (sequence, KV head)
    const int bh = ir / d.n_rows;
    const int b = bh / d.Hkv, hkv = bh - b * d.Hkv;
    const int r = grow % kRowTile;
    const int ib = bh * d.n_rt + grow / kRowTile;
    const float* po = as_global(d.part);
    const float* pml = as_global(d.part) + (size_t)d.B * d.Hkv * d.n_rt * S * kRowTile * D;
    const int tid = threadIdx.x;
    const int q4 = tid & 15;           // column quad within the chunk
    const int sl = tid >> 4;           // split lane: splits sl, sl + 16, ...
    const int col = ch * kCombCols + 4 * q4;
    const int64_t sstride = (int64_t)kRowTile * D;
    const float* src = po + (((int64_t)ib * S) * kRowTile + r) * D + col;
    const float* msrc = pml + (((int64_t)ib * S) * kRowTile + r) * 2;

    float ms[kCombMaxPer], ls[kCombMaxPer];
    f32x4 os[kCombMaxPer];
#pragma unroll
    for (int j = 0; j < kCombMaxPer; ++j) {
        const int s = sl + kCombLanes * j;
        if (s < S) {
            const float2 ml = *reinterpret_cast<const float2*>(msrc + (int64_t)s * kRowTile * 2);
            ms[j] = ml.x;
            ls[j] = ml.y;
            if (d.part_h) {                    // o / l as fp16: back to o
                const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(po) +
                                                                (((int64_t)ib * S + s) * kRowTile + r) * D + col);
                const f16x2 lo = __builtin_bit_cast(f16x2, w.x), hi = __builtin_bit_cast(f16x2, w.y);
                os[j] = (f32x4){(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]} * ml.y;
            } else {
                os[j] = *reinterpret_cast<const f32x4*>(src + s * sstride);
            }
        } else {
            ms[j] = -INFINITY;
            ls[j] = 0.0f;
            os[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCombMaxPer; ++j) M = fmaxf(M, ms[j]);
    float L = 0.0f;
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kCombMaxPer; ++j) {
        if (ms[j] == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(ms[j] - M);
        L += w * ls[j];
        acc += w * os[j];
    }
    red_o[sl][q4] = acc;
    if (q4 == 0) { red_m[sl] = M; red_l[sl] = L; }
    __syncthreads();
    if (sl != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombLanes; ++i) Mt = fmaxf(Mt, red_m[i]);
    float Lt = 0.0f;
    f32x4 ot = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kCombLanes; ++i) {
        const float mi = red_m[i];
        if (mi == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(mi - Mt);
        Lt += w * red_l[i];
        ot += w * red_o[i][q4];
    }
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
    ot *= inv;
    const RowMap rm = map_row(d, hkv, grow);
    uint16_t* orow = as_global(d.out[rm.layer]) + ((((int64_t)b * d.Hq + rm.hq) * d.C + rm.qi) * D);
    uint2 w;
    w.x = f32_to_bf16_rne(ot[0]) | ((uint32_t)f32_to_bf16_rne(ot[1]) << 16);
    w.y = f32_to_bf16_rne(ot[2]) | ((uint32_t)f32_to_bf16_rne(ot[3]) << 16);
    *reinterpret_cast<uint2*>(orow + col) = w;
}

hipError_t launch_attn(const AttnParams& p, int total_items, bool multi, hipStream_t stream)
{
    const dim3 grid(total_items);
    if (multi) {
        for (int i = 0; i < p.n_desc; ++i)
            if (p.d[i].k_new != nullptr && !p.d[i].tok_fold) return hipErrorInvalidValue;
        return launch_read(attn_kernel_multi, grid, dim3(256), p, stream);
    }
    // one descriptor without a token: the plain kernel; otherwise the kernel that
    // takes folded tokens (a token as a split of its own launches from attn_step.hip)
    const bool plain = p.n_desc == 1 && p.d[0].k_new == nullptr;
    for (int i = 0; i < p.n_desc; ++i)
        if (p.d[i].k_new != nullptr && !p.d[i].tok_fold) return hipErrorInvalidValue;
    switch (p.d[0].cfg) {
#define KVQ_CASE(D_, KB_, VB_) \
    case cfg_of(D_, KB_, VB_): \
        return plain ? launch_read(attn_kernel<D_, KB_, VB_, true, kTokNone>, grid, dim3(64 * Shape<D_>::NW), p, stream) \
                     : launch_read(attn_kernel<D_, KB_, VB_, false, kTokFold>, grid, dim3(64 * Shape<D_>::NW), p, stream);
#define KVQ_D(D_) KVQ_CASE(D_, 4, 4) KVQ_CASE(D_, 4, 8) KVQ_CASE(D_, 8, 4) KVQ_CASE(D_, 8, 8)
    KVQ_D(64) KVQ_D(128) KVQ_D(192) KVQ_D(256) KVQ_D(320) KVQ_D(384) KVQ_D(448) KVQ_D(512)
#undef KVQ_D
#undef KVQ_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const AttnParams& p, hipStream_t stream)
{
    int blocks = 0;
    for (int i = 0; i < p.n_desc; ++i)
        if (p.d[i].S > 1)
            blocks = p.d[i].comb_begin + p.d[i].B * p.d[i].Hkv * p.d[i].n_rows * (p.d[i].D / kCombCols);
    if (blocks == 0) return hipSuccess;
    combine_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace kvq

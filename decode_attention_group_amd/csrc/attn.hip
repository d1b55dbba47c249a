// Split-KV flash attention over an affine group-quantized cache, gfx950.
//
// What it computes (page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0
// diff, gemma4/model.ts header notes and attentionTraining): for every query
// row, softmax(scale * q . khat_j) over the visible keys j, times vhat_j, where
// khat = code * scale + bias per 64-value group (page 78, gemma4-e4b.ts
// Gemma4Layer.kv).  Query rows that share a KV head (GQA heads, KV-sharing
// layers, chunk queries) form 16-row tiles; keys stream in steps of 32.
//
// The contractions run on MFMA 16x16x32 (fp16 in, fp32 accumulate) in the
// transposed form S^T = K Q^T and O^T = V^T P^T, so that each lane ends a QK
// step holding the probabilities of one query row for 8 consecutive keys --
// exactly the B operand the PV step needs, with no shuffle between the two.
// Codes become fp16 exactly in registers (no dequantized copy); the per-group
// scale and bias are folded in instead of applied per element:
//   q . khat_j = sum_g s_jg * (sum_{d in g} q_d c_jd) + sum_g b_jg * Q_g,
//   Q_g = sum_{d in g} q_d (one extra bf16 MFMA per tile, Q_g split in 3 bf16
//   parts), and
//   sum_j p_j vhat_jd = sum_j (p_j s_jg) c_jd + sum_j p_j b_jg
//   (the second term for all groups at once in one fp16 MFMA per step).
// Scales and biases of a step are staged in LDS.  The online-softmax max is
// reduced across the four 16-lane groups of the wave with lane shuffles.
// Each workgroup has 4 waves that take alternate steps of its key range and
// merge (max, sum, output) through LDS at the end; a split with S > 1 leaves
// fp32 partials that the combine kernel reduces.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kWaves = 4;

constexpr int kMergeChunk = 256;   // head_dim columns merged per LDS round

template <int D>
struct AttnSmem {
    static constexpr int G = D / 64;
    union {
        struct {
            uint32_t k_kg[kWaves][kStep][G];   // K scale|bias, key-major
            uint32_t k_gk[kWaves][G][kStep];   // K scale|bias, group-major
            uint32_t v_gk[kWaves][G][kStep];   // V scale|bias, group-major
        } sb;
        float mrg[kWaves - 1][kRowTile][kMergeChunk + 4];
    } u;
    float ml[kWaves][kRowTile][2];
};

struct RowMap {
    int layer, qi, hq;
};

__device__ __forceinline__ RowMap map_row(const AttnDesc& P, int hkv, int grow)
{
    RowMap r;
    const int hh = grow % P.hpk;
    if (P.C == 1) { r.layer = grow / P.hpk; r.qi = 0; }
    else { r.layer = 0; r.qi = grow / P.hpk; }
    r.hq = hkv * P.hpk + hh;
    return r;
}

__device__ __forceinline__ int wrap(int slot, int R) { return slot >= R ? slot - R : slot; }

template <int D, int KB, int VB>
__device__ __forceinline__ void attn_body(const AttnDesc& P, int idx, AttnSmem<D>& sm)
{
    constexpr int G = D / 64;
    constexpr int DT = D / 16;
    constexpr int KW = D * KB / 32;      // K words per slot
    constexpr int VW = VB / 4;           // V words per (block, d)
    constexpr int NL = G / 2;            // scale|bias words each lane stages per step

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;

    const int S = P.S;
    const int s = idx % S;
    const int rt = (idx / S) % P.n_rt;
    const int bh = idx / (S * P.n_rt);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int len = min(max(P.len[b], 0), P.max_len);
    const int R = P.R, W = P.W, C = P.C;

    // ---- key range of this work item
    const int row0 = rt * kRowTile;
    const int last_row = min(row0 + kRowTile, P.n_rows) - 1;
    const int qi_lo = C == 1 ? 0 : row0 / P.hpk;
    const int qi_hi = C == 1 ? 0 : last_row / P.hpk;
    int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
    lo = max(lo, max(0, len - R));
    const int hi = len - C + qi_hi;
    const int base = lo & ~(kStep - 1);
    const int j0 = max(lo, base + s * P.split_len);
    const int j1 = min(hi + 1, base + (s + 1) * P.split_len);

    // ---- this lane's query row
    const int grow = row0 + m;
    const bool row_ok = grow < P.n_rows;
    const RowMap rm = map_row(P, hkv, row_ok ? grow : row0);
    const int p_row = len - C + rm.qi;
    int klo = max(j0, W > 0 ? p_row - W + 1 : 0);
    int khi = min(j1 - 1, p_row);
    if (!row_ok) { klo = 1; khi = 0; }

    // ---- q as MFMA B operand (fp16, element order matching the K code order),
    //      and the per-group sums Q_g for the bias term
    f16x8 qf[G][2];
    float qsum[G];
    {
        const uint16_t* qrow = P.q[rm.layer] + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            u32x4 u0 = 0, u1 = 0;
            if (row_ok) {
                u0 = *reinterpret_cast<const u32x4*>(qrow + gi * 64 + lg * 16);
                u1 = *reinterpret_cast<const u32x4*>(qrow + gi * 64 + lg * 16 + 8);
            }
            float f[16];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = bf16_lo_to_f32(u0[e]);
                f[2 * e + 1] = bf16_hi_to_f32(u0[e]);
                f[8 + 2 * e] = bf16_lo_to_f32(u1[e]);
                f[8 + 2 * e + 1] = bf16_hi_to_f32(u1[e]);
            }
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc += f[e];
            qsum[gi] = sum_across_groups(acc);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int e0 = KB == 8 ? e : nib_order(e);
                qf[gi][0][e] = (_Float16)f[e0];
                qf[gi][1][e] = (_Float16)f[8 + e0];
            }
        }
    }
    bf16x8 qb;
    {
        u32x4 w = 0;
        if (lg < 3) {
            uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const float q1 = __uint_as_float((uint32_t)f32_to_bf16_rne(qsum[gi]) << 16);
                const float r1 = qsum[gi] - q1;
                const float q2 = __uint_as_float((uint32_t)f32_to_bf16_rne(r1) << 16);
                const float r2 = r1 - q2;
                h[gi] = lg == 0 ? (uint16_t)(__float_as_uint(q1) >> 16)
                      : lg == 1 ? (uint16_t)(__float_as_uint(q2) >> 16)
                                : f32_to_bf16_rne(r2);
            }
            w = (u32x4){h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                        h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
        }
        qb = __builtin_bit_cast(bf16x8, w);
    }

    const float sl2e = P.scale_log2e;
    f32x4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    f32x4 corr = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    const int st0 = j0 & ~(kStep - 1);
    const int64_t kslot0 = (int64_t)bh * R;
    const uint32_t* kcodes = P.k_codes;
    const uint32_t* vcodes = P.v_codes;

    for (int si = wave; si < nsteps; si += kWaves) {
        const int st = st0 + si * kStep;
        const int st_mod = st % R;

        // ---- stage this step's scale|bias words in LDS
        {
            const int kk = lane >> 1, g0 = (lane & 1) * NL;
            const int slot = wrap(st_mod + kk, R);
            const uint32_t* ks = P.k_sb + (kslot0 + slot) * G + g0;
            const uint32_t* vs = P.v_sb + (kslot0 + slot) * G + g0;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const uint32_t kw = ks[i], vw = vs[i];
                sm.u.sb.k_kg[wave][kk][g0 + i] = kw;
                sm.u.sb.k_gk[wave][g0 + i][kk] = kw;
                sm.u.sb.v_gk[wave][g0 + i][kk] = vw;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- S^T = K Q^T for the step's two 16-key tiles.  Tile t row r holds
        //      key 8*(r/4) + 4*t + r%4, so lane group lg ends with keys 8*lg .. 8*lg+7.
        float z[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            const int slot = wrap(st_mod + kk, R);
            const uint32_t* krow = kcodes + (kslot0 + slot) * KW;
            bf16x8 ab;
            {
                u32x4 w = 0;
                if (lg < 3) {
                    uint32_t bw[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) bw[e] = e < G ? sm.u.sb.k_kg[wave][kk][e < G ? e : 0] >> 16 : 0u;
                    w = (u32x4){bw[0] | (bw[1] << 16), bw[2] | (bw[3] << 16),
                                bw[4] | (bw[5] << 16), bw[6] | (bw[7] << 16)};
                }
                ab = __builtin_bit_cast(bf16x8, w);
            }
            f32x4 sacc = mfma_bf16(ab, qb, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                f16x8 a0, a1;
                if constexpr (KB == 8) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(krow + gi * 16 + lg * 4);
                    codes8x16_to_f16(w, a0, a1);
                } else {
                    const u32x2 w = *reinterpret_cast<const u32x2*>(krow + gi * 8 + lg * 2);
                    a0 = codes4x8_to_f16(w.x);
                    a1 = codes4x8_to_f16(w.y);
                }
                f32x4 x = mfma_f16(a0, qf[gi][0], (f32x4){0.f, 0.f, 0.f, 0.f});
                x = mfma_f16(a1, qf[gi][1], x);
                const u32x4 sw = *reinterpret_cast<const u32x4*>(&sm.u.sb.k_gk[wave][gi][8 * lg + 4 * t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[i] += bf16_lo_to_f32(sw[i]) * x[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = st + 8 * lg + 4 * t + i;
                z[4 * t + i] = (key >= klo && key <= khi) ? sacc[i] * sl2e : -INFINITY;
            }
        }

        // ---- online softmax (base 2); one query row per lane, max over the 4 lane groups
        float mloc = z[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, z[k]);
        const float m_new = fmaxf(m_run, max_across_groups(mloc));
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float p[8];
        float psum = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) { p[k] = __builtin_amdgcn_exp2f(z[k] - m_use); psum += p[k]; }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
            corr *= alpha;
        }

        // ---- O^T += V^T (P * s_v)^T per group, and the bias term for all groups
        // vk: key visible to this lane's query row (B side, per row);
        // kin: key inside the item's range, i.e. its slot holds real data (A side,
        // shared by all rows -- an A row here is a quantization group, not a query row).
        bool vk[8], kin[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int key = st + 8 * lg + k;
            vk[k] = z[k] != -INFINITY;
            kin[k] = key >= j0 && key < j1;
        }
        {
            f16x8 pb, ac;
            u32x4 w0 = 0, w1 = 0;
            if (m < G) {
                w0 = *reinterpret_cast<const u32x4*>(&sm.u.sb.v_gk[wave][m < G ? m : 0][8 * lg]);
                w1 = *reinterpret_cast<const u32x4*>(&sm.u.sb.v_gk[wave][m < G ? m : 0][8 * lg + 4]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = VB == 8 ? e : nib_order(e);
                const uint32_t bw = k < 4 ? w0[k & 3] : w1[k & 3];
                pb[e] = (_Float16)p[k];
                ac[e] = kin[k] ? (_Float16)bf16_hi_to_f32(bw) : (_Float16)0.0f;
            }
            corr = mfma_f16(ac, pb, corr);
        }
        const int vslot = wrap(st_mod + 8 * lg, R);
        const uint32_t* vrow = vcodes + (((int64_t)bh * (R / 8) + (vslot >> 3)) * D + m) * VW;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const u32x4 s0 = *reinterpret_cast<const u32x4*>(&sm.u.sb.v_gk[wave][gi][8 * lg]);
            const u32x4 s1 = *reinterpret_cast<const u32x4*>(&sm.u.sb.v_gk[wave][gi][8 * lg + 4]);
            f16x8 bs;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = VB == 8 ? e : nib_order(e);
                const float sv = bf16_lo_to_f32(k < 4 ? s0[k & 3] : s1[k & 3]);
                bs[e] = vk[k] ? (_Float16)(p[k] * sv) : (_Float16)0.0f;
            }
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const int dt = 4 * gi + dd;
                f16x8 a;
                if constexpr (VB == 8) a = codes8x8_to_f16(*reinterpret_cast<const u32x2*>(vrow + 16 * dt * VW));
                else a = codes4x8_to_f16(vrow[16 * dt * VW]);
                O[dt] = mfma_f16(a, bs, O[dt]);
            }
        }
    }

    // ---- fold the bias term into O: lane (m, lg) holds corr[group 4*lg+i][row m]
    const float l_row = sum_across_groups(l_run);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        const float c = __shfl(corr[gi & 3], m + 16 * (gi >> 2));
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) O[4 * gi + dd] += c;
    }

    // ---- merge the 4 waves through LDS, kMergeChunk columns at a time
    __syncthreads();                                   // all waves are done with the sb area
    if (lg == 0) { sm.ml[wave][m][0] = m_run; sm.ml[wave][m][1] = l_row; }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.ml[w][m][0]);
    float L = 0.0f, scl0 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.ml[w][m][0];
        const float sw = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        L += sw * sm.ml[w][m][1];
        if (w == 0) scl0 = sw;
    }
    const float scl_self = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    constexpr int TPC = kMergeChunk / 16;              // d-tiles per merge chunk
#pragma unroll
    for (int c = 0; c < (DT + TPC - 1) / TPC; ++c) {
        if (wave > 0) {
            float* dst = &sm.u.mrg[wave - 1][m][4 * lg];
#pragma unroll
            for (int dt = c * TPC; dt < (c + 1) * TPC && dt < DT; ++dt)
                *reinterpret_cast<f32x4*>(dst + 16 * (dt - c * TPC)) = O[dt] * scl_self;
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int dt = c * TPC; dt < (c + 1) * TPC && dt < DT; ++dt) {
                f32x4 acc = O[dt] * scl0;
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
                    acc += *reinterpret_cast<const f32x4*>(&sm.u.mrg[w - 1][m][16 * (dt - c * TPC) + 4 * lg]);
                O[dt] = acc;
            }
        }
        __syncthreads();
    }
    if (wave != 0 || !row_ok) return;

    if (S == 1) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* orow = P.out[rm.layer] + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = O[dt] * inv;
            uint2 w;
            w.x = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
            w.y = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
            *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * lg) = w;
        }
    } else {
        const int64_t ib = (int64_t)bh * P.n_rt + rt;
        const int64_t prow = (ib * S + s) * kRowTile + m;
        float* po = P.part + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * lg) = O[dt];
        if (lg == 0) {
            float* pml = P.part + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
            pml[0] = M;
            pml[1] = L;
        }
    }
}

__device__ __forceinline__ int find_desc(const AttnParams& P, int bid)
{
    int di = 0;
    while (di + 1 < P.n_desc && bid >= P.d[di + 1].item_begin) ++di;
    return di;
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams P)
{
    __shared__ AttnSmem<D> sm;
    const int bid = blockIdx.x;
    const int di = find_desc(P, bid);
    attn_body<D, KB, VB>(P.d[di], bid - P.d[di].item_begin, sm);
}

// One launch over descriptors of different configurations: the Gemma 4 decode
// step reads a head_dim 256 sliding donor and a head_dim 512 full donor.
__global__ __launch_bounds__(256) void attn_kernel_multi(AttnParams P)
{
    // One LDS block sized for head_dim 512; the head_dim 256 bodies use a prefix of it.
    static_assert(sizeof(AttnSmem<256>) <= sizeof(AttnSmem<512>), "LDS reuse");
    __shared__ AttnSmem<512> sm;
    AttnSmem<256>& sm256 = *reinterpret_cast<AttnSmem<256>*>(&sm);
    const int bid = blockIdx.x;
    const int di = find_desc(P, bid);
    const AttnDesc& d = P.d[di];
    const int idx = bid - d.item_begin;
    switch (d.cfg) {
    case 4: attn_body<256, 4, 4>(d, idx, sm256); break;
    case 5: attn_body<256, 4, 8>(d, idx, sm256); break;
    case 6: attn_body<256, 8, 4>(d, idx, sm256); break;
    case 7: attn_body<256, 8, 8>(d, idx, sm256); break;
    case 8: attn_body<512, 4, 4>(d, idx, sm); break;
    case 9: attn_body<512, 4, 8>(d, idx, sm); break;
    case 10: attn_body<512, 8, 4>(d, idx, sm); break;
    case 11: attn_body<512, 8, 8>(d, idx, sm); break;
    default: break;
    }
}

__global__ __launch_bounds__(256) void combine_kernel(AttnParams P)
{
    __shared__ float wts[kRowTile][kMaxSplits];
    const int bid = blockIdx.x;
    int di = -1;
    for (int i = 0; i < P.n_desc; ++i)
        if (P.d[i].S > 1 && bid >= P.d[i].comb_begin) di = i;
    if (di < 0) return;
    const AttnDesc& d = P.d[di];
    const int ib = bid - d.comb_begin;
    const int rt = ib % d.n_rt;
    const int bh = ib / d.n_rt;
    const int b = bh / d.Hkv, hkv = bh - b * d.Hkv;
    const int S = d.S, D = d.D;
    const float* po = d.part;
    const float* pml = d.part + (size_t)d.B * d.Hkv * d.n_rt * S * kRowTile * D;
    const int tid = threadIdx.x;
    if (tid < kRowTile) {
        const int64_t r0 = ((int64_t)ib * S) * kRowTile + tid;
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) M = fmaxf(M, pml[(r0 + (int64_t)s * kRowTile) * 2]);
        float L = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float ms = pml[(r0 + (int64_t)s * kRowTile) * 2];
            const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            wts[tid][s] = w;
            L += w * pml[(r0 + (int64_t)s * kRowTile) * 2 + 1];
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        for (int s = 0; s < S; ++s) wts[tid][s] *= inv;
    }
    __syncthreads();
    const int D4 = D / 4;
    for (int e = tid; e < kRowTile * D4; e += blockDim.x) {
        const int r = e / D4, d4 = e - r * D4;
        const int grow = rt * kRowTile + r;
        if (grow >= d.n_rows) continue;
        f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; ++s) {
            const float w = wts[r][s];
            if (w == 0.0f) continue;
            acc += w * *reinterpret_cast<const f32x4*>(po + ((((int64_t)ib * S + s) * kRowTile + r) * D + 4 * d4));
        }
        const RowMap rm = map_row(d, hkv, grow);
        uint16_t* orow = d.out[rm.layer] + ((((int64_t)b * d.Hq + rm.hq) * d.C + rm.qi) * D);
        uint2 w;
        w.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        w.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(orow + 4 * d4) = w;
    }
}

hipError_t launch_attn(const AttnParams& p, int total_items, bool multi, hipStream_t stream)
{
    const dim3 grid(total_items), block(64 * kWaves);
    if (multi) {
        attn_kernel_multi<<<grid, block, 0, stream>>>(p);
        return hipGetLastError();
    }
    switch (p.d[0].cfg) {
#define KVQ_CASE(D_, KB_, VB_) \
    case (D_ == 128 ? 0 : D_ == 256 ? 1 : 2) * 4 + (KB_ == 8 ? 2 : 0) + (VB_ == 8 ? 1 : 0): \
        attn_kernel<D_, KB_, VB_><<<grid, block, 0, stream>>>(p); break;
    KVQ_CASE(128, 4, 4) KVQ_CASE(128, 4, 8) KVQ_CASE(128, 8, 4) KVQ_CASE(128, 8, 8)
    KVQ_CASE(256, 4, 4) KVQ_CASE(256, 4, 8) KVQ_CASE(256, 8, 4) KVQ_CASE(256, 8, 8)
    KVQ_CASE(512, 4, 4) KVQ_CASE(512, 4, 8) KVQ_CASE(512, 8, 4) KVQ_CASE(512, 8, 8)
#undef KVQ_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const AttnParams& p, hipStream_t stream)
{
    int blocks = 0;
    for (int i = 0; i < p.n_desc; ++i)
        if (p.d[i].S > 1) blocks = p.d[i].comb_begin + p.d[i].B * p.d[i].Hkv * p.d[i].n_rt;
    if (blocks == 0) return hipSuccess;
    combine_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace kvq

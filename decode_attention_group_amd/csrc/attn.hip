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
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// Waves of a workgroup split head_dim: wave w owns the quantization groups
// [w*GPW, (w+1)*GPW).  All waves walk the same 32-key steps; each computes a
// partial S^T over its groups, the partials meet in LDS (one barrier per step,
// double-buffered by step parity), every wave then holds the full scores and
// the same softmax state, and accumulates O^T for its own head_dim columns.
template <int D>
struct Shape {
    static constexpr int G = D / 64;
    static constexpr int NW = G >= 4 ? 4 : G;      // waves per workgroup
    static constexpr int GPW = G / NW;              // groups per wave
    static constexpr int DTW = 4 * GPW;             // 16-column tiles of O^T per wave
};

template <int D>
struct AttnSmem {
    static constexpr int NW = Shape<D>::NW, GPW = Shape<D>::GPW;
    f32x4 spart[2][NW][2][kWave];          // partial S^T tiles, [step parity][wave][tile][lane]
    uint32_t ksb[NW][GPW][kStep];          // this step's K scale|bias words, per wave, group-major
    uint32_t vsb[NW][GPW][kStep];          // V scale|bias words
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

// Registers holding one step's codes and scale|bias words (the prefetch unit).
template <int D, int KB, int VB>
struct StepRegs {
    static constexpr int GPW = Shape<D>::GPW, DTW = Shape<D>::DTW;
    typename std::conditional<KB == 8, u32x4, u32x2>::type kc[2][GPW];
    typename std::conditional<VB == 8, u32x2, uint32_t>::type vc[DTW];
    uint32_t ksb, vsb;
};

template <int D, int KB, int VB>
__device__ __forceinline__ void attn_body(const AttnDesc& P, int idx, AttnSmem<D>& sm)
{
    using Sh = Shape<D>;
    constexpr int G = Sh::G, NW = Sh::NW, GPW = Sh::GPW, DTW = Sh::DTW;
    constexpr int KW = D * KB / 32;      // K words per slot
    constexpr int VW = VB / 4;           // V words per (block, d)

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;
    const int g0 = wave * GPW;           // first group of this wave

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

    // ---- q of this wave's groups as MFMA B operand (fp16, element order matching
    //      the K code order), and the group sums Q_g for the bias term
    f16x8 qf[GPW][2];
    bf16x8 qb;
    {
        const uint16_t* qrow = P.q[rm.layer] + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
        float qsum[GPW];
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int gg = g0 + gi;
            u32x4 u0 = 0, u1 = 0;
            if (row_ok) {
                u0 = *reinterpret_cast<const u32x4*>(qrow + gg * 64 + lg * 16);
                u1 = *reinterpret_cast<const u32x4*>(qrow + gg * 64 + lg * 16 + 8);
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
        // k-slots 8*lg + e: Q_g split in three bf16 parts (lg = 0, 1, 2) for group g0+e
        u32x4 w = 0;
        if (lg < 3) {
            uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
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
    f32x4 O[DTW];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    f32x4 corr = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    const int st0 = j0 & ~(kStep - 1);
    const int64_t kslot0 = (int64_t)bh * R;
    const uint32_t* __restrict__ kcodes = P.k_codes;
    const uint32_t* __restrict__ vcodes = P.v_codes;
    // lane -> (key, group) of the scale|bias word it stages each step
    const int sb_key = GPW == 2 ? lane >> 1 : lane & 31;
    const int sb_g = GPW == 2 ? lane & 1 : 0;
    const bool sb_on = GPW == 2 || lane < 32;

    auto load_step = [&](StepRegs<D, KB, VB>& r, int st) {
        const int st_mod = st % R;
        // scale|bias words first: they are the first thing a step consumes
        const int64_t sbi = (kslot0 + wrap(st_mod + sb_key, R)) * G + g0 + sb_g;
        r.ksb = P.k_sb[sb_on ? sbi : kslot0 * G];
        r.vsb = P.v_sb[sb_on ? sbi : kslot0 * G];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            const uint32_t* krow = kcodes + (kslot0 + wrap(st_mod + kk, R)) * KW;
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
                if constexpr (KB == 8) r.kc[t][gi] = *reinterpret_cast<const u32x4*>(krow + (g0 + gi) * 16 + lg * 4);
                else r.kc[t][gi] = *reinterpret_cast<const u32x2*>(krow + (g0 + gi) * 8 + lg * 2);
            }
        }
        const int vslot = wrap(st_mod + 8 * lg, R);
        const uint32_t* vrow = vcodes + (((int64_t)bh * (R / 8) + (vslot >> 3)) * D + 64 * g0 + m) * VW;
#pragma unroll
        for (int dd = 0; dd < DTW; ++dd) {
            if constexpr (VB == 8) r.vc[dd] = *reinterpret_cast<const u32x2*>(vrow + 16 * dd * VW);
            else r.vc[dd] = vrow[16 * dd * VW];
        }
    };

    // One step: stage scale|bias, partial scores, exchange, softmax, PV.
    // `par` alternates the LDS score buffer between consecutive steps.
    auto compute_step = [&](const StepRegs<D, KB, VB>& cr, int st, int par) {
        // ---- stage the step's scale|bias words in this wave's LDS region
        if (sb_on) {
            sm.ksb[wave][sb_g][sb_key] = cr.ksb;
            sm.vsb[wave][sb_g][sb_key] = cr.vsb;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- partial S^T over this wave's groups.  Tile t row r holds key
        //      8*(r/4) + 4*t + r%4, so lane group lg ends with keys 8*lg .. 8*lg+7.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            bf16x8 ab;
            {
                u32x4 w = 0;
                if (lg < 3) {
                    uint32_t bw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                    for (int e = 0; e < GPW; ++e) bw[e] = sm.ksb[wave][e][kk] >> 16;
                    w = (u32x4){bw[0] | (bw[1] << 16), bw[2] | (bw[3] << 16),
                                bw[4] | (bw[5] << 16), bw[6] | (bw[7] << 16)};
                }
                ab = __builtin_bit_cast(bf16x8, w);
            }
            f32x4 sacc = mfma_bf16(ab, qb, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
                f16x8 a0, a1;
                if constexpr (KB == 8) codes8x16_to_f16(cr.kc[t][gi], a0, a1);
                else { a0 = codes4x8_to_f16(cr.kc[t][gi].x); a1 = codes4x8_to_f16(cr.kc[t][gi].y); }
                f32x4 x = mfma_f16(a0, qf[gi][0], (f32x4){0.f, 0.f, 0.f, 0.f});
                x = mfma_f16(a1, qf[gi][1], x);
                const u32x4 sw = *reinterpret_cast<const u32x4*>(&sm.ksb[wave][gi][8 * lg + 4 * t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[i] += bf16_lo_to_f32(sw[i]) * x[i];
            }
            sm.spart[par][wave][t][lane] = sacc;
        }
        __syncthreads();

        // ---- full scores (same in every wave) and the online softmax, base 2
        float z[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 sacc = sm.spart[par][0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sacc += sm.spart[par][w][t][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = st + 8 * lg + 4 * t + i;
                z[4 * t + i] = (key >= klo && key <= khi) ? sacc[i] * sl2e : -INFINITY;
            }
        }
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
            for (int dt = 0; dt < DTW; ++dt) O[dt] *= alpha;
            corr *= alpha;
        }

        // ---- O^T += V^T (P * s_v)^T per group; the bias term of all groups in one MFMA.
        //      vk: key visible to this lane's query row (B side, per row).  kin: key
        //      inside the item's range, so its slot holds data (A side, where a row
        //      is a quantization group and not a query row).
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
            if (m < GPW) {
                w0 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg]);
                w1 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg + 4]);
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
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const u32x4 s0 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][gi][8 * lg]);
            const u32x4 s1 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][gi][8 * lg + 4]);
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
                if constexpr (VB == 8) a = codes8x8_to_f16(cr.vc[dt]);
                else a = codes4x8_to_f16(cr.vc[dt]);
                O[dt] = mfma_f16(a, bs, O[dt]);
            }
        }
    };

    // Ping-pong between two register sets so the next step's loads stay in
    // flight while this step computes (a register copy would force a wait).
    // The loads are issued unconditionally (the step index is clamped, so past
    // the end the last step is read again and hits L2): a load under a branch
    // would make the wait counters fall back to waiting for every load.
    StepRegs<D, KB, VB> ra, rb;
    const int last = max(nsteps - 1, 0);
    if (nsteps > 0) load_step(ra, st0);
    for (int si = 0; si < nsteps; si += 2) {
        const int st = st0 + si * kStep;
        load_step(rb, st0 + min(si + 1, last) * kStep);
        compute_step(ra, st, 0);
        if (si + 1 >= nsteps) break;
        load_step(ra, st0 + min(si + 2, last) * kStep);
        compute_step(rb, st + kStep, 1);
    }

    // ---- fold the bias term into O: lane (m, lg) holds corr[group row 4*lg+i][query row m]
    const float L = sum_across_groups(l_run);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const float c = __shfl(corr[gi & 3], m + 16 * (gi >> 2));
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) O[4 * gi + dd] += c;
    }
    if (!row_ok) return;
    const int dcol = 64 * g0 + 4 * lg;   // + 16 * dt + i
    if (S == 1) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* orow = P.out[rm.layer] + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
            const f32x4 o = O[dt] * inv;
            uint2 w;
            w.x = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
            w.y = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
            *reinterpret_cast<uint2*>(orow + dcol + 16 * dt) = w;
        }
    } else {
        const int64_t ib = (int64_t)bh * P.n_rt + rt;
        const int64_t prow = (ib * S + s) * kRowTile + m;
        float* po = P.part + prow * D;
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) *reinterpret_cast<f32x4*>(po + dcol + 16 * dt) = O[dt];
        if (wave == 0 && lg == 0) {
            float* pml = P.part + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
            pml[0] = m_run;
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
__global__ __launch_bounds__(64 * Shape<D>::NW) void attn_kernel(AttnParams P)
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

// One workgroup per (descriptor, row tile item, row, 64-column chunk):
// out = sum_s w_s o_s / sum_s w_s l_s, w_s = 2^(m_s - max m).  The 256 threads
// are 16 column quads x 16 split lanes; each split lane sums every 16th split
// and the 16 sums meet in LDS.  Splits that saw no key (m_s = -inf) are skipped.
constexpr int kCombCols = 64;

__global__ __launch_bounds__(256) void combine_kernel(AttnParams P)
{
    __shared__ float wts[kMaxSplits];
    __shared__ f32x4 red[16][16];
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
    const int r = ir % kRowTile;
    const int ib = ir / kRowTile;
    const int rt = ib % d.n_rt;
    const int bh = ib / d.n_rt;
    const int b = bh / d.Hkv, hkv = bh - b * d.Hkv;
    const int grow = rt * kRowTile + r;
    if (grow >= d.n_rows) return;
    const float* po = d.part;
    const float* pml = d.part + (size_t)d.B * d.Hkv * d.n_rt * S * kRowTile * D;
    const int tid = threadIdx.x;
    if (tid < 64) {
        float M = -INFINITY;
        for (int s = tid; s < S; s += 64) M = fmaxf(M, pml[(((int64_t)ib * S + s) * kRowTile + r) * 2]);
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        float L = 0.0f;
        for (int s = tid; s < S; s += 64) {
            const float* ml = pml + (((int64_t)ib * S + s) * kRowTile + r) * 2;
            const float w = ml[0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[0] - M);
            wts[s] = w;
            L += w * ml[1];
        }
        for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        for (int s = tid; s < S; s += 64) wts[s] *= inv;
    }
    __syncthreads();
    const int q4 = tid & 15;           // column quad within the chunk
    const int sl = tid >> 4;           // split lane
    const int col = ch * kCombCols + 4 * q4;
    const float* src = po + (((int64_t)ib * S) * kRowTile + r) * D + col;
    const int64_t sstride = (int64_t)kRowTile * D;
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int s = sl; s < S; s += 16) {
        const float w = wts[s];
        if (w != 0.0f) acc += w * *reinterpret_cast<const f32x4*>(src + s * sstride);
    }
    red[sl][q4] = acc;
    __syncthreads();
    if (sl != 0) return;
#pragma unroll
    for (int i = 1; i < 16; ++i) acc += red[i][q4];
    const RowMap rm = map_row(d, hkv, grow);
    uint16_t* orow = d.out[rm.layer] + ((((int64_t)b * d.Hq + rm.hq) * d.C + rm.qi) * D);
    uint2 w;
    w.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    w.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<uint2*>(orow + col) = w;
}

hipError_t launch_attn(const AttnParams& p, int total_items, bool multi, hipStream_t stream)
{
    const dim3 grid(total_items);
    if (multi) {
        attn_kernel_multi<<<grid, dim3(256), 0, stream>>>(p);
        return hipGetLastError();
    }
    switch (p.d[0].cfg) {
#define KVQ_CASE(D_, KB_, VB_) \
    case (D_ == 128 ? 0 : D_ == 256 ? 1 : 2) * 4 + (KB_ == 8 ? 2 : 0) + (VB_ == 8 ? 1 : 0): \
        attn_kernel<D_, KB_, VB_><<<grid, dim3(64 * Shape<D_>::NW), 0, stream>>>(p); break;
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
        if (p.d[i].S > 1)
            blocks = p.d[i].comb_begin + p.d[i].B * p.d[i].Hkv * p.d[i].n_rt * kRowTile * (p.d[i].D / kCombCols);
    if (blocks == 0) return hipSuccess;
    combine_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace kvq

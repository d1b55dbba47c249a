// Split-KV flash attention over an affine group-quantized cache, gfx950: the
// device code shared by attn.hip (plain reads, the multi-configuration launch,
// the combine) and attn_step.hip (the fused decode step's kernels).
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
// The waves of a workgroup split head_dim (see Shape); their partial scores meet
// in LDS once per step.  A split with S > 1 leaves fp32 partials (output, max,
// sum) that the combine kernel reduces.
#pragma once

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "quant.h"

namespace kvq {

// Waves of a workgroup split head_dim: wave w owns the quantization groups
// [w*GPW, (w+1)*GPW).  All waves walk the same 32-key steps; each computes a
// partial S^T over its groups, the partials meet in LDS (one barrier per step,
// double-buffered by step parity), every wave then holds the full scores and
// the same softmax state, and accumulates O^T for its own head_dim columns.
template <int D>
struct Shape {
    static constexpr int G = D / 64;
    // waves per workgroup: one per group up to four groups, else one per pair of
    // groups (6, 8) or one per group (5, 7)
    static constexpr int NW = G <= 4 ? G : (G % 2 == 0 ? G / 2 : G);
    static constexpr int GPW = G / NW;              // groups per wave (1 or 2)
    static constexpr int DTW = 4 * GPW;             // 16-column tiles of O^T per wave
    static_assert(G * 64 == D && G >= 1 && G <= 8 && NW * GPW == G, "head_dim a multiple of 64 up to 512");
};

// TOK: room for a folded token's values (kTokFold kernels).
template <int D, bool TOK>
struct AttnSmem {
    static constexpr int NW = Shape<D>::NW, GPW = Shape<D>::GPW;
    f32x4 spart[2][NW][2][kWave];          // partial S^T tiles, [step parity][wave][tile][lane]
    uint32_t ksb[NW][GPW][kStep];          // this step's K scale|bias words, per wave, group-major
    uint32_t vsb[NW][GPW][kStep];          // V scale|bias words
    float tokv[TOK ? D : 4];               // fused step: the token's dequantized values
};

struct RowMap {
    int layer, qi, hq;
};

// (readfirstlane keeps a pointer a scalar value.)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Query / output pointer of each lane's layer.  The 16 rows of a tile cover
// layers LO..HI (uniform); a short uniform loop loads each of those pointers
// with a scalar load and selects per lane.  (An unrolled select over all
// entries is turned by the compiler into a per-lane table lookup: a vector
// load that delays the q loads, or a private copy in scratch.)
#define KVQ_LAYER_PTR(T, ARR, LO, HI, LAYER) ([&]() {                              \
        uint64_t p_ = 0;                                                          \
        _Pragma("nounroll") for (int l_ = (LO); l_ <= (HI); ++l_) {               \
            const uint64_t a_ = uniform_u64(reinterpret_cast<uint64_t>((ARR)[l_])); \
            if ((LAYER) == l_) p_ = a_;                                           \
        }                                                                         \
        return as_global(reinterpret_cast<T*>(p_));                              \
    }())

__device__ __forceinline__ RowMap map_row(const AttnDesc& P, int hkv, int grow)
{
    RowMap r;
    const int hh = grow % P.hpk;
    if (P.C == 1) { r.layer = grow / P.hpk; r.qi = 0; }
    else { r.layer = 0; r.qi = grow / P.hpk; }
    r.hq = hkv * P.hpk + hh;
    return r;
}


// Registers holding one step's K codes / V codes and scale|bias words (the
// prefetch units; K runs one step ahead of V).
template <int D, int KB>
struct KRegs {
    typename std::conditional<KB == 8, u32x4, u32x2>::type kc[2][Shape<D>::GPW];
    uint32_t sb;
};
template <int D, int VB>
struct VRegs {
    typename std::conditional<VB == 8, u32x2, uint32_t>::type vc[Shape<D>::DTW];
    uint32_t sb;
};

constexpr int kTokNone = 0, kTokSplit = 1, kTokFold = 2;

// Largest growth (log2 units) of a row's running max absorbed without
// rescaling: probabilities are taken against a stale max and may reach 2^8.
constexpr float kRescaleSlack = 8.0f;

// (lds in the LDS address space: generic stores here could alias the kernel
// arguments, which would then be copied to private memory)
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Fused decode step, as a split of its own (a launch of one descriptor).  The
// token at position len-1 is quantized here with the
// append kernel's device code (so the codes are the same bit for bit), written
// into the cache by the item of row tile 0, and attended from its dequantized
// values as one more split of every item: for each row, m = scale*log2(e) *
// (q . khat), l = 1, o = vhat; the other splits leave that position out.  The
// V words of the token's 8-slot block are read, merged and written while other
// workgroups may be reading them: only the token's own bits change, so either
// order gives them the other slots' codes.
template <int D, int KB, int VB>
__device__ __forceinline__ void new_token_split(const AttnDesc& P, int bh, int rt, int s, lds_f32* lds)
{
    constexpr int NT = 64 * Shape<D>::NW;           // threads
    constexpr int G = D / 64, CH = D / 8, VW = VB / 4;
    // lanes per query row in the dot product: a power of 2 (shuffle reduction)
    // that leaves each lane a multiple of 8 elements
    constexpr int PARTS = NT / kRowTile >= 16 && G % 2 == 0 ? 16 : NT / kRowTile >= 8 ? 8 : NT / kRowTile;
    constexpr int EPP = D / PARTS;                  // elements per lane
    static_assert(2 * CH <= NT && EPP % 8 == 0 && EPP * PARTS == D, "one chunk per thread");
    static_assert((2 * D * 4 + D) <= (int)sizeof(AttnSmem<D, false>), "fits the attention LDS");
    lds_f32* khat = lds;
    lds_f32* vhat = lds + D;
    lds_u8* vq = reinterpret_cast<lds_u8*>(lds + 2 * D);
    const int tid = threadIdx.x;
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int R = P.R;
    const int len = min(max(__builtin_amdgcn_readfirstlane(as_global(P.len)[b]), 1), P.max_len);
    const int slot = (len - 1) % R;
    const bool writer = rt == 0;
    // the cache arrays of a fused step are the caller's writable cache
    uint32_t* k_codes = const_cast<uint32_t*>(as_global(P.k_codes));
    uint32_t* v_codes = const_cast<uint32_t*>(as_global(P.v_codes));
    uint32_t* k_sb = const_cast<uint32_t*>(as_global(P.k_sb));
    uint32_t* v_sb = const_cast<uint32_t*>(as_global(P.v_sb));
    if (tid < 2 * CH) {                              // lanes [0, CH): K chunks; [CH, 2CH): V chunks
        const bool is_v = tid >= CH;
        const int ch = is_v ? tid - CH : tid;
        const float* src = as_global(is_v ? P.v_new : P.k_new) + ((int64_t)bh * D + ch * 8);
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 c = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        uint32_t q[8];
        float scale, bias;
        quantize_group8(v, is_v ? (1 << VB) - 1 : (1 << KB) - 1, q, scale, bias);
        lds_f32* xh = is_v ? vhat : khat;
#pragma unroll
        for (int e = 0; e < 8; ++e) xh[ch * 8 + e] = (float)q[e] * scale + bias;
        if (writer) {
            if ((ch & 7) == 0) (is_v ? v_sb : k_sb)[((int64_t)bh * R + slot) * G + ch / 8] = sb_word(scale, bias);
            if (!is_v) store_k_chunk(k_codes + ((int64_t)bh * R + slot) * (D * KB / 32), ch, KB, q);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vq[ch * 8 + e] = (uint8_t)q[e];
            }
        }
    }
    __syncthreads();
    if (writer) {                                    // the token's bits of its V block
        const int t = slot & 7;
        for (int d = tid; d < D; d += NT) {
            uint32_t* w = v_codes + (((int64_t)bh * (R / 8) + slot / 8) * D + d) * VW;
            if constexpr (VB == 4) {
                w[0] = (w[0] & ~(0xFu << (4 * t))) | ((uint32_t)vq[d] << (4 * t));
            } else {
                const int wi = t >> 2, sh = 8 * (t & 3);
                w[wi] = (w[wi] & ~(0xFFu << sh)) | ((uint32_t)vq[d] << sh);
            }
        }
    }
    // q . khat for each row of the tile: PARTS consecutive lanes per row
    const int r = tid / PARTS, part = tid % PARTS;     // threads past 16 rows compute nothing used
    const int grow = rt * kRowTile + r;
    const bool row_ok = r < kRowTile && grow < P.n_rows;
    const RowMap rm = map_row(P, hkv, row_ok ? grow : rt * kRowTile);
    // the tile's rows may belong to several layers (a shared read): each row's own q
    const int lay_lo = map_row(P, hkv, rt * kRowTile).layer;
    const int lay_hi = map_row(P, hkv, min(rt * kRowTile + kRowTile, P.n_rows) - 1).layer;
    const uint16_t* qrow = KVQ_LAYER_PTR(const uint16_t, P.q, lay_lo, lay_hi, rm.layer) +
                           ((((int64_t)b * P.Hq + rm.hq) * P.C + rm.qi) * D + part * EPP);
    const lds_f32* kh = khat + part * EPP;
    float acc = 0.0f;
#pragma unroll
    for (int e0 = 0; e0 < EPP; e0 += 8) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(qrow + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc += bf16_lo_to_f32(u[i]) * kh[e0 + 2 * i] + bf16_hi_to_f32(u[i]) * kh[e0 + 2 * i + 1];
    }
#pragma unroll
    for (int o = 1; o < PARTS; o <<= 1) acc += __shfl_xor(acc, o);
    if (!row_ok) return;
    const int64_t prow = (((int64_t)bh * P.n_rt + rt) * P.S + s) * kRowTile + r;
    float* po = as_global(P.part) + prow * D + part * EPP;
#pragma unroll
    for (int e0 = 0; e0 < EPP; e0 += 4)
        *reinterpret_cast<f32x4*>(po + e0) =
            *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(vhat + part * EPP + e0);
    if (part == 0) {
        float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * P.S * kRowTile * D + prow * 2;
        pml[0] = acc * P.scale_log2e;
        pml[1] = 1.0f;
    }
}

// TOK: the fused decode step's token, if the descriptor carries one (k_new):
//   kTokNone   plain reads only;
//   kTokSplit  the token is split S-1 of every item (new_token_split), beside
//              the others: the shortest path for a launch of one descriptor;
//   kTokFold   the last split of every item takes the token after its keys: no
//              extra split, so an unsplit item (a sliding donor) stays without
//              partials (launches of several descriptors).
template <int D, int KB, int VB, int TOK>
__device__ __forceinline__ void attn_body(const AttnDesc& P, int idx, AttnSmem<D, TOK == kTokFold>& sm)
{
    using Sh = Shape<D>;
    constexpr int G = Sh::G, NW = Sh::NW, GPW = Sh::GPW, DTW = Sh::DTW;
    constexpr int KW = D * KB / 32;      // K words per slot
    constexpr int VW = VB / 4;           // V words per (block, d)
    constexpr int NSLOT = 6 * GPW;       // bias MFMA k-slots in use: {b, s} x 3 parts x groups

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;
    const int g0 = wave * GPW;           // first group of this wave

    const int S = P.S;
    const int s = idx % S;
    const int rt = (idx / S) % P.n_rt;
    const int bh = idx / (S * P.n_rt);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    if (TOK == kTokSplit && P.k_new != nullptr && s == S - 1) {
        new_token_split<D, KB, VB>(P, bh, rt, s, (lds_f32*)(&sm));
        return;
    }
    const int R = P.R, W = P.W, C = P.C;
    // len[b] is read in flight: the ranges below are first taken for the
    // common case len == max_len, so the first code loads go out without
    // waiting for it, and are reissued when it differs.
    // (a vector load: a scalar one would share its wait counter with the
    // kernel-argument loads and be waited for before the first code loads)
    int opaque_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    const int len_lane = as_global(P.len)[b + opaque_zero];

    // ---- key range of this work item, and of this lane's query row
    const int row0 = rt * kRowTile;
    const int last_row = min(row0 + kRowTile, P.n_rows) - 1;
    const int qi_lo = C == 1 ? 0 : row0 / P.hpk;
    const int qi_hi = C == 1 ? 0 : last_row / P.hpk;
    const int grow = row0 + m;
    const bool row_ok = grow < P.n_rows;
    const RowMap rm = map_row(P, hkv, row_ok ? grow : row0);
    const int lay_lo = map_row(P, hkv, row0).layer, lay_hi = map_row(P, hkv, last_row).layer;
    int j0, j1, full_lo, full_hi, klo, khi;
    auto ranges = [&](int len) {
        int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
        lo = max(lo, max(0, len - R));
        const int hi = len - C + qi_hi - P.excl;
        const int base = lo & ~(kStep - 1);
        j0 = max(lo, base + s * P.split_len);
        j1 = min(hi + 1, base + (s + 1) * P.split_len);
        // keys every row of the tile sees (steps inside need no mask)
        full_lo = max(j0, W > 0 ? len - C + qi_hi - W + 1 : 0);
        full_hi = min(j1 - 1, len - C + qi_lo - P.excl);
        const int p_row = len - C + rm.qi;
        klo = max(j0, W > 0 ? p_row - W + 1 : 0);
        khi = min(j1 - 1, p_row - P.excl);
        if (!row_ok) { klo = 1; khi = 0; }
    };
    ranges(P.max_len);

    // ---- q of this wave's groups as MFMA B operand (fp16, element order matching
    //      the K code order); Q_g = sum of the group's q for the bias MFMA
    f16x8 qf[GPW][2];
    float qinv[GPW];     // 2^-k: undoes the power of 2 that put each (row, group) of q in fp16 range
    bf16x8 qb;
    // q loads are unconditional (a lane past the last row reads row 0 of the
    // tile and zeroes it afterwards), so no branch forces an early wait.
    u32x4 qraw[GPW][2];
    auto load_q = [&]() {
        const uint16_t* qrow = KVQ_LAYER_PTR(const uint16_t, P.q, lay_lo, lay_hi, rm.layer) + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            qraw[gi][0] = *reinterpret_cast<const u32x4*>(qrow + (g0 + gi) * 64 + lg * 16);
            qraw[gi][1] = *reinterpret_cast<const u32x4*>(qrow + (g0 + gi) * 64 + lg * 16 + 8);
        }
    };
    auto setup_q = [&]() {
        float qpart[3][GPW];
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const u32x4 u0 = row_ok ? qraw[gi][0] : (u32x4)0;
            const u32x4 u1 = row_ok ? qraw[gi][1] : (u32x4)0;
            float f[16];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = bf16_lo_to_f32(u0[e]);
                f[2 * e + 1] = bf16_hi_to_f32(u0[e]);
                f[8 + 2 * e] = bf16_lo_to_f32(u1[e]);
                f[8 + 2 * e + 1] = bf16_hi_to_f32(u1[e]);
            }
            float acc = 0.0f, amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) { acc += f[e]; amax = fmaxf(amax, fabsf(f[e])); }
            const float Q = sum_across_groups(acc);
            // The row's 64 values of this group enter the MFMA as fp16 after a power
            // of 2 that puts their largest magnitude in [2^14, 2^15): bf16 -> fp16 is
            // then exact for every value within 2^-28 of it, at any magnitude of q.
            // The partial score is multiplied back by qinv (exact).
            const uint32_t ex = min(max((__float_as_uint(max_across_groups(amax)) >> 23) & 0xFFu, 15u), 254u);
            const float qmul = __uint_as_float((268u - ex) << 23);
            qinv[gi] = __uint_as_float((ex - 14u) << 23);
            // Q in three bf16 parts: their sum carries ~24 bits of Q
            const float q1 = __uint_as_float((uint32_t)f32_to_bf16_rne(Q) << 16);
            const float q2 = __uint_as_float((uint32_t)f32_to_bf16_rne(Q - q1) << 16);
            const float q3 = __uint_as_float((uint32_t)f32_to_bf16_rne(Q - q1 - q2) << 16);
            qpart[0][gi] = q1;
            qpart[1][gi] = q2;
            qpart[2][gi] = q3;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int e0 = KB == 8 ? e : nib_order(e);
                qf[gi][0][e] = (_Float16)(f[e0] * qmul);
                qf[gi][1][e] = (_Float16)(f[8 + e0] * qmul);
            }
        }
        // bias k-slot k = (term*3 + part)*GPW + gi: term 0 pairs b with Q, term 1
        // pairs s with -1024 Q (the K codes enter the MFMA as 1024 + code)
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = 8 * lg + e;
            float v = 0.0f;
#pragma unroll
            for (int kk = 0; kk < NSLOT; ++kk)
                if (kk == k) {
                    const int term = kk / (3 * GPW), part = (kk / GPW) % 3, gi = kk % GPW;
                    v = term == 0 ? qpart[part][gi] : -1024.0f * qpart[part][gi];
                }
            h[e] = (uint16_t)(__float_as_uint(v) >> 16);   // exact: bf16 values times a power of 2
        }
        const u32x4 w = {h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                         h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
        qb = __builtin_bit_cast(bf16x8, w);
    };

    const float sl2e = P.scale_log2e;
    f32x4 O[DTW];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    f32x4 corr = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    int st0 = j0 & ~(kStep - 1);
    // step i of the item (clamped to its last step)
    int last = max(nsteps - 1, 0);
    auto stp = [&](int i) { return st0 + min(i, last) * kStep; };
    const int64_t kslot0 = (int64_t)bh * R;
    const uint32_t* __restrict__ kcodes = as_global(P.k_codes) + kslot0 * KW;
    const uint32_t* __restrict__ vcodes = as_global(P.v_codes) + (int64_t)bh * (R / 8) * D * VW;
    const int vlane = (64 * g0 + m) * VW;          // this lane's column within a V block
    // lane -> (key, group) of the scale|bias word it stages each step
    const int sb_key = GPW == 2 ? lane >> 1 : lane & 31;
    const int sb_g = GPW == 2 ? lane & 1 : 0;
    const bool sb_on = GPW == 2 || lane < 32;
    const uint32_t* __restrict__ ksbp = as_global(P.k_sb) + kslot0 * G + g0 + sb_g;
    const uint32_t* __restrict__ vsbp = as_global(P.v_sb) + kslot0 * G + g0 + sb_g;

    auto load_k = [&](KRegs<D, KB>& r, int i) {
        const int st_mod = stp(i) % R;
        r.sb = ksbp[sb_on ? wrap_slot(st_mod + sb_key, R) * G : 0];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            const uint32_t* krow = kcodes + wrap_slot(st_mod + kk, R) * KW;
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
                if constexpr (KB == 8) r.kc[t][gi] = *reinterpret_cast<const u32x4*>(krow + (g0 + gi) * 16 + lg * 4);
                else r.kc[t][gi] = *reinterpret_cast<const u32x2*>(krow + (g0 + gi) * 8 + lg * 2);
            }
        }
    };
    auto load_v = [&](VRegs<D, VB>& r, int i) {
        const int st_mod = stp(i) % R;
        r.sb = vsbp[sb_on ? wrap_slot(st_mod + sb_key, R) * G : 0];
        const uint32_t* vrow = vcodes + ((int64_t)(wrap_slot(st_mod + 8 * lg, R) >> 3) * (D * VW) + vlane);
#pragma unroll
        for (int dd = 0; dd < DTW; ++dd) {
            if constexpr (VB == 8) r.vc[dd] = *reinterpret_cast<const u32x2*>(vrow + 16 * dd * VW);
            else r.vc[dd] = vrow[16 * dd * VW];
        }
    };

    // ---- Staging of a step's scale|bias words in this wave's LDS rows (the
    //      words are read back by other lanes of the same wave after sync_wave).
    auto stage_k = [&](const KRegs<D, KB>& kr) {
        if (sb_on) sm.ksb[wave][sb_g][sb_key] = kr.sb;
    };
    auto stage_v = [&](const VRegs<D, VB>& vr) {
        if (sb_on) sm.vsb[wave][sb_g][sb_key] = vr.sb;
    };
    auto sync_wave = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // ---- QK of one step (its K words staged): partial S^T over this wave's
    //      groups into spart[par].  Tile t row r holds key 8*(r/4) + 4*t + r%4,
    //      so lane group lg ends with keys 8*lg .. 8*lg+7.
    auto qk = [&](const KRegs<D, KB>& kr, int par) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            bf16x8 ab;
            {
                // k-slot k = 8*lg + e < NSLOT holds term k/(3*GPW) (0: the bias, 1: the
                // scale) of group k%GPW.  The group words are read unconditionally and
                // picked with selects: an LDS read under a lane-dependent condition
                // would become a branch with its own wait, once per slot.
                uint32_t wg[GPW];
#pragma unroll
                for (int gi = 0; gi < GPW; ++gi) wg[gi] = sm.ksb[wave][gi][kk];
                uint32_t hw[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = 8 * lg + e;
                    const uint32_t w = wg[GPW - 1] ^ ((k % GPW == 0) ? (wg[0] ^ wg[GPW - 1]) : 0u);
                    const uint32_t v = k / (3 * GPW) == 0 ? (w >> 16) : (w & 0xFFFFu);
                    hw[e] = k < NSLOT ? v : 0u;
                }
                const u32x4 w = {hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16),
                                 hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16)};
                ab = __builtin_bit_cast(bf16x8, w);
            }
            f32x4 sacc = mfma_bf16(ab, qb, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
                f16x8 a0, a1;
                if constexpr (KB == 8) codes8x16_to_f16_off(kr.kc[t][gi], a0, a1);
                else { a0 = codes4x8_to_f16_off(kr.kc[t][gi].x); a1 = codes4x8_to_f16_off(kr.kc[t][gi].y); }
                f32x4 x = mfma_f16(a0, qf[gi][0], (f32x4){0.f, 0.f, 0.f, 0.f});
                x = mfma_f16(a1, qf[gi][1], x);
                const u32x4 sw = *reinterpret_cast<const u32x4*>(&sm.ksb[wave][gi][8 * lg + 4 * t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[i] += (bf16_lo_to_f32(sw[i]) * qinv[gi]) * x[i];
            }
            sm.spart[par][wave][t][lane] = sacc;
        }
    };

    // ---- full scores of one step (the same in every wave once the partials
    //      met behind a barrier), in base 2, and their maximum over the row;
    //      FULL: every key visible to every row.
    auto scores = [&](int st, int par, float (&z)[8], auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 sacc = sm.spart[par][0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sacc += sm.spart[par][w][t][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (FULL) {
                    z[4 * t + i] = sacc[i] * sl2e;
                } else {
                    const int key = st + 8 * lg + 4 * t + i;
                    z[4 * t + i] = (key >= klo && key <= khi) ? sacc[i] * sl2e : -INFINITY;
                }
            }
        }
        float mloc = z[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, z[k]);
        return max_across_groups(mloc);
    };
    // the online softmax in base 2: the running max moves (and O, corr and l
    // are rescaled) only when a row's max grows by more than the slack
    auto rescale = [&](float mt) {
        if (__any(mt > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) O[dt] *= alpha;
            corr *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
    };
    auto probs = [&](const float (&z)[8], float (&p)[8], auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // masked keys come out as exactly 0 (exp2(-inf)); p < 0 flags them for PV
            const float e = __builtin_amdgcn_exp2f(z[k] - m_use);
            l_run += e;
            p[k] = FULL || z[k] != -INFINITY ? e : -1.0f;
        }
    };

    // fp16 operands hold p * s_v (p <= 2^8) and the V bias only while s_v < 2^7
    // and |bias| < 2^15; a visible key beyond that sends this wave's step down
    // the bf16 path, whose operands have fp32 range.
    auto is_wide = [&](const VRegs<D, VB>& vr, int st) {
        const int vkey = st + sb_key;
        const bool big = sb_on && vkey >= j0 && vkey < j1 &&
                         ((vr.sb & 0x7FFFu) >= 0x4300u || ((vr.sb >> 16) & 0x7FFFu) >= 0x4700u);
        return __builtin_amdgcn_ballot_w64(big) != 0;
    };

    // ---- PV of one step with bf16 operands (any V scale and bias): every fp32
    //      weight w (p, or p * s_v) enters as hi = bf16(w) plus lo = bf16(w - hi),
    //      two MFMAs against the exact bf16 codes and biases (about 16 bits of w).
    auto pv_wide = [&](const VRegs<D, VB>& vr, const float (&p)[8], const float (&pp)[8], const bool (&kin)[8],
                       bool full) {
        auto hi_of = [](float w) { return (__bf16)w; };
        auto lo_of = [](float w) { return (__bf16)(w - (float)(__bf16)w); };
        {
            u32x4 w0 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg]);
            u32x4 w1 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg + 4]);
            if (m >= GPW) { w0 = (u32x4)0; w1 = (u32x4)0; }
            bf16x8 ac, ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = VB == 8 ? e : nib_order(e);
                const uint32_t bw = k < 4 ? w0[k & 3] : w1[k & 3];
                ac[e] = kin[k] ? (__bf16)bf16_hi_to_f32(bw) : (__bf16)0.0f;
                ph[e] = hi_of(pp[k]);
                pl[e] = lo_of(pp[k]);
            }
            f32x4 c = corr;
            c = mfma_bf16(ac, ph, c);
            corr = mfma_bf16(ac, pl, c);
        }
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const u32x4 s0 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][gi][8 * lg]);
            const u32x4 s1 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][gi][8 * lg + 4]);
            bf16x8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = VB == 8 ? e : nib_order(e);
                const float sv = bf16_lo_to_f32(k < 4 ? s0[k & 3] : s1[k & 3]);
                const float w = full || p[k] >= 0.0f ? p[k] * sv : 0.0f;
                bh[e] = hi_of(w);
                bl[e] = lo_of(w);
            }
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const int dt = 4 * gi + dd;
                f16x8 a16;
                if constexpr (VB == 8) a16 = codes8x8_to_f16(vr.vc[dt]);
                else a16 = codes4x8_to_f16(vr.vc[dt]);
                bf16x8 a;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = (__bf16)(float)a16[e];     // codes <= 255: exact
                f32x4 o = O[dt];
                o = mfma_bf16(a, bh, o);
                O[dt] = mfma_bf16(a, bl, o);
            }
        }
    };

    // ---- PV of one step (its V words staged): O^T += V^T (P * s_v)^T per
    //      group; the bias term of all groups in one MFMA.  Per-row visibility
    //      is carried by p (< 0: hidden); kin: key inside the item's range, so
    //      its slot holds data (A side, where a row is a quantization group and
    //      not a query row).  WIDE: the step needs the bf16 operands.
    auto pv = [&](const VRegs<D, VB>& vr, int st, const float (&p)[8], auto full_tag, auto wide_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr bool WIDE = decltype(wide_tag)::value;
        bool kin[8];
        float pp[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int key = st + 8 * lg + k;
            kin[k] = FULL || (key >= j0 && key < j1);
            pp[k] = FULL ? p[k] : fmaxf(p[k], 0.0f);
        }
        if constexpr (WIDE) {
            pv_wide(vr, p, pp, kin, FULL);
            return;
        }
        {
            f16x8 pb, ac;
            // rows m < GPW of the bias operand carry group m's V biases (read for
            // every lane, then zeroed by a select rather than a branch)
            u32x4 w0 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg]);
            u32x4 w1 = *reinterpret_cast<const u32x4*>(&sm.vsb[wave][m < GPW ? m : 0][8 * lg + 4]);
            if (m >= GPW) { w0 = (u32x4)0; w1 = (u32x4)0; }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = VB == 8 ? e : nib_order(e);
                const uint32_t bw = k < 4 ? w0[k & 3] : w1[k & 3];
                pb[e] = (_Float16)pp[k];
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
                bs[e] = FULL || p[k] >= 0.0f ? (_Float16)(p[k] * sv) : (_Float16)0.0f;
            }
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const int dt = 4 * gi + dd;
                f16x8 a;
                if constexpr (VB == 8) a = codes8x8_to_f16(vr.vc[dt]);
                else a = codes4x8_to_f16(vr.vc[dt]);
                O[dt] = mfma_f16(a, bs, O[dt]);
            }
        }
    };

    auto is_full = [&](int st) { return st >= full_lo && st + kStep - 1 <= full_hi; };

    // Software pipeline over steps.  Step i runs, in one block of straight-line
    // code: the scores of step i (its partials met behind the last barrier) and
    // the softmax, QK of step i+1 (independent of them, so their LDS, MFMA and
    // VALU latencies overlap), PV of step i; then one barrier.  Which code runs
    // is chosen once per step: keys all visible or not (FULL), fp16 or bf16 PV
    // operands (WIDE).  K and V codes are loaded two steps ahead into ping-pong
    // register sets (no copies: a copy would wait for the load); a set is
    // refilled right after its last use, so the first two steps of both go out
    // with q and a two-step split waits for memory once.  Loads are issued
    // unconditionally with the step index clamped, so the wait counters stay
    // exact; past the end the last step is read again from L2.
    KRegs<D, KB> ka, kb;
    VRegs<D, VB> va, vb;
    // q and the first steps' codes go out together, before len[b] is known
    // (unconditional: a branch around loads would make every later wait a full one;
    // with no step the clamped index still names slots inside the cache)
    load_q();
    // Fused decode step: the last split of every item takes the step's token
    // (position len-1, which every split's key range leaves out).  Its K and V
    // rows go out with q, one 8-value chunk per thread (K: threads [0, CH),
    // V: [CH, 2CH)).
    constexpr int NT = 64 * NW, CH = D / 8;
    const bool tok = TOK == kTokFold && P.k_new != nullptr && s == S - 1;
    const bool tok_v = tid >= CH;
    const int tok_ch = tok_v ? tid - CH : tid;
    float4 tka = {0.f, 0.f, 0.f, 0.f}, tkb = tka;
    if (__builtin_expect(tok, 0) && tid < 2 * CH) {
        const float* src = as_global(tok_v ? P.v_new : P.k_new) + ((int64_t)bh * D + tok_ch * 8);
        tka = *reinterpret_cast<const float4*>(src);
        tkb = *reinterpret_cast<const float4*>(src + 4);
    }
    load_k(ka, 0);
    load_v(va, 0);
    load_k(kb, 1);
    load_v(vb, 1);
    const int len_act = min(max(__builtin_amdgcn_readfirstlane(len_lane), 0), P.max_len);
    if (len_act != P.max_len) {
        ranges(len_act);
        nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
        st0 = j0 & ~(kStep - 1);
        last = max(nsteps - 1, 0);
        if (nsteps > 0) {
            load_k(ka, 0);
            load_v(va, 0);
            load_k(kb, 1);
            load_v(vb, 1);
        }
    }
    // the token's slot, and (item of row tile 0: the writer) the words of its
    // 8-slot V block that hold this thread's columns, read now and merged below
    const int tok_slot = (max(len_act, 1) - 1) % R;
    const bool tok_writer = tok && rt == 0;
    constexpr int VPT = (D + NT - 1) / NT;          // V columns per thread
    uint32_t tok_vw[VPT];
    uint32_t* tok_vp = const_cast<uint32_t*>(as_global(P.v_codes)) +
                       (((int64_t)bh * (R / 8) + tok_slot / 8) * D) * VW + (VB == 8 ? (tok_slot & 7) >> 2 : 0);
#pragma unroll
    for (int j = 0; j < VPT; ++j) tok_vw[j] = 0u;
    if (__builtin_expect(tok_writer, 0)) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (tid + j * NT < D) tok_vw[j] = tok_vp[(tid + j * NT) * VW];
    }
    setup_q();

    // ---- The fused step's token: quantized with the append kernel's device
    //      code (the same codes bit for bit), written into the cache by the
    //      writer, its score taken here from the fp32 q and the dequantized key,
    //      and its dequantized values joined to this split's softmax after the
    //      last step.  The token's V block is merged and written while this split
    //      may be reading it: only the token's bits change, and the split masks
    //      that slot, so either order gives it the other slots' codes.
    float s_tok = 0.0f;
    if (__builtin_expect(tok, 0)) {
        static_assert(2 * CH <= NT, "one 8-value chunk per thread");
        static_assert((5 * D + 4 * 16 * NW) <= (int)sizeof(sm.spart), "token scratch fits the partial tiles");
        // scratch in the partial-score tiles, free until the first QK
        lds_f32* khat = (lds_f32*)(&sm.spart[0][0][0][0]);
        lds_u8* vq = reinterpret_cast<lds_u8*>(khat + D);
        lds_f32* wsum = khat + D + D / 4;           // [NW][16] per-wave partial scores
        lds_f32* tokv = (lds_f32*)(&sm.tokv[0]);
        // the cache arrays of a fused step are the caller's writable cache
        uint32_t* k_codes_w = const_cast<uint32_t*>(as_global(P.k_codes));
        uint32_t* k_sb_w = const_cast<uint32_t*>(as_global(P.k_sb));
        uint32_t* v_sb_w = const_cast<uint32_t*>(as_global(P.v_sb));
        if (tid < 2 * CH) {
            const float v[8] = {tka.x, tka.y, tka.z, tka.w, tkb.x, tkb.y, tkb.z, tkb.w};
            uint32_t q[8];
            float scale, bias;
            quantize_group8(v, tok_v ? (1 << VB) - 1 : (1 << KB) - 1, q, scale, bias);
            lds_f32* xh = tok_v ? tokv : khat;
#pragma unroll
            for (int e = 0; e < 8; ++e) xh[tok_ch * 8 + e] = (float)q[e] * scale + bias;
            if (tok_writer) {
                if ((tok_ch & 7) == 0)
                    (tok_v ? v_sb_w : k_sb_w)[((int64_t)bh * R + tok_slot) * G + tok_ch / 8] = sb_word(scale, bias);
                if (!tok_v) store_k_chunk(k_codes_w + ((int64_t)bh * R + tok_slot) * (D * KB / 32), tok_ch, KB, q);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vq[tok_ch * 8 + e] = (uint8_t)q[e];
                }
            }
        }
        __syncthreads();
        if (tok_writer) {                            // the token's bits of its V block
            const int t = tok_slot & 7;
            const int sh = VB == 4 ? 4 * t : 8 * (t & 3);
            const uint32_t mask = (VB == 4 ? 0xFu : 0xFFu) << sh;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int dv = tid + j * NT;
                if (dv < D) tok_vp[dv * VW] = (tok_vw[j] & ~mask) | ((uint32_t)vq[dv] << sh);
            }
        }
        // q . khat for the lane's row m: this wave's groups, then the waves in order
        float acc = 0.0f;
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int d0 = (g0 + gi) * 64 + lg * 16;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t u = qraw[gi][h][e];
                    acc += bf16_lo_to_f32(u) * khat[d0 + 8 * h + 2 * e] + bf16_hi_to_f32(u) * khat[d0 + 8 * h + 2 * e + 1];
                }
        }
        acc = sum_across_groups(acc);
        if (lg == 0) wsum[wave * 16 + m] = acc;
        __syncthreads();
        float sc = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sc += wsum[w * 16 + m];
        s_tok = sc * sl2e;
        __syncthreads();                             // the scratch is free again
    }

    // step i with a step after it: kq holds step i+1's K words, kl is refilled
    // with step i+2's, vr holds step i's V words and is refilled with step i+2's
    auto step = [&](int i, int par, const KRegs<D, KB>& kq, KRegs<D, KB>& kl, VRegs<D, VB>& vr, auto full_tag,
                    auto wide_tag) {
        const int st = st0 + i * kStep;
        stage_k(kq);
        stage_v(vr);
        sync_wave();
        load_k(kl, i + 2);
        float z[8], p[8];
        const float mt = scores(st, par, z, full_tag);
        rescale(mt);
        probs(z, p, full_tag);
        qk(kq, par ^ 1);
        pv(vr, st, p, full_tag, wide_tag);
        load_v(vr, i + 2);
        __syncthreads();
    };
    auto run_step = [&](int i, int par, const KRegs<D, KB>& kq, KRegs<D, KB>& kl, VRegs<D, VB>& vr) {
        const int st = st0 + i * kStep;
        const bool wide = is_wide(vr, st);
        if (is_full(st)) {
            if (wide) step(i, par, kq, kl, vr, std::true_type{}, std::true_type{});
            else step(i, par, kq, kl, vr, std::true_type{}, std::false_type{});
        } else {
            if (wide) step(i, par, kq, kl, vr, std::false_type{}, std::true_type{});
            else step(i, par, kq, kl, vr, std::false_type{}, std::false_type{});
        }
    };
    // the last step: its softmax and PV only
    auto last_step = [&](int i, int par, const VRegs<D, VB>& vr) {
        const int st = st0 + i * kStep;
        const bool wide = is_wide(vr, st);
        stage_v(vr);
        sync_wave();
        float z[8], p[8];
        auto tail = [&](auto full_tag) {
            const float mt = scores(st, par, z, full_tag);
            rescale(mt);
            probs(z, p, full_tag);
            if (wide) pv(vr, st, p, full_tag, std::true_type{});
            else pv(vr, st, p, full_tag, std::false_type{});
        };
        if (is_full(st)) tail(std::true_type{});
        else tail(std::false_type{});
    };

    if (nsteps > 0) {
        stage_k(ka);
        sync_wave();
        qk(ka, 0);
        __syncthreads();
    }
    for (int i = 0; i < nsteps; i += 2) {
        if (i + 1 >= nsteps) {
            last_step(i, 0, va);
            break;
        }
        run_step(i, 0, kb, ka, va);
        if (i + 2 >= nsteps) {
            last_step(i + 1, 1, vb);
            break;
        }
        run_step(i + 1, 1, ka, kb, vb);
    }

    // ---- fold the bias term into O: lane (m, lg) holds corr[group row 4*lg+i][query row m]
    float L = sum_across_groups(l_run);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const float c = __shfl(corr[gi & 3], m + 16 * (gi >> 2));
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) O[4 * gi + dd] += c;
    }
    const int dcol = 64 * g0 + 4 * lg;   // + 16 * dt + i
    if (__builtin_expect(tok, 0)) {      // the fused step's token joins the softmax last
        const float m_new = fmaxf(m_run, s_tok);
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float pt = __builtin_amdgcn_exp2f(s_tok - m_new);
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
            const f32x4 vh = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                (lds_f32*)(&sm.tokv[0]) + dcol + 16 * dt);
            O[dt] = O[dt] * alpha + pt * vh;
        }
        L = L * alpha + pt;
        m_run = m_new;
    }
    if (S == 1) {
        if (!row_ok) return;
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* orow = KVQ_LAYER_PTR(uint16_t, P.out, lay_lo, lay_hi, rm.layer) + ((((int64_t)b * P.Hq + rm.hq) * C + rm.qi) * D);
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
            const f32x4 o = O[dt] * inv;
            uint2 w;
            w.x = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
            w.y = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
            *reinterpret_cast<uint2*>(orow + dcol + 16 * dt) = w;
        }
        return;
    }
    if (!row_ok) return;
    const int64_t ib = (int64_t)bh * P.n_rt + rt;
    const int64_t prow = (ib * S + s) * kRowTile + m;
    float* po = as_global(P.part) + prow * D;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) *reinterpret_cast<f32x4*>(po + dcol + 16 * dt) = O[dt];
    if (wave == 0 && lg == 0) {
        float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
        pml[0] = m_run;
        pml[1] = L;
    }
}

__device__ __forceinline__ int find_desc(const AttnParams& P, int bid)
{
    int di = 0;
    while (di + 1 < P.n_desc && bid >= P.d[di + 1].item_begin) ++di;
    return di;
}

// ONE: a single descriptor, so every field sits at a constant offset and the
// kernel-argument loads issue together instead of after a descriptor search.
// TOK: the token path it is built with (the plain reads of a single descriptor
// run without one: no extra code, registers or LDS).
template <int D, int KB, int VB, bool ONE, int TOK>
__global__ __launch_bounds__(64 * Shape<D>::NW) void attn_kernel(AttnParams P)
{
    __shared__ AttnSmem<D, TOK == kTokFold> sm;
    const int bid = blockIdx.x;
    if constexpr (ONE) {
        attn_body<D, KB, VB, TOK>(P.d[0], bid, sm);
    } else {
        const int di = find_desc(P, bid);
        const AttnDesc& d = P.d[di];
        attn_body<D, KB, VB, TOK>(d, bid - d.item_begin, sm);
    }
}

}  // namespace kvq



// Chunked prefill over an affine group-quantized cache, gfx950: the codes are
// read and converted in registers by the attention kernel itself (no
// dequantized copy of the key band), on 32x32x16 fp16 MFMAs.
//
// What it computes (page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0
// diff, gemma4/model.ts: a prompt chunk's tokens are appended to the cache and
// its queries then attend the cache read -- causal inside the chunk, windowed
// on sliding layers): for query i of a chunk of C, at position p = len - C + i,
// softmax(scale * q . khat_j) over max(0, p-W+1, len-R) <= j <= p, times vhat_j,
// khat = code * scale + bias per 64-value group (page 78, gemma4-e4b.ts
// Gemma4Layer.kv).
//
// Work item: 32 query rows of one (sequence, KV head) (rows ordered query-major,
// row = query * Hq/Hkv + head, as everywhere in this library), and a split of
// their keys.  Eight waves, two per SIMD: NS = D/128 of them split head_dim (128
// columns, two 64-groups each; their partial scores meet in LDS once per step)
// and NKG = 8/NS key groups take alternate 32-key steps, merged through LDS at
// the end.  Per 32-key step a wave computes
//   S^T = K Q^T   (keys x rows) with the key rows of K loaded in the order
//                 pi(i) = 16*((i/4)%2) + 4*(i/8) + i%4, so that the MFMA result
//                 leaves lane l holding row l%32 and keys 16*(l/32) .. +15;
//   O^T += V^T P^T  (head_dim x rows), whose B operand is exactly those 16 keys:
//                 MFMA m takes keys 16h + 8m + 0..7 (h = l/32), one 8-slot V
//                 block per lane and head_dim element, so no data moves between
//                 the two products.
// Codes enter the MFMAs as exact fp16 values; the K scale of each group is applied
// to the group's partial score in fp32 and the K bias joins through one bf16 MFMA
// against the per-row group sums of q (split in three bf16 parts, as in the decode
// kernel); the V scale multiplies P per group and the V bias joins through one
// more MFMA per 16 keys.  q enters after a power of 2 per row and 128-column slice
// that puts its largest magnitude in [2^14, 2^15).  Online softmax in base 2 with
// a lazy rescale (the running max may trail by up to 2^8).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 4-bit codes (one word, element e at bits 4e) -> fp16 values 1024 + code, in
// the element order {0, 2, 4, 6, 1, 3, 5, 7}: the even nibbles are spread to
// bytes with one mask, the odd ones with a shift and a mask, and each fp16 pair is
// one byte permute against 0x64 high bytes.
__device__ __forceinline__ f16x8 qp_codes4_off(uint32_t w)
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t c = 0x64646464u;
    const u32x4 x = {__builtin_amdgcn_perm(c, lo, 0x04010400u), __builtin_amdgcn_perm(c, lo, 0x04030402u),
                     __builtin_amdgcn_perm(c, hi, 0x04010400u), __builtin_amdgcn_perm(c, hi, 0x04030402u)};
    return __builtin_bit_cast(f16x8, x);
}
__device__ __forceinline__ constexpr int qp_order4(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }
// Slot of code t (0..7) of a word in that order.
__device__ __forceinline__ constexpr int qp_slot4(int t) { return (t & 1) * 4 + (t >> 1); }

constexpr int kQpRows = kQprefillRows;      // query rows per work item
constexpr float kQpRescaleSlack = 8.0f;
constexpr int kQpSpinLimit = 1 << 20;      // polls of a partner's step count before giving up

constexpr int kQpWaves = 8;

template <int D>
struct QpShape {
    static constexpr int NS = D / 128;      // waves splitting head_dim
    static constexpr int NKG = kQpWaves / NS;  // key groups
    static constexpr int GW = 2;            // 64-groups per wave
    static constexpr int NDT = 4;           // 32-column tiles of O^T per wave
    static_assert(NS * 128 == D && NS * NKG == kQpWaves, "head_dim 256 or 512");
};

template <int D>
struct QpSmem {
    static constexpr int NS = QpShape<D>::NS, NKG = QpShape<D>::NKG;
    union {
        struct {
            float ks[kQpWaves][2][32];        // [wave][group][key]: K scales of the wave's current step
            _Float16 vs[kQpWaves][2][32];     // [wave][group][slot]: V scales (fp16, MFMA slot order)
            _Float16 vb[kQpWaves][2][32];     // [wave][group][slot]: V biases
            union {
                f32x4 spart[2][kQpWaves][4][64];  // partial S^T [step parity][wave][quad][lane]
                u32x4 qs[kQpRows][D / 8 + 1];     // before the loop: the item's q rows (16-byte
                                                  // chunks, one pad chunk per row)
            };
            f16x8 qf[NS][2][4][64];           // q operands [slice][group][part][lane]
            int done[kQpWaves];               // per wave: steps whose partial scores are in spart
        } loop;
        struct {
            f32x4 o[kQpWaves][QpShape<D>::NDT][4][64];  // every wave's O^T tiles
            float ml[kQpWaves][2][32];                 // and its (m, l) per row
        } merge;
    };
};

// Key of row i of the permuted K operand (see the header).
__device__ __forceinline__ int qp_key(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <int D, int KB, int VB>
__global__ __launch_bounds__(64 * kQpWaves) void qprefill_kernel(AttnParams Pp)
{
    using Sh = QpShape<D>;
    constexpr int NS = Sh::NS, NKG = Sh::NKG, NDT = Sh::NDT;
    constexpr int G = D / 64;                  // groups per key row
    constexpr int KW = D * KB / 32;            // K words per slot
    constexpr int VW = VB / 4;                 // V words per (block, element)
    __shared__ QpSmem<D> sm;
    const AttnDesc& P = Pp.d[0];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave: uniform (scalar)
    const int li = lane & 31, h = lane >> 5;
    const int ds = wave % NS, kg = wave / NS;  // head_dim slice, key group
    const int c0 = ds * 128;                   // first column of the slice
    const int gq0 = ds * 2;                    // first group of the slice

    const int idx = xcd_item(blockIdx.x, gridDim.x);
    const int S = P.S;
    const int n_rt32 = (P.n_rows + kQpRows - 1) / kQpRows;
    const int rt = idx % n_rt32;               // row items of one split side by side (one XCD's L2)
    const int s = (idx / n_rt32) % S;
    const int bh = idx / (S * n_rt32);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int R = P.R, W = P.W, C = P.C;

    int opaque_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    const int len_lane = as_global(P.len)[b + opaque_zero];

    // ---- rows of this item; this lane's row is li
    const int row0 = rt * kQpRows;
    const int last_row = min(row0 + kQpRows, P.n_rows) - 1;
    const int qi_lo = row0 / P.hpk, qi_hi = last_row / P.hpk;
    const int grow = row0 + li;
    const bool row_ok = grow < P.n_rows;
    const int qi = (row_ok ? grow : row0) / P.hpk;
    const int hq = hkv * P.hpk + (row_ok ? grow : row0) % P.hpk;

    int j0, j1, full_lo, full_hi, klo, khi;
    auto ranges = [&](int len) {
        int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
        lo = max(lo, max(0, len - R));
        const int hi = len - C + qi_hi;
        const int base = lo & ~(kStep - 1);
        j0 = max(lo, base + s * P.split_len);
        j1 = min(hi + 1, base + (s + 1) * P.split_len);
        full_lo = max(j0, W > 0 ? len - C + qi_hi - W + 1 : 0);
        full_hi = min(j1 - 1, len - C + qi_lo);
        const int p_row = len - C + qi;
        klo = max(j0, W > 0 ? p_row - W + 1 : 0);
        khi = min(j1 - 1, p_row);
        if (!row_ok) { klo = 1; khi = 0; }
    };
    ranges(P.max_len);

    // ---- q of the item's rows, loaded with a row's 16-byte chunks on consecutive
    //      lanes (rows past the last are zero); staged in LDS below
    constexpr int QCH = D / 8;                          // 16-byte chunks per row
    constexpr int QLD = kQpRows * QCH / (64 * kQpWaves);  // chunks per thread
    static_assert(QLD * 64 * kQpWaves == kQpRows * QCH, "q chunks per thread");
    u32x4 qld[QLD];
#pragma unroll
    for (int k = 0; k < QLD; ++k) {
        const int c = tid + 64 * kQpWaves * k;
        const int gr = row0 + c / QCH;
        qld[k] = (u32x4)0;
        if (gr < P.n_rows) {
            const int qk = gr / P.hpk, hk = hkv * P.hpk + gr % P.hpk;
            qld[k] = *reinterpret_cast<const u32x4*>(as_global(P.q[0]) + (((int64_t)b * P.Hq + hk) * C + qk) * D +
                                                     8 * (c % QCH));
        }
    }

    // ---- per-step register sets: K codes of this lane's key (32 columns of each
    //      of the slice's 2 groups), its K scale|bias words, V code words of this
    //      lane's element for blocks 2h, 2h+1 of each of the 4 column tiles, and the
    //      V scale|bias word this lane stages (key li, group h)
    using KCode = typename std::conditional<KB == 8, u32x4[2][2], u32x4[2][1]>::type;
    using VCode = typename std::conditional<VB == 8, u32x2[NDT][2], uint32_t[NDT][2]>::type;
    struct Regs {
        KCode kc;
        u32x2 ksb;
        VCode vc;
        uint32_t vsb;
    };
    const int64_t slot0 = (int64_t)bh * R;
    const uint32_t* kcodes = as_global(P.k_codes) + slot0 * KW;
    const uint32_t* ksbp = as_global(P.k_sb) + slot0 * G + gq0;
    const uint32_t* vsbp = as_global(P.v_sb) + slot0 * G + gq0;
    const uint32_t* vcodes = as_global(P.v_codes) + ((int64_t)bh * (R / 8) * D + c0 + li) * VW;
    const int my_key = qp_key(li);

    auto load = [&](Regs& r, int st) {
        const int st_mod = st % R;
        const int kslot = wrap_slot(st_mod + my_key, R);
        const uint32_t* krow = kcodes + (int64_t)kslot * KW;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int w0 = (c0 + 64 * g + 32 * h) * KB / 32;     // first word of the lane's 32 columns
            r.kc[g][0] = *reinterpret_cast<const u32x4*>(krow + w0);
            if constexpr (KB == 8) r.kc[g][1] = *reinterpret_cast<const u32x4*>(krow + w0 + 4);
        }
        r.ksb = *reinterpret_cast<const u32x2*>(ksbp + (int64_t)kslot * G);
        const int vslot = wrap_slot(st_mod + li, R);
        r.vsb = vsbp[(int64_t)vslot * G + h];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int blk = wrap_slot(st_mod + 8 * (2 * h + m), R) >> 3;
            const uint32_t* vb = vcodes + (int64_t)blk * D * VW;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                if constexpr (VB == 8) r.vc[dt][m] = *reinterpret_cast<const u32x2*>(vb + 32 * dt * VW);
                else r.vc[dt][m] = vb[32 * dt * VW];
            }
        }
    };

    // ---- steps of this key group: t = kg, kg + NKG, ...
    int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    int st0 = j0 & ~(kStep - 1);
    int n_my = nsteps > kg ? (nsteps - kg + NKG - 1) / NKG : 0;
    int n_all = (nsteps + NKG - 1) / NKG;      // loop trips, the same in every wave
    auto stp = [&](int i) { return st0 + (kg + NKG * min(i, max(n_my - 1, 0))) * kStep; };

    Regs ra, rb;
    load(ra, stp(0));
    load(rb, stp(1));
    const int len_act = min(max(__builtin_amdgcn_readfirstlane(len_lane), 0), P.max_len);
    if (len_act != P.max_len) {
        ranges(len_act);
        nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
        st0 = j0 & ~(kStep - 1);
        n_my = nsteps > kg ? (nsteps - kg + NKG - 1) / NKG : 0;
        n_all = (nsteps + NKG - 1) / NKG;
        if (nsteps > 0) {
            load(ra, stp(0));
            load(rb, stp(1));
        }
    }

    // ---- q of this row and slice from LDS: B operands of the 16 QK MFMAs (group g,
    //      part j: slot 8h+e holds column c0 + 64g + 32h + 8j + order(e)), and the
    //      group sums
#pragma unroll
    for (int k = 0; k < QLD; ++k) {
        const int c = tid + 64 * kQpWaves * k;
        sm.loop.qs[c / QCH][c % QCH] = qld[k];
    }
    __syncthreads();
    u32x4 qraw[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) qraw[g][j] = sm.loop.qs[li][(c0 + 64 * g + 32 * h + 8 * j) / 8];

    // q: power of 2 per row and slice, fp16 operands (to LDS), group sums in three
    // bf16 parts
    bf16x8 qb;
    float qinv;
    {
        float amax = 0.0f, gs[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 u = row_ok ? qraw[g][j] : (u32x4)0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_lo_to_f32(u[e]), hi = bf16_hi_to_f32(u[e]);
                    acc += lo + hi;
                    amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
                }
            }
            gs[g] = acc + __shfl_xor(acc, 32);
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const uint32_t ex = min(max((__float_as_uint(amax) >> 23) & 0xFFu, 15u), 254u);
        const float qmul = __uint_as_float((268u - ex) << 23);
        qinv = __uint_as_float((ex - 14u) << 23) * P.scale_log2e;   // and the softmax scale
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 u = row_ok ? qraw[g][j] : (u32x4)0;
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) { f[2 * e] = bf16_lo_to_f32(u[e]); f[2 * e + 1] = bf16_hi_to_f32(u[e]); }
                f16x8 qv;
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] = (_Float16)(f[KB == 8 ? e : qp_order4(e)] * qmul);
                if (kg == 0) sm.loop.qf[ds][g][j][lane] = qv;
            }
        // bias MFMA slots: combo c = term*6 + part*2 + g (term 0: b_g * Q_g part,
        // term 1: s_g * (-1024 Q_g part)), c < 12; slot 8h+e holds combo 8h+e
        // (the group sums carry the softmax scale, scale*log2(e), so the scores come
        // out of the bias MFMA already scaled)
        float parts[3][2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float gq = gs[g] * P.scale_log2e;
            const float q1 = __uint_as_float((uint32_t)f32_to_bf16_rne(gq) << 16);
            const float q2 = __uint_as_float((uint32_t)f32_to_bf16_rne(gq - q1) << 16);
            const float q3 = __uint_as_float((uint32_t)f32_to_bf16_rne(gq - q1 - q2) << 16);
            parts[0][g] = q1;
            parts[1][g] = q2;
            parts[2][g] = q3;
        }
        uint16_t hw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = 0.0f;
#pragma unroll
            for (int cc = 0; cc < 12; ++cc)
                if (cc == 8 * h + e) {
                    const int term = cc / 6, part = (cc / 2) % 3, g = cc % 2;
                    v = term == 0 ? parts[part][g] : -1024.0f * parts[part][g];
                }
            hw[e] = row_ok ? (uint16_t)(__float_as_uint(v) >> 16) : (uint16_t)0;
        }
        const u32x4 w = {hw[0] | ((uint32_t)hw[1] << 16), hw[2] | ((uint32_t)hw[3] << 16),
                         hw[4] | ((uint32_t)hw[5] << 16), hw[6] | ((uint32_t)hw[7] << 16)};
        qb = __builtin_bit_cast(bf16x8, w);
    }

    if (lane == 0) sm.loop.done[wave] = 0;
    __syncthreads();                           // the q operands are in LDS
    f32x16 O[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[dt] = (f32x16){};
    f32x16 corr = (f32x16){};
    float m_run = -INFINITY, l_run = 0.0f;

    // ---- one step: QK (partial over the slice), exchange within the key group,
    //      softmax, PV.  full: every key of the step is visible to every row (no masks)
    // The partial scores of a step meet only within a key group (its NS waves), so
    // the exchange waits on the group's waves alone: each wave publishes its count
    // of steps whose partials are in LDS and waits for its partners' counts to
    // reach the same step.  Key groups then drift apart, and the two waves on a
    // SIMD (different key groups) overlap one's MFMAs with the other's VALU work.
    // The partials are double-buffered (step parity): a wave overwrites its
    // buffer two steps later only after its partners published the step in
    // between, which they do after reading it.  Every wave of a group runs the
    // same steps (the step count depends on the group alone).
    // The wait is bounded (kQpSpinLimit polls of about 64 clocks, tens of
    // milliseconds): the partners reach every step of their group, so the bound
    // is never met; it only guarantees that every wave exits.
    auto exchange_wait = [&](int n) {
        if (lane == 0) __hip_atomic_store(&sm.loop.done[wave], n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int o = 1; o < NS; ++o) {
            const int w = kg * NS + (ds + o) % NS;
            for (int spin = 0; spin < kQpSpinLimit &&
                               __hip_atomic_load(&sm.loop.done[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < n;
                 ++spin)
                __builtin_amdgcn_s_sleep(1);
        }
    };
    auto step = [&](const Regs& r, int st, int i, bool active, bool full) {
        if (!active) return;                   // this key group has no step here (uniform per group)
        const int par = i & 1;
        // stage this step's K scales (fp32) and V scales and biases (fp16, in the
        // slot order of the PV operands; keys outside the item's range, which may
        // sit in slots no append wrote, as 0); lane (li, h) holds key qp_key(li)'s
        // K words and key li's V words of groups 2h, 2h+1
        sm.loop.ks[wave][h][my_key] = bf16_lo_to_f32(h ? r.ksb.y : r.ksb.x);
        {
            const int key = st + li;
            const bool kin = full || (key >= j0 && key < j1);
            const int pos = VB == 8 ? li : (li & ~7) | qp_slot4(li & 7);
            const uint32_t w = kin ? r.vsb : 0u;
            sm.loop.vs[wave][h][pos] = (_Float16)bf16_lo_to_f32(w);
            sm.loop.vb[wave][h][pos] = (_Float16)bf16_hi_to_f32(w);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // K codes against q per group, then the group's scale per key
        f32x16 xs = (f32x16){};
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            f16x8 a[4];
            if constexpr (KB == 8) {
                codes8x16_to_f16_off(r.kc[g][0], a[0], a[1]);
                codes8x16_to_f16_off(r.kc[g][1], a[2], a[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = qp_codes4_off(r.kc[g][0][j]);
            }
            f32x16 x = (f32x16){};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = mfma32_f16(a[j], sm.loop.qf[ds][g][j][lane], x);
            const float* ksg = &sm.loop.ks[wave][g][16 * h];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(ksg + 4 * v4);
#pragma unroll
                for (int i = 0; i < 4; ++i) xs[4 * v4 + i] += sv[i] * x[4 * v4 + i];
            }
        }
        // undo q's power of 2 (times the softmax scale), then the K bias: A slot 8h+e holds combo 8h+e (term 0:
        // b_g, term 1: s_g; g = combo % 2) of this lane's key, group pairs from byte
        // permutes (the codes entered as 1024 + code: term 1 cancels that)
#pragma unroll
        for (int v = 0; v < 16; ++v) xs[v] *= qinv;
        f32x16 z;
        {
            const uint32_t bp = __builtin_amdgcn_perm(r.ksb.y, r.ksb.x, 0x07060302u);
            const uint32_t sp = __builtin_amdgcn_perm(r.ksb.y, r.ksb.x, 0x05040100u);
            const u32x4 a = {h ? sp : bp, h ? sp : bp, h ? 0u : bp, h ? 0u : sp};
            z = mfma32_bf16(__builtin_bit_cast(bf16x8, a), qb, xs);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            sm.loop.spart[par][wave][q4][lane] = (f32x4){z[4 * q4], z[4 * q4 + 1], z[4 * q4 + 2], z[4 * q4 + 3]};
        exchange_wait(i + 1);
#pragma unroll
        for (int o = 1; o < NS; ++o)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 t = sm.loop.spart[par][kg * NS + (ds + o) % NS][q4][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) z[4 * q4 + i] += t[i];
            }

        // softmax over this lane's 16 keys st + 16h + v for row li
        if (!full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = st + 16 * h + v;
                z[v] = (key >= klo && key <= khi) ? z[v] : -INFINITY;
            }
        }
        float mloc = z[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mloc = fmaxf(mloc, z[v]);
        const float mt = fmaxf(mloc, __shfl_xor(mloc, 32));
        if (__any(mt > m_run + kQpRescaleSlack)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
            corr *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            p[v] = __builtin_amdgcn_exp2f(z[v] - m_use);      // masked keys: exactly 0
            l_run += p[v];
        }

        // PV: MFMA m takes keys 16h + 8m + order(e); P times the fp16 V scale of each
        // group, and the V biases of the 4 groups (A rows 0..3) through one MFMA per m
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (_Float16)p[8 * m + (VB == 8 ? e : qp_order4(e))];
            const int ga = li < 2 ? li : 0;
            f16x8 ab = *reinterpret_cast<const f16x8*>(&sm.loop.vb[wave][ga][16 * h + 8 * m]);
            if (li >= 2) ab = (f16x8){};
            corr = mfma32_f16(ab, pb, corr);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const f16x8 sv = *reinterpret_cast<const f16x8*>(&sm.loop.vs[wave][g][16 * h + 8 * m]);
                const f16x8 bs = pb * sv;
#pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
                    const int dt = 2 * g + dd;
                    f16x8 a;
                    if constexpr (VB == 8) a = codes8x8_to_f16(r.vc[dt][m]);
                    else a = qp_codes4_off(r.vc[dt][m]) - (f16x8)(_Float16)1024.0f;
                    O[dt] = mfma32_f16(a, bs, O[dt]);
                }
            }
        }
    };

    auto is_full = [&](int st) { return st >= full_lo && st + kStep - 1 <= full_hi; };
    auto do_step = [&](const Regs& r, int i) {
        const int st = stp(i);
        step(r, st, i, i < n_my, is_full(st));
    };
    for (int i = 0; i < n_all; i += 2) {
        do_step(ra, i);
        load(ra, stp(i + 2));
        if (i + 1 >= n_all) break;
        do_step(rb, i + 1);
        load(rb, stp(i + 3));
    }

    // ---- fold the V bias term into O: corr row g (lanes h = 0, v = g) per group
    {
        float cg[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) cg[g] = __shfl(corr[g], li);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) O[dt] += cg[dt / 2];
    }
    float L = l_run + __shfl_xor(l_run, 32);

    // ---- merge the key groups: every wave leaves (O, m, l) in LDS; wave (kg, ds)
    //      then merges column tiles kg*TPW .. kg*TPW+TPW-1 of slice ds over the
    //      groups and writes them
    constexpr int TPW = NDT / NKG;
    static_assert(TPW * NKG == NDT, "column tiles per wave");
    __syncthreads();                           // the loop's LDS is free
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            sm.merge.o[wave][dt][q4][lane] = (f32x4){O[dt][4 * q4], O[dt][4 * q4 + 1], O[dt][4 * q4 + 2],
                                                     O[dt][4 * q4 + 3]};
    if (h == 0) {
        sm.merge.ml[wave][0][li] = m_run;
        sm.merge.ml[wave][1][li] = L;
    }
    __syncthreads();
    float mk[NKG], wk[NKG];
    float mx = -INFINITY;
#pragma unroll
    for (int k1 = 0; k1 < NKG; ++k1) {
        mk[k1] = sm.merge.ml[k1 * NS + ds][0][li];
        mx = fmaxf(mx, mk[k1]);
    }
    float Lm = 0.0f;
#pragma unroll
    for (int k1 = 0; k1 < NKG; ++k1) {
        wk[k1] = mk[k1] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk[k1] - mx);   // empty groups: 0
        Lm += wk[k1] * sm.merge.ml[k1 * NS + ds][1][li];
    }
    f32x16 Om[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        Om[t] = (f32x16){};
#pragma unroll
        for (int k1 = 0; k1 < NKG; ++k1)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 v = sm.merge.o[k1 * NS + ds][kg * TPW + t][q4][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) Om[t][4 * q4 + i] += wk[k1] * v[i];
            }
    }
    if (!row_ok) return;

    // ---- write: lane (li, h) holds columns c0 + 32 dt + 8 (v/4) + 4h + v%4 of row li
    if (S == 1) {
        const float inv = Lm > 0.0f ? 1.0f / Lm : 0.0f;
        uint16_t* orow = as_global(P.out[0]) + (((int64_t)b * P.Hq + hq) * C + qi) * D + c0 + 4 * h;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16& o = Om[t];
                uint2 w;
                w.x = f32_to_bf16_rne(o[4 * q4] * inv) | ((uint32_t)f32_to_bf16_rne(o[4 * q4 + 1] * inv) << 16);
                w.y = f32_to_bf16_rne(o[4 * q4 + 2] * inv) | ((uint32_t)f32_to_bf16_rne(o[4 * q4 + 3] * inv) << 16);
                *reinterpret_cast<uint2*>(orow + 32 * (kg * TPW + t) + 8 * q4) = w;
            }
        return;
    }
    // split partials in the combine kernel's 16-row layout
    const int rt16 = 2 * rt + (li >> 4), r16 = li & 15;
    const int64_t prow = (((int64_t)bh * P.n_rt + rt16) * S + s) * kRowTile + r16;
    float* po = as_global(P.part) + prow * D + c0 + 4 * h;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(po + 32 * (kg * TPW + t) + 8 * q4) =
                (f32x4){Om[t][4 * q4], Om[t][4 * q4 + 1], Om[t][4 * q4 + 2], Om[t][4 * q4 + 3]};
    if (wave == 0 && h == 0) {
        float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
        pml[0] = mx;
        pml[1] = Lm;
    }
}

hipError_t launch_qprefill(const AttnParams& p, int total_items, hipStream_t stream)
{
    const dim3 grid(total_items), block(64 * kQpWaves);
    switch (p.d[0].cfg) {
#define KVQ_QP(D_, KB_, VB_) \
    case cfg_of(D_, KB_, VB_): return launch_read(qprefill_kernel<D_, KB_, VB_>, grid, block, p, stream);
    KVQ_QP(256, 4, 4) KVQ_QP(256, 4, 8) KVQ_QP(256, 8, 4) KVQ_QP(256, 8, 8)
    KVQ_QP(512, 4, 4) KVQ_QP(512, 4, 8) KVQ_QP(512, 8, 4) KVQ_QP(512, 8, 8)
#undef KVQ_QP
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq

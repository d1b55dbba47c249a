// Attention of a short chunk (a speculative-verify window: a few queries per
// sequence, up to 64 query rows per KV head) straight from the quantized cache,
// gfx950.  What it computes is the chunked-prefill read (page 80 of the
// @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff, gemma4/model.ts: the chunk's
// tokens are appended, then its queries attend the read -- causal inside the
// chunk, windowed on sliding layers): for query i of a chunk of C, at position
// p = len - C + i, softmax(scale * q . khat_j) over max(0, p-W+1, len-R) <= j
// <= p, times vhat_j.
//
// One workgroup holds all the rows of its (sequence, KV head), so every key is
// read from HBM once per split; each 32-key step is dequantized into LDS once
// and read by every wave (4 row tiles of 16 rows):
//   * all threads dequantize the step's K (token-major) and V (d-major) to
//     fp16, x = code * scale + bias in one packed fp16 FMA per value pair;
//   * each wave runs S^T = Khat Q^T and O^T = Vhat^T P^T on 16x16x32 fp16 MFMA
//     from LDS, with the online softmax (base 2, lazy rescale).  For D = 512 two
//     waves share a row tile, each accumulating half of head_dim: both compute
//     the tile's full scores (the same instructions on the same data, so the
//     same softmax state), which keeps a wave's accumulators, q and in-flight
//     codes within 256 registers and puts two waves on each SIMD.
// Codes and scale|bias words are fetched two and three steps ahead; LDS holds
// two steps; one barrier per step.  Rows follow the decode layout
// (row = query * (Hq/Hkv) + head), so split partials go through the decode
// combine kernel (as o / l in fp16: this kernel's V values are fp16 already).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kCpTiles = 4;                    // 16-row tiles per workgroup
constexpr int kCpRows = kCpTiles * kRowTile;   // query rows per workgroup (kCodesPrefillRows)
static_assert(kCpRows == kCodesPrefillRows, "host and kernel agree on the row block");

template <int D>
struct CpShape {
    static constexpr int DH = D == 512 ? 2 : 1;   // waves per row tile (head_dim parts)
    static constexpr int NW = kCpTiles * DH;      // waves per workgroup
    static constexpr int NT = 64 * NW;            // threads
    static constexpr int DW = D / DH;             // output columns of one wave
    static constexpr int KCH = NT / kStep;        // K dequant: threads per key
    static constexpr int CH = D / KCH;            // K values per thread
    static constexpr int VD = D / NT;             // V dequant: head_dim columns per thread
    static_assert(CH % 32 == 0 && CH <= 64 && VD >= 1 && NT * VD == D, "dequant assignment");
};
constexpr float kCpRescaleSlack = 8.0f;

template <int D>
struct __attribute__((aligned(16))) CpSmem {
    static constexpr int G = D / 64;
    // K rows of a step in MFMA order: LDS row 16*t + r holds key 8*(r/4) + 4*t + r%4,
    // so the 16 rows one MFMA tile reads are consecutive; the row stride is
    // 4 dwords past a multiple of 64 banks, so those 16 reads hit distinct banks.
    _Float16 kh[2][kStep][D + 8];
    // V^T rows: vt[d][8*blk + e] holds key 8*blk + (e for 8-bit V, nibble order
    // {0,4,1,5,2,6,3,7} for 4-bit V); 80-byte stride, conflict-free 16-lane reads.
    _Float16 vt[2][D][kStep + 8];
    uint16_t ks[2][G][kStep], kb[2][G][kStep];   // fp16 K scale / bias, natural key order
    uint16_t vs[2][G][kStep], vb[2][G][kStep];   // fp16 V scale / bias, V^T element order
};

template <int D, int KB, int VB>
struct CpCodes {
    // K: thread -> (key t/KCH, head_dim chunk t%KCH of CH values); V: thread -> d (+ NT, ...)
    static constexpr int KWT = CpShape<D>::CH * KB / 32;  // K words per thread
    static constexpr int VD = CpShape<D>::VD;             // head_dim columns per thread
    static constexpr int VWT = VD * 4 * (VB / 4);         // V words per thread (4 blocks of 8 keys)
    uint32_t k[KWT];
    uint32_t v[VWT];
};

__device__ __forceinline__ uint16_t cp_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

template <int I, int N, class F>
__device__ __forceinline__ void cp_static_for(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        cp_static_for<I + 1, N>(f);
    }
}

// Register sets of in-flight step loads (NSET - 1 steps ahead of their use).
template <int D, int KB, int VB>
constexpr int cp_nset() { return D == 512 ? 3 : 4; }

template <int D, int KB, int VB>
__device__ __forceinline__ void codes_body(const AttnDesc& P, int idx, CpSmem<D>& sm)
{
    using Sh = CpShape<D>;
    constexpr int NSET = cp_nset<D, KB, VB>();
    constexpr int G = D / 64, KS = D / 32, NT = Sh::NT;
    constexpr int DT = Sh::DW / 16;      // 16-column output tiles of this wave
    constexpr int KW = D * KB / 32;      // K words per slot
    constexpr int VW = VB / 4;           // V words per (block, d)
    using Codes = CpCodes<D, KB, VB>;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;
    const int wtile = wave % kCpTiles;           // row tile of this wave
    const int dh = wave / kCpTiles;              // head_dim part of this wave
    const int dcol0 = dh * Sh::DW;               // its first output column

    // ---- work item: (b, kv head, 64-row block, split)
    const int S = P.S;
    const int n_rb = (P.n_rt + kCpTiles - 1) / kCpTiles;
    const int s = idx % S;
    const int rb = (idx / S) % n_rb;
    const int bh = idx / (S * n_rb);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int len = min(max(__builtin_amdgcn_readfirstlane(as_global(P.len)[b]), 0), P.max_len);
    const int R = P.R, W = P.W, C = P.C, hpk = P.hpk;

    const int row0 = rb * kCpRows;
    const int last_row = min(row0 + kCpRows, P.n_rows) - 1;
    const int qi_lo = row0 / hpk, qi_hi = last_row / hpk;
    int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
    lo = max(lo, max(0, len - R));
    const int hi = len - C + qi_hi;
    const int base = lo & ~(kStep - 1);
    const int j0 = max(lo, base + s * P.split_len);
    const int j1 = min(hi + 1, base + (s + 1) * P.split_len);
    const int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    const int st0 = j0 & ~(kStep - 1);

    // ---- this wave's 16 rows and this lane's row
    const int rt = rb * kCpTiles + wtile;                 // 16-row tile index
    const int wrow0 = rt * kRowTile;
    const bool wave_on = wrow0 < P.n_rows;
    const int wlast = min(wrow0 + kRowTile, P.n_rows) - 1;
    const int grow = wrow0 + m;
    const bool row_ok = grow < P.n_rows;
    const int qi = (row_ok ? grow : wrow0) / hpk;
    const int hq = hkv * hpk + (row_ok ? grow : wrow0) % hpk;
    const int p_row = len - C + qi;
    int klo = max(j0, W > 0 ? p_row - W + 1 : 0);
    int khi = min(j1 - 1, p_row);
    if (!row_ok) { klo = 1; khi = 0; }
    // keys every row of this wave sees
    const int full_lo = max(j0, W > 0 ? len - C + (wave_on ? wlast : wrow0) / hpk - W + 1 : 0);
    const int full_hi = min(j1 - 1, len - C + wrow0 / hpk);

    const int64_t kslot0 = (int64_t)bh * R;
    const uint32_t* __restrict__ kcodes = as_global(P.k_codes) + kslot0 * KW;
    const uint32_t* __restrict__ vcodes = as_global(P.v_codes) + (int64_t)bh * (R / 8) * D * VW;

    // ---- loads of one step into registers
    // K dequant assignment: lane l of a 32-lane half writes LDS row l (MFMA order,
    // below), i.e. key 8*((l/4)%4) + 4*(l/16) + l%4, chunk tid/32: the 16 lanes of
    // one LDS write pass write 16 consecutive rows, whose 4-bank row offsets keep
    // them on distinct banks
    const int k_row = tid & 31;
    const int k_key = (((k_row >> 2) & 3) << 3) | (((k_row >> 4) & 1) << 2) | (k_row & 3);
    const int k_chunk = tid >> 5;
    static_assert(Sh::KCH * kStep == NT, "one K chunk per thread");
    auto load_codes = [&](Codes& c, int st) {
        const int st_mod = st % R;
        const uint32_t* krow = kcodes + wrap_slot(st_mod + k_key, R) * KW + k_chunk * Codes::KWT;
#pragma unroll
        for (int w = 0; w < Codes::KWT; w += 4) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(krow + w);
            c.k[w] = x.x; c.k[w + 1] = x.y; c.k[w + 2] = x.z; c.k[w + 3] = x.w;
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int vblk = wrap_slot(st_mod + 8 * blk, R) >> 3;
#pragma unroll
            for (int dd = 0; dd < Codes::VD; ++dd) {
                const uint32_t* vw = vcodes + ((int64_t)vblk * D + tid + NT * dd) * VW;
                if constexpr (VB == 8) {
                    const u32x2 x = *reinterpret_cast<const u32x2*>(vw);
                    c.v[(dd * 4 + blk) * 2] = x.x;
                    c.v[(dd * 4 + blk) * 2 + 1] = x.y;
                } else {
                    c.v[dd * 4 + blk] = vw[0];
                }
            }
        }
    };
    // scale|bias words: thread t stages K word t and V word t of the step (32*G each)
    constexpr int NSB = kStep * G;
    const int sb_key = tid % kStep, sb_g = tid / kStep;
    auto load_sb = [&](uint32_t (&w)[2], int st) {
        const int o = NSB >= NT || tid < NSB ? (int)(wrap_slot(st % R + sb_key, R) * G + (sb_g % G)) : 0;
        w[0] = as_global(P.k_sb)[kslot0 * G + o];
        w[1] = as_global(P.v_sb)[kslot0 * G + o];
    };
    // Positions at or past len (the tail of the last step) may sit in slots no
    // append wrote, whose words can be anything (NaN included); their scale and
    // bias are staged as 0, so they dequantize to 0 and a zero weight cannot
    // meet a NaN value.
    auto stage_sb = [&](const uint32_t (&w_in)[2], int slot, int st) {
        if (NSB >= NT || tid < NSB) {
            const int g = sb_g % G, key = sb_key;
            const bool held = st + key < len;
            const uint32_t w[2] = {held ? w_in[0] : 0u, held ? w_in[1] : 0u};
            // V scale/bias go to the V^T element position of the key
            const int j = key & 7;
            const int pos = (key & ~7) + (VB == 8 ? j : (j < 4 ? 2 * j : 2 * (j - 4) + 1));
            sm.ks[slot][g][key] = cp_f16_bits(bf16_lo_to_f32(w[0]));
            sm.kb[slot][g][key] = cp_f16_bits(bf16_hi_to_f32(w[0]));
            sm.vs[slot][g][pos] = cp_f16_bits(bf16_lo_to_f32(w[1]));
            sm.vb[slot][g][pos] = cp_f16_bits(bf16_hi_to_f32(w[1]));
        }
    };
    // ---- dequantize one step into LDS buffer `slot`
    auto dequant = [&](const Codes& c, int slot) {
        {   // K: 8 values per code word (4-bit) / 4 (8-bit), one group per thread
            const int g = (k_chunk * Sh::CH) / 64;
            const uint32_t sw = sm.ks[slot][g][k_key], bw = sm.kb[slot][g][k_key];
            const f16x2 s2 = __builtin_bit_cast(f16x2, sw | (sw << 16));
            const f16x2 b2 = __builtin_bit_cast(f16x2, bw | (bw << 16));
            _Float16* dst = &sm.kh[slot][k_row][k_chunk * Sh::CH];   // row k_row holds key k_key
#pragma unroll
            for (int w = 0; w < Codes::KWT; w += (KB == 8 ? 2 : 1)) {
                f16x2 pr[4];
                if constexpr (KB == 8) {
                    pr[0] = u8pair_to_f16x2(c.k[w], 0x04010400u);
                    pr[1] = u8pair_to_f16x2(c.k[w], 0x04030402u);
                    pr[2] = u8pair_to_f16x2(c.k[w + 1], 0x04010400u);
                    pr[3] = u8pair_to_f16x2(c.k[w + 1], 0x04030402u);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = u4pair_to_f16x2(c.k[w], i);
                }
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(pr[i], s2, b2));
                *reinterpret_cast<u32x4*>(dst + (KB == 8 ? w * 4 : w * 8)) = o;
            }
        }
#pragma unroll
        for (int dd = 0; dd < Codes::VD; ++dd) {   // V: this thread's column d, 32 keys
            const int d = tid + NT * dd;
            const int g = d / 64;
            _Float16* dst = &sm.vt[slot][d][0];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                f16x2 pr[4];
                if constexpr (VB == 8) {
                    const uint32_t w0 = c.v[(dd * 4 + blk) * 2], w1 = c.v[(dd * 4 + blk) * 2 + 1];
                    pr[0] = u8pair_to_f16x2(w0, 0x04010400u);
                    pr[1] = u8pair_to_f16x2(w0, 0x04030402u);
                    pr[2] = u8pair_to_f16x2(w1, 0x04010400u);
                    pr[3] = u8pair_to_f16x2(w1, 0x04030402u);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = u4pair_to_f16x2(c.v[dd * 4 + blk], i);
                }
                const u32x4 s4 = *reinterpret_cast<const u32x4*>(&sm.vs[slot][g][8 * blk]);
                const u32x4 b4 = *reinterpret_cast<const u32x4*>(&sm.vb[slot][g][8 * blk]);
                u32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // element to a scalar first: bit_cast of a vector element expression
                    // reads element 0 in this compiler
                    const uint32_t sw = s4[i], bw = b4[i];
                    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                        pr[i], __builtin_bit_cast(f16x2, sw), __builtin_bit_cast(f16x2, bw)));
                }
                *reinterpret_cast<u32x4*>(dst + 8 * blk) = o;
            }
        }
    };

    // ---- q of this lane's row as MFMA B operands, in the K element order
    // The row enters the MFMA as fp16 after a power of 2 that puts its largest
    // magnitude in [2^14, 2^15) (bf16 -> fp16 exact for every value within 2^-28
    // of it, at any magnitude of q); the scores are multiplied back by qinv.
    f16x8 qf[KS];
    float qinv;
    {
        const uint16_t* qrow = as_global(P.q[0]) + ((((int64_t)b * P.Hq + hq) * C + qi) * D);
        u32x4 u[KS];
        float amax = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u[ks] = 0;
            if (row_ok) u[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_lo_to_f32(u[ks][e])), fabsf(bf16_hi_to_f32(u[ks][e]))));
        }
        const uint32_t ex = min(max((__float_as_uint(max_across_groups(amax)) >> 23) & 0xFFu, 15u), 254u);
        const float qmul = __uint_as_float((268u - ex) << 23);
        qinv = __uint_as_float((ex - 14u) << 23);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { f[2 * e] = bf16_lo_to_f32(u[ks][e]); f[2 * e + 1] = bf16_hi_to_f32(u[ks][e]); }
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (_Float16)(f[KB == 8 ? e : nib_order(e)] * qmul);
        }
    }

    const float sl2e = P.scale_log2e * qinv;
    f32x4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // ---- one step of this wave's rows from LDS buffer `slot`
    auto compute = [&](int st, int slot, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        float z[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 sacc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = *reinterpret_cast<const f16x8*>(&sm.kh[slot][16 * t + m][32 * ks + 8 * lg]);
                sacc = mfma_f16(a, qf[ks], sacc);
            }
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
        const float mt = max_across_groups(mloc);
        if (__any(mt > m_run + kCpRescaleSlack)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { p[k] = __builtin_amdgcn_exp2f(z[k] - m_use); l_run += p[k]; }
        f16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (_Float16)p[VB == 8 ? e : nib_order(e)];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(&sm.vt[slot][dcol0 + 16 * dt + m][8 * lg]);
            O[dt] = mfma_f16(a, pb, O[dt]);
        }
    };
    auto do_compute = [&](int st, int slot) {
        if (!wave_on) return;
        if (st >= full_lo && st + kStep - 1 <= full_hi) compute(st, slot, std::true_type{});
        else compute(st, slot, std::false_type{});
    };

    // ---- pipeline over steps h = 0 .. nsteps-1, one barrier per step.  At step h:
    //      issue the codes of step h+NSET and the scale|bias words of step
    //      h+NSET+1, stage the scale|bias of step h+2 into LDS, dequantize step
    //      h+1 and run the MFMAs of step h.  Every register set is consumed
    //      NSET-1 steps after its loads were issued, so NSET-1 steps of loads
    //      are in flight; loads are unconditional with the step index clamped.
    //      Register sets rotate with h % NSET (compile-time indices), LDS
    //      buffers with h & 1.
    const int last = max(nsteps - 1, 0);
    auto stp = [&](int i) { return st0 + min(i, last) * kStep; };
    Codes cs[NSET];
    uint32_t sbs[NSET][2];
    if (nsteps > 0) {
        uint32_t s0[2];
        load_sb(s0, stp(0));
        cp_static_for<0, NSET>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            load_codes(cs[r], stp(r));
            load_sb(sbs[(r + 1) % NSET], stp(r + 1));
        });
        stage_sb(s0, 0, stp(0));
        stage_sb(sbs[1], 1, stp(1));
        __syncthreads();
        dequant(cs[0], 0);
        __syncthreads();
    }
    for (int h0 = 0; h0 < nsteps; h0 += NSET) {
        cp_static_for<0, NSET>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int h = h0 + r;
            if (h >= nsteps) return;
            const int slot = h & 1;
            load_codes(cs[r], stp(h + NSET));
            load_sb(sbs[(r + 1) % NSET], stp(h + NSET + 1));
            stage_sb(sbs[(r + 2) % NSET], slot, stp(h + 2));
            if (h + 1 < nsteps) dequant(cs[(r + 1) % NSET], slot ^ 1);
            do_compute(st0 + h * kStep, slot);
            __syncthreads();
        });
    }

    // ---- write this wave's rows
    if (!wave_on || !row_ok) return;
    const float L = sum_across_groups(l_run);
    const int dcol = dcol0 + 4 * lg;
    if (S == 1) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* orow = as_global(P.out[0]) + ((((int64_t)b * P.Hq + hq) * C + qi) * D);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = O[dt] * inv;
            uint2 w;
            w.x = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
            w.y = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
            *reinterpret_cast<uint2*>(orow + dcol + 16 * dt) = w;
        }
    } else {
        // o / l as fp16 (part_h): a convex combination of this kernel's fp16 V values
        const int64_t ib = (int64_t)bh * P.n_rt + rt;
        const int64_t prow = (ib * S + s) * kRowTile + m;
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* po = reinterpret_cast<uint16_t*>(as_global(P.part)) + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = O[dt] * inv;
            const f16x2 lo = {(_Float16)o[0], (_Float16)o[1]}, hi = {(_Float16)o[2], (_Float16)o[3]};
            *reinterpret_cast<uint2*>(po + dcol + 16 * dt) =
                (uint2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
        if (lg == 0 && dh == 0) {
            float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
            pml[0] = m_run;
            pml[1] = L;
        }
    }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(CpShape<D>::NT) void codes_prefill_kernel(AttnParams P)
{
    __shared__ CpSmem<D> sm;
    codes_body<D, KB, VB>(P.d[0], blockIdx.x, sm);
}

hipError_t launch_prefill_codes(const AttnParams& p, int total_items, hipStream_t stream)
{
    const dim3 grid(total_items);
    switch (p.d[0].cfg) {
#define KVQ_CP(D_, KB_, VB_) \
    case cfg_of(D_, KB_, VB_): \
        return launch_read(codes_prefill_kernel<D_, KB_, VB_>, grid, dim3(CpShape<D_>::NT), p, stream);
    KVQ_CP(256, 4, 4) KVQ_CP(256, 4, 8) KVQ_CP(256, 8, 4) KVQ_CP(256, 8, 8)
    KVQ_CP(512, 4, 4) KVQ_CP(512, 4, 8) KVQ_CP(512, 8, 4) KVQ_CP(512, 8, 8)
#undef KVQ_CP
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq

// Chunked-prefill attention over an unquantized bf16 cache (the pages' bf16
// sliding layers), gfx950.  Quantized caches have their own prefill kernel
// (prefill_q.hip), which reads the codes in place.
//
// What it computes (page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0
// diff, gemma4/model.ts: a prompt chunk's tokens are appended to the cache and
// its queries then attend the cache read -- causal inside the chunk, windowed
// on sliding layers): for query i of a chunk of C, at position p = len - C + i,
// softmax(scale * q . k_j) over max(0, p-W+1, len-R) <= j <= p, times v_j.
//
//   prefill_kernel: one workgroup per (sequence, KV head, 32 query rows,
//     split).  Each 32-key step's tiles -- its 32 K rows (in MFMA row order),
//     then its D V^T rows (keys contiguous per element), 16-byte chunks
//     XOR-swizzled so the MFMA operand reads hit distinct banks -- are copied
//     global -> LDS with LDS DMA (no register staging) one round ahead of
//     their use, every lane addressing its own 16-byte chunk of the cache, and
//     the V^T entries of positions outside the band [base0, len) (base0 = the
//     lowest position any query of the chunk sees, rounded down to 32), which a
//     ring slot or a never-written slot may fill with anything, are zeroed.
//     Each wave owns RT row tiles of 16 rows, so every K / V^T operand read
//     from LDS feeds RT MFMAs; the NG wave groups take alternate steps and
//     merge in LDS at the end.  S^T = K Q^T and O^T = V^T P^T run on 16x16x32
//     bf16 MFMA with an online softmax in base 2 (lazy rescale: the running
//     max may trail the true one by up to 2^8).
//   band_bf16_kernel: the same tiles as a copy in the workspace, for caches
//     too large for the DMA's 32-bit offsets; prefill_kernel then reads them.
// Rows follow the decode layout (row = query * (Hq/Hkv) + head), so split
// partials, if any, go through the same combine kernel.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kPfWaves = 2;                    // row tiles per workgroup
constexpr int kPfRows = kPfWaves * kRowTile;   // query rows per workgroup
constexpr float kPfRescaleSlack = 8.0f;
// Band tiles kept per (sequence, KV head): the band's steps plus kBandPad more,
// so a round past the last step may copy past the band without a bounds check
// (those tiles are never computed on).
constexpr int kBandPad = 4;

// Lowest position any query of the chunk sees; the band starts there rounded
// down to a step.  The two kernels and the host sizing agree on this.
__device__ __forceinline__ int band_lo(int len, int C, int W, int R)
{
    const int lo = W > 0 ? len - C - W + 1 : 0;
    return max(lo, max(0, len - R));
}

// Two fp32 values to a bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Tile image of one 32-key step, in 16-byte chunks (8 bf16): the K part, 32 rows
// of D/8 chunks in MFMA row order (k_row), chunk c of a row's elements stored at
// position c ^ (row % 16); then the V^T part, D rows of 4 chunks (keys 8c ..
// 8c+7), chunk c of row d stored at position c ^ ((d / 4) % 4).
// MFMA reads of 16 rows at one logical chunk then touch 16 distinct chunk
// positions modulo 16, i.e. distinct banks.
template <int D> constexpr int tile_elems() { return 64 * D; }     // bf16 per step tile
// LDS row of key k within a step (row 16*t + r holds key 8*(r/4) + 4*t + r%4)
__device__ __forceinline__ int k_row(int key) { return 16 * ((key >> 2) & 1) + 4 * (key >> 3) + (key & 3); }
template <int D>
__device__ __forceinline__ int k_chunk_pos(int row, int c) { return row * (D / 8) + (c ^ (row & 15)); }
template <int D>
__device__ __forceinline__ int v_chunk_pos(int d, int c) { return 4 * D + d * 4 + (c ^ ((d >> 2) & 3)); }

// ---------------------------------------------------------------------------
// Band of an unquantized bf16 cache (page 80, gemma4/model.ts, note on
// cacheLayers: sliding layers stay bf16 under the other KV scheme): the tile
// image above, copied from the stored bf16 values with no arithmetic (a K row's
// words are already pairs in element order, a V block's 16 bytes the 8 keys of
// one element).  Grid (band steps, Hkv, B), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void band_bf16_kernel(AttnDesc P)
{
    constexpr int KE = D / 8;                // K elements per thread
    constexpr int VD = D / 256;              // elements d per thread (head_dim 256, 512)
    const int tid = threadIdx.x;
    const int step = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    const int bh = b * P.Hkv + hkv;
    const int R = P.R;
    const int len = min(max(__builtin_amdgcn_readfirstlane(as_global(P.len)[b]), 0), P.max_len);
    const int vis_lo = band_lo(len, P.C, P.W, R);
    const int p0 = (vis_lo & ~(kStep - 1)) + step * kStep;
    if (p0 >= len) return;                   // past every query: never read
    uint16_t* tile = as_global(P.band) + ((int64_t)bh * (P.nk / kStep + kBandPad) + step) * tile_elems<D>();
    {   // K: key tid/8, elements [KE*(tid%8), +KE); positions no query sees are zeros
        const int key = tid >> 3, ch = tid & 7;
        const int kpos = p0 + key;
        const bool kok = kpos >= vis_lo && kpos < len;
        const uint32_t* src = as_global(P.k_codes) + ((int64_t)bh * R + kpos % R) * (D / 2) + ch * (KE / 2);
        const int row = k_row(key);
#pragma unroll
        for (int e0 = 0; e0 < KE; e0 += 8) {
            u32x4 x = *reinterpret_cast<const u32x4*>(src + e0 / 2);
            if (!kok) x = (u32x4)0;
            *reinterpret_cast<u32x4*>(tile + 8 * k_chunk_pos<D>(row, (ch * KE + e0) / 8)) = x;
        }
    }
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) {       // V: element d, the step's 32 keys (4 blocks of 8 slots)
        const int d = tid + 256 * dd;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int pos8 = p0 + 8 * blk;
            const int slot8 = pos8 % R;                      // a multiple of 8
            const u32x4 x = *reinterpret_cast<const u32x4*>(
                as_global(P.v_codes) + (((int64_t)bh * (R / 8) + slot8 / 8) * D + d) * 4);
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool lo_ok = pos8 + 2 * i >= vis_lo && pos8 + 2 * i < len;
                const bool hi_ok = pos8 + 2 * i + 1 >= vis_lo && pos8 + 2 * i + 1 < len;
                w[i] = x[i] & ((lo_ok ? 0x0000FFFFu : 0u) | (hi_ok ? 0xFFFF0000u : 0u));
            }
            *reinterpret_cast<u32x4*>(tile + 8 * v_chunk_pos<D>(d, blk)) = (u32x4){w[0], w[1], w[2], w[3]};
        }
    }
}

// ---------------------------------------------------------------------------
// Attention over the band tiles (read in place from a bf16 cache, or copied).
//
// A workgroup covers 32 query rows (two row tiles: the 8192 rows of a 512-query
// chunk fill 256 workgroups, one per CU).  Each wave owns RT row tiles of 16
// rows, so 2 / RT waves cover the block; NG such wave groups take alternate
// steps (a key split inside the workgroup) and merge in LDS at the end.
// head_dim 256 runs two key groups (4 waves); head_dim 512 one (its 32 output
// tiles take most of a lane's registers and the step tiles twice the LDS).
template <int D> constexpr int pf_rt() { return 1; }                    // row tiles per wave
template <int D> constexpr int pf_groups() { return D == 256 ? 2 : 1; } // key groups
template <int D> constexpr int pf_waves() { return kPfWaves / pf_rt<D>() * pf_groups<D>(); }

template <int D>
struct __attribute__((aligned(16))) PfSmem {
    static constexpr int NG = pf_groups<D>();
    uint16_t tile[2][NG][tile_elems<D>()];     // [buffer][key group]: step tiles
};

// Copy of one round's step tiles (NG consecutive band tiles, contiguous in the
// workspace) into LDS buffer `slot` with LDS DMA: with NT threads, instruction j
// moves chunks j*NT + tid (16 bytes per lane; a wave's 64 chunks are contiguous
// in LDS and in the band), addressed as the round's base (scalar) plus the lane
// offset 16*(tid + j*NT) (a loop-invariant vector).  Inline assembly keeps the
// compiler from ordering every later LDS read behind the copy: the caller waits
// with vmcnt before the barrier that publishes the buffer.  Each statement
// restores M0 (the LDS base of a DMA), which the compiler reserves.
template <int D>
__device__ __forceinline__ void dma_round(PfSmem<D>& sm, int slot, const uint16_t* src, int tid)
{
    constexpr int NT = 64 * pf_waves<D>();                           // threads
    constexpr int NJ = pf_groups<D>() * tile_elems<D>() / 8 / NT;    // instructions per thread
    static_assert(NJ * NT * 8 == pf_groups<D>() * tile_elems<D>(), "whole chunks per thread");
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&sm.tile[slot][0][0]) + (tid & ~63) * 16);
    const uint64_t base = (uint64_t)(uintptr_t)src;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %1\n\t"
                     "s_nop 0\n\t"
                     "global_load_lds_dwordx4 %2, %3\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "s"(lds0 + j * NT * 16), "v"((uint32_t)tid * 16u + j * NT * 16u), "s"(base)
                     : "memory");
    }
}

// The same round copied straight from a bf16 cache (no band): every lane
// addresses its own 16-byte chunk.  Tile chunk ci of step g (position pos_g, a
// multiple of 32) is, in the K part, chunk c = (ci mod D/8) ^ (row mod 16) of
// the key that LDS row ci / (D/8) holds (k_row inverted), and in the V part the
// 8 keys 8c .. 8c+7 of element d, c = (ci mod 4) ^ ((d / 4) mod 4): one cache V
// block entry.  Slots wrap modulo R (R >= 32 and a multiple of 8, so a step
// base plus 31 wraps at most once and a V block never straddles the wrap).
// Offsets are unsigned 32-bit from the (sequence, KV head) base, which the host
// guarantees by R * D * 2 < 2^31.
template <int D>
__device__ __forceinline__ void dma_round_direct(PfSmem<D>& sm, int slot, uint64_t kbase, uint64_t vbase,
                                                 int pos0, int R, int tid)
{
    constexpr int NT = 64 * pf_waves<D>();
    constexpr int NG = pf_groups<D>();
    constexpr int JT = 8 * D / NT;                   // instructions per step tile
    constexpr int JK = 4 * D / NT;                   // of which K
    static_assert(JT * NT == 8 * D && JK * NT == 4 * D, "whole chunks per thread");
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&sm.tile[slot][0][0]) + (tid & ~63) * 16);
    int pm[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) pm[g] = __builtin_amdgcn_readfirstlane((pos0 + g * kStep) % R);
#pragma unroll
    for (int j = 0; j < NG * JT; ++j) {
        const int g = j / JT, jj = j % JT;
        uint32_t off;
        uint64_t base;
        if (jj < JK) {
            const int ci = jj * NT + tid;
            const int row = ci / (D / 8), r16 = row & 15;
            const int c = (ci % (D / 8)) ^ r16;
            const int key = 8 * (r16 >> 2) + 4 * (row >> 4) + (r16 & 3);
            int sl = pm[g] + key;
            sl = sl >= R ? sl - R : sl;
            off = (uint32_t)sl * (uint32_t)(D * 2) + (uint32_t)c * 16u;
            base = kbase;
        } else {
            const int cv = (jj - JK) * NT + tid;
            const int d = cv >> 2;
            const int c = (cv & 3) ^ ((d >> 2) & 3);
            int s8 = pm[g] + 8 * c;
            s8 = s8 >= R ? s8 - R : s8;
            off = ((uint32_t)(s8 >> 3) * (uint32_t)D + (uint32_t)d) * 16u;
            base = vbase;
        }
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %1\n\t"
                     "s_nop 0\n\t"
                     "global_load_lds_dwordx4 %2, %3\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "s"(lds0 + j * NT * 16), "v"(off), "s"(base)
                     : "memory");
    }
}

template <int D, bool DIRECT>
__device__ __forceinline__ void prefill_body(const AttnDesc& P, int idx, PfSmem<D>& sm)
{
    constexpr int NG = pf_groups<D>(), RT = pf_rt<D>();
    constexpr int RW = kPfWaves / RT;                     // waves per key group
    constexpr int DT = D / 16, KS = D / 32;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;
    const int grp = wave / RW;                            // key group: steps h with h % NG == grp
    const int wrt = (wave % RW) * RT;                     // first row tile of this wave in the block

    // ---- work item: (b, kv head, 32-row block, split)
    const int S = P.S;
    const int n_rb = (P.n_rt + kPfWaves - 1) / kPfWaves;
    const int s = idx % S;
    const int rb = (idx / S) % n_rb;
    const int bh = idx / (S * n_rb);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int R = P.R, W = P.W, C = P.C, hpk = P.hpk;
    // len[b] (a vector load, waited for only where it is used) arrives while
    // the q rows and the first band tiles are requested for len = max_len,
    // the common case; another len re-plans and copies again.
    int oz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(oz));
    const int len_lane = as_global(P.len)[b + oz];

    // ---- this wave's row tiles and this lane's row in each
    const int row0 = rb * kPfRows;
    const int last_row = min(row0 + kPfRows, P.n_rows) - 1;
    const int qi_lo = row0 / hpk, qi_hi = last_row / hpk;
    const int wrow0 = (rb * kPfWaves + wrt) * kRowTile;   // first row of the wave
    const bool wave_on = wrow0 < P.n_rows;
    const int wlast = min(wrow0 + RT * kRowTile, P.n_rows) - 1;
    int qi[RT], hq[RT];
    bool row_ok[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int grow = wrow0 + r * kRowTile + m;
        row_ok[r] = grow < P.n_rows;
        qi[r] = (row_ok[r] ? grow : wrow0) / hpk;
        hq[r] = hkv * hpk + (row_ok[r] ? grow : wrow0) % hpk;
    }

    // ---- q of this lane's rows as MFMA B operands (bf16, natural element order);
    //      a lane past the last row reads the wave's first row and zeroes it
    bf16x8 qf[RT][KS];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const uint16_t* qrow = as_global(P.q[0]) + ((((int64_t)b * P.Hq + hq[r]) * C + qi[r]) * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 u = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
            if (!row_ok[r]) u = (u32x4)0;
            qf[r][ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- key ranges for a given len: the block's keys [j0, j1) in nsteps steps
    //      from st0, each row's [klo, khi], the keys every row of the wave sees
    //      [full_lo, full_hi], and the band tile t0 of step st0
    int j0, j1, nsteps, st0, full_lo, full_hi, t0, vis_lo, len_p;
    int klo[RT], khi[RT];
    auto plan = [&](int len) {
        vis_lo = band_lo(len, C, W, R);
        len_p = len;
        const int base0 = vis_lo & ~(kStep - 1);
        int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
        lo = max(lo, max(0, len - R));
        const int hi = len - C + qi_hi;
        const int base = lo & ~(kStep - 1);
        j0 = max(lo, base + s * P.split_len);
        j1 = min(hi + 1, base + (s + 1) * P.split_len);
        nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
        st0 = j0 & ~(kStep - 1);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int p_row = len - C + qi[r];
            klo[r] = max(j0, W > 0 ? p_row - W + 1 : 0);
            khi[r] = min(j1 - 1, p_row);
            if (!row_ok[r]) { klo[r] = 1; khi[r] = 0; }
        }
        full_lo = max(j0, W > 0 ? len - C + (wave_on ? wlast : wrow0) / hpk - W + 1 : 0);
        full_hi = min(j1 - 1, len - C + wrow0 / hpk);
        t0 = (st0 - base0) / kStep;
    };

    // ---- step tiles: round u copies band tiles t0 + NG*u .. +NG-1, or (DIRECT,
    //      a bf16 cache) the same steps st0 + kStep*(NG*u + g) from the cache
    const uint16_t* band_bh = DIRECT ? nullptr : as_global(P.band) + (int64_t)bh * (P.nk / kStep + kBandPad) * tile_elems<D>();
    const uint64_t kbase = (uint64_t)(uintptr_t)(P.k_codes + (int64_t)bh * R * (D / 2));
    const uint64_t vbase = (uint64_t)(uintptr_t)(P.v_codes + (int64_t)bh * (R / 8) * D * 4);
    auto copy_round = [&](int u, int slot) {
        if constexpr (DIRECT) dma_round_direct<D>(sm, slot, kbase, vbase, st0 + NG * u * kStep, R, tid);
        else dma_round<D>(sm, slot, band_bh + (int64_t)(t0 + NG * u) * tile_elems<D>(), tid);
    };
    plan(P.max_len);
    copy_round(0, 0);
    {
        const int len = min(max(__builtin_amdgcn_readfirstlane(len_lane), 0), P.max_len);
        if (len != P.max_len) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the first copy lands before the second
            plan(len);
            copy_round(0, 0);
        }
    }

    const float sl2e = P.scale_log2e;
    f32x4 O[RT][DT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[r][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.0f; }

    // ---- one step of this wave's rows from its group's LDS buffer `slot`
    auto compute = [&](int st, int slot, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        float z[RT][8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 sacc[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) sacc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    &sm.tile[slot][grp][8 * k_chunk_pos<D>(16 * t + m, 4 * ks + lg)]);
#pragma unroll
                for (int r = 0; r < RT; ++r) sacc[r] = mfma_bf16(a, qf[r][ks], sacc[r]);
            }
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (FULL) {
                        z[r][4 * t + i] = sacc[r][i] * sl2e;
                    } else {
                        const int key = st + 8 * lg + 4 * t + i;
                        z[r][4 * t + i] = (key >= klo[r] && key <= khi[r]) ? sacc[r][i] * sl2e : -INFINITY;
                    }
                }
        }
        // DIRECT: slots of positions outside [vis_lo, len) may hold anything
        // (a stale ring entry, a never-written slot); their weights are 0, and
        // their V^T entries are zeroed here so 0 * NaN cannot reach O.  Keys
        // 8*lg .. 8*lg+7 of the step are this lane's V^T columns.
        u32x4 vmask = (u32x4){~0u, ~0u, ~0u, ~0u};
        if constexpr (DIRECT && !FULL) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k0 = st + 8 * lg + 2 * i;
                vmask[i] = (k0 >= vis_lo && k0 < len_p ? 0x0000FFFFu : 0u) |
                           (k0 + 1 >= vis_lo && k0 + 1 < len_p ? 0xFFFF0000u : 0u);
            }
        }
        bf16x8 pb[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float mloc = z[r][0];
#pragma unroll
            for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, z[r][k]);
            const float mt = max_across_groups(mloc);
            if (__any(mt > m_run[r] + kPfRescaleSlack)) {
                const float m_new = fmaxf(m_run[r], mt);
                const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) O[r][dt] *= alpha;
                l_run[r] *= alpha;
                m_run[r] = m_new;
            }
            const float m_use = m_run[r] == -INFINITY ? 0.0f : m_run[r];
            float p[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                p[k] = __builtin_amdgcn_exp2f(z[r][k] - m_use);
                l_run[r] += p[k];
            }
            // p[k] is key 8*lg + k, the same order as the V^T columns
            const u32x4 pw = {bf16x2_rne(p[0], p[1]), bf16x2_rne(p[2], p[3]),
                              bf16x2_rne(p[4], p[5]), bf16x2_rne(p[6], p[7])};
            pb[r] = __builtin_bit_cast(bf16x8, pw);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.tile[slot][grp][8 * v_chunk_pos<D>(16 * dt + m, lg)]);
            if constexpr (DIRECT && !FULL) a = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, a) & vmask);
#pragma unroll
            for (int r = 0; r < RT; ++r) O[r][dt] = mfma_bf16(a, pb[r], O[r][dt]);
        }
    };
    auto do_compute = [&](int st, int slot) {
        if (!wave_on) return;
        if (st >= full_lo && st + kStep - 1 <= full_hi) compute(st, slot, std::true_type{});
        else compute(st, slot, std::false_type{});
    };

    // ---- pipeline over rounds u = 0 .. nu-1; round u is step NG*u + g for key
    //      group g (a step past nsteps computes nothing).  At round u: start the
    //      copy of round u+1 into LDS buffer (u+1) & 1, run the MFMAs of round u
    //      from buffer u & 1, wait for this thread's copies, one barrier.
    const int nu = (nsteps + NG - 1) / NG;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int u = 0; u < nu; ++u) {
        copy_round(u + 1, (u + 1) & 1);
        const int h = NG * u + grp;
        if (h < nsteps) do_compute(st0 + h * kStep, u & 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- merge the key groups: group g > 0 leaves (m, l, O) in LDS (the tile
    //      buffers are free after the last barrier), group 0 folds them in
    const int wig = wave % RW;                            // wave index within its group
    if constexpr (NG > 1) {
        static_assert(NG == 2, "two key groups");
        float* xo = reinterpret_cast<float*>(&sm.tile[0][0][0]);        // [wig][r][dt][4][lane]
        float* xm = xo + RW * RT * DT * 4 * 64;                        // [wig][r][2][lane]
        static_assert(sizeof(float) * (RW * RT * (DT * 4 + 2) * 64) <= sizeof(PfSmem<D>), "merge fits");
        if (grp == 1) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xo[(((wig * RT + r) * DT + dt) * 4 + i) * 64 + lane] = O[r][dt][i];
                xm[((wig * RT + r) * 2 + 0) * 64 + lane] = m_run[r];
                xm[((wig * RT + r) * 2 + 1) * 64 + lane] = l_run[r];
            }
        }
        __syncthreads();
        if (grp != 0) return;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float m1 = xm[((wig * RT + r) * 2 + 0) * 64 + lane];
            const float l1 = xm[((wig * RT + r) * 2 + 1) * 64 + lane];
            const float mm = fmaxf(m_run[r], m1);
            const float a0 = m_run[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[r] - mm);
            const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    O[r][dt][i] = O[r][dt][i] * a0 + xo[(((wig * RT + r) * DT + dt) * 4 + i) * 64 + lane] * a1;
            l_run[r] = l_run[r] * a0 + l1 * a1;
            m_run[r] = mm;
        }
    }

    // ---- write this wave's rows
    if (!wave_on) return;
    const int dcol = 4 * lg;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const float L = sum_across_groups(l_run[r]);
        if (!row_ok[r]) continue;
        if (S == 1) {
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            uint16_t* orow = as_global(P.out[0]) + ((((int64_t)b * P.Hq + hq[r]) * C + qi[r]) * D);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o = O[r][dt] * inv;
                uint2 w;
                w.x = bf16x2_rne(o[0], o[1]);
                w.y = bf16x2_rne(o[2], o[3]);
                *reinterpret_cast<uint2*>(orow + dcol + 16 * dt) = w;
            }
        } else {
            const int rt = rb * kPfWaves + wrt + r;       // 16-row tile index
            const int64_t ib = (int64_t)bh * P.n_rt + rt;
            const int64_t prow = (ib * S + s) * kRowTile + m;
            float* po = as_global(P.part) + prow * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dcol + 16 * dt) = O[r][dt];
            if (lg == 0) {
                float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
                pml[0] = m_run[r];
                pml[1] = L;
            }
        }
    }
}

// Workgroup i runs on XCD i % 8 (round-robin dispatch).  Consecutive work items
// (the row blocks of one sequence and KV head, which all read the same band)
// are given to one XCD, so the band is fetched into that XCD's L2 once and the
// other row blocks hit it there.

template <int D, bool DIRECT>
__global__ __launch_bounds__(64 * pf_waves<D>()) void prefill_kernel(AttnParams P)
{
    __shared__ PfSmem<D> sm;
    prefill_body<D, DIRECT>(P.d[0], xcd_item(blockIdx.x, gridDim.x), sm);
}

hipError_t launch_band(const AttnParams& p, hipStream_t stream)
{
    const AttnDesc& d = p.d[0];
    const dim3 dq_grid(d.nk / kStep, d.Hkv, d.B), block(256);
    switch (d.cfg) {
    case cfg_of(256, 16, 16): case cfg_of(512, 16, 16):   // bf16: the attention kernel reads the cache itself
        if (d.band != nullptr) {
            if (d.cfg == cfg_of(256, 16, 16)) band_bf16_kernel<256><<<dq_grid, block, 0, stream>>>(d);
            else band_bf16_kernel<512><<<dq_grid, block, 0, stream>>>(d);
        }
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const AttnParams& p, int total_items, hipStream_t stream)
{
    const AttnDesc& d = p.d[0];
    const bool direct = cfg_is_bf16(d.cfg) && d.band == nullptr;
    const dim3 grid(total_items);
    if (d.D == 256) {
        const dim3 block(64 * pf_waves<256>());
        return direct ? launch_read(prefill_kernel<256, true>, grid, block, p, stream)
                      : launch_read(prefill_kernel<256, false>, grid, block, p, stream);
    }
    if (d.D == 512) {
        const dim3 block(64 * pf_waves<512>());
        return direct ? launch_read(prefill_kernel<512, true>, grid, block, p, stream)
                      : launch_read(prefill_kernel<512, false>, grid, block, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvq

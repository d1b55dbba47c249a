// Unquantized bf16 caches, gfx950: append and split-KV attention.
//
// Page 80 of the @mlx-bun/inference 0.0.0-stage -> 1.0.0 diff (gemma4/model.ts,
// the note on cacheLayers) keeps the sliding layers' caches in bf16 under the
// model's other KV scheme: a ring of the window, read by the same SDPA as the
// quantized caches (read.attend(q, 1.0) in attentionTraining).  A bf16 cache
// uses the quantized layouts with 16-bit "codes" that are the bf16 values
// themselves and no scale or bias:
//   K  uint32 [B][H][R][D/2]      token-major, element 2w in the low half of word w
//   V  uint32 [B][H][R/8][D][4]   blocked: the 8 values of one head_dim element
//                                 for 8 consecutive slots in 16 bytes, slot 8n+t
//                                 in halfword t
// so a K row is read along head_dim and a V block along keys, as the two
// contractions read them.
//
// Attention: one workgroup per (descriptor, sequence and KV head, 16-row tile,
// split), the work items, row maps, key ranges and partials of the quantized
// decode kernel (attn.hip), so splits go through the same combine kernel.  The
// four waves split head_dim; per 32-key step each computes S^T = K Q^T over
// its columns on 16x16x32 bf16 MFMA (K rows straight from memory as the A
// operand, q as B), the partial scores meet in LDS, every wave runs the same
// online softmax (base 2, lazy rescale) and accumulates O^T = V^T P^T for its
// columns with the bf16 V block as the A operand and P in bf16 as B.  K and V
// of the next step are loaded while the current one is computed.
//
// Fused decode step (page 80, attentionTraining: the token is appended, then
// read): one more split per item takes the step's token at position len-1 --
// the item of row tile 0 writes it into the cache, and every item emits, per
// row, the partial m = scale*log2(e)*(q . k), l = 1, o = v of that one key
// from the token's bf16-rounded values -- while the other splits leave that
// position out.  The token's slot is outside every other split's range (and
// outside the window of the position it replaces), so no read depends on the
// write's timing.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// ---- append: one workgroup per (token, KV head, sequence); a thread converts
//      element pairs.  Distinct tokens of a call land in distinct slots, and V
//      is written one halfword per (slot, element), so no two threads touch the
//      same bytes.
__global__ __launch_bounds__(256) void append_bf16_kernel(AppendParams p)
{
    const int t = p.t_first + (int)blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int D = p.D, R = p.R;
    const int64_t bh = (int64_t)b * p.H + h;
    const int64_t pos = (int64_t)p.pos0[b] + t;
    const int slot = (int)(((pos % R) + R) % R);
    const float* ksrc = p.k + (bh * p.T + t) * D;
    const float* vsrc = p.v + (bh * p.T + t) * D;
    uint32_t* kdst = p.k_codes + (bh * R + slot) * (D / 2);
    uint16_t* vdst = reinterpret_cast<uint16_t*>(p.v_codes) + ((bh * (R / 8) + slot / 8) * D) * 8 + (slot & 7);
    for (int d = 2 * (int)threadIdx.x; d < D; d += 2 * (int)blockDim.x) {
        const float2 k2 = *reinterpret_cast<const float2*>(ksrc + d);
        const float2 v2 = *reinterpret_cast<const float2*>(vsrc + d);
        kdst[d / 2] = (uint32_t)f32_to_bf16_rne(k2.x) | ((uint32_t)f32_to_bf16_rne(k2.y) << 16);
        vdst[(int64_t)d * 8] = f32_to_bf16_rne(v2.x);
        vdst[(int64_t)(d + 1) * 8] = f32_to_bf16_rne(v2.y);
    }
}

hipError_t launch_append_bf16(const AppendParams& p, hipStream_t stream)
{
    if (p.n_written <= 0) return hipSuccess;
    append_bf16_kernel<<<dim3(p.n_written, p.H, p.B), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

// ---- attention
template <int D>
struct BfShape {
    static constexpr int NW = 4;          // waves; wave w owns columns [w*DW, (w+1)*DW)
    static constexpr int DW = D / NW;     // 32, 64 or 128
    static constexpr int KC = DW / 32;    // 32-column chunks of the QK contraction per wave
    static constexpr int DT = DW / 16;    // 16-column output tiles per wave
};

struct BfSmem {
    f32x4 spart[2][4][2][kWave];          // partial S^T tiles [step parity][wave][tile][lane]
};

template <int D>
struct BfRegs {
    u32x4 k[2][BfShape<D>::KC];           // K rows of the step (A operands of the two score tiles)
    u32x4 v[BfShape<D>::DT];              // V blocks of the step (A operands of the output tiles)
};

constexpr float kBfRescaleSlack = 8.0f;

// The fused step's token split (see the header): 16 lanes per query row.
template <int D>
__device__ __forceinline__ void bf16_new_token(const AttnDesc& P, int bh, int rt, int s)
{
    constexpr int PARTS = 16, EPP = D / PARTS;     // elements per lane: 8, 16 or 32
    const int tid = threadIdx.x;
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    const int R = P.R, C = P.C;
    const int len = min(max(__builtin_amdgcn_readfirstlane(as_global(P.len)[b]), 1), P.max_len);
    const int slot = (len - 1) % R;
    const float* ksrc = as_global(P.k_new) + (int64_t)bh * D;
    const float* vsrc = as_global(P.v_new) + (int64_t)bh * D;
    if (rt == 0) {                                  // the cache write, once per (sequence, KV head)
        // the cache arrays of a fused step are the caller's writable cache
        uint32_t* kdst = const_cast<uint32_t*>(as_global(P.k_codes)) + ((int64_t)bh * R + slot) * (D / 2);
        uint16_t* vdst = reinterpret_cast<uint16_t*>(const_cast<uint32_t*>(as_global(P.v_codes))) +
                         (((int64_t)bh * (R / 8) + slot / 8) * D) * 8 + (slot & 7);
        for (int d = 2 * tid; d < D; d += 2 * (int)blockDim.x) {
            const float2 k2 = *reinterpret_cast<const float2*>(ksrc + d);
            const float2 v2 = *reinterpret_cast<const float2*>(vsrc + d);
            kdst[d / 2] = (uint32_t)f32_to_bf16_rne(k2.x) | ((uint32_t)f32_to_bf16_rne(k2.y) << 16);
            vdst[(int64_t)d * 8] = f32_to_bf16_rne(v2.x);
            vdst[(int64_t)(d + 1) * 8] = f32_to_bf16_rne(v2.y);
        }
    }
    const int r = tid / PARTS, part = tid % PARTS;
    const int grow = rt * kRowTile + r;
    if (grow >= P.n_rows) return;
    const int layer = C == 1 ? grow / P.hpk : 0;
    const int qi = C == 1 ? 0 : grow / P.hpk;
    const int hq = hkv * P.hpk + grow % P.hpk;
    const uint16_t* qrow = as_global(P.q[layer]) + ((((int64_t)b * P.Hq + hq) * C + qi) * D) + part * EPP;
    const float* kp = ksrc + part * EPP;
    float acc = 0.0f;
#pragma unroll
    for (int e0 = 0; e0 < EPP; e0 += 8) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(qrow + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float k0 = __uint_as_float((uint32_t)f32_to_bf16_rne(kp[e0 + 2 * i]) << 16);
            const float k1 = __uint_as_float((uint32_t)f32_to_bf16_rne(kp[e0 + 2 * i + 1]) << 16);
            acc += bf16_lo_to_f32(u[i]) * k0 + bf16_hi_to_f32(u[i]) * k1;
        }
    }
#pragma unroll
    for (int o = 1; o < PARTS; o <<= 1) acc += __shfl_xor(acc, o);
    const int64_t prow = (((int64_t)bh * P.n_rt + rt) * P.S + s) * kRowTile + r;
    float* po = as_global(P.part) + prow * D + part * EPP;
    const float* vp = vsrc + part * EPP;
#pragma unroll
    for (int e0 = 0; e0 < EPP; e0 += 4) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float((uint32_t)f32_to_bf16_rne(vp[e0 + i]) << 16);
        *reinterpret_cast<f32x4*>(po + e0) = o;
    }
    if (part == 0) {
        float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * P.S * kRowTile * D + prow * 2;
        pml[0] = acc * P.scale_log2e;
        pml[1] = 1.0f;
    }
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float x) { return f32_to_bf16_rne(x); }

template <int D>
__device__ __forceinline__ void attn_bf16_body(const AttnDesc& P, int idx, BfSmem& sm)
{
    using Sh = BfShape<D>;
    constexpr int NW = Sh::NW, DW = Sh::DW, KC = Sh::KC, DT = Sh::DT;
    constexpr int KW = D / 2;             // K words per slot

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, lg = lane >> 4;
    const int c0 = wave * DW;             // first column of this wave

    const int S = P.S;
    const int s = idx % S;
    const int rt = (idx / S) % P.n_rt;
    const int bh = idx / (S * P.n_rt);
    const int b = bh / P.Hkv, hkv = bh - b * P.Hkv;
    if (P.k_new != nullptr && s == S - 1) {
        bf16_new_token<D>(P, bh, rt, s);
        return;
    }
    const int R = P.R, W = P.W, C = P.C;
    const int len = min(max(__builtin_amdgcn_readfirstlane(as_global(P.len)[b]), 0), P.max_len);

    // ---- rows of this tile and key range of this work item (as in attn.hip)
    const int row0 = rt * kRowTile;
    const int last_row = min(row0 + kRowTile, P.n_rows) - 1;
    const int qi_lo = C == 1 ? 0 : row0 / P.hpk;
    const int qi_hi = C == 1 ? 0 : last_row / P.hpk;
    const int grow = row0 + m;
    const bool row_ok = grow < P.n_rows;
    const int rsel = row_ok ? grow : row0;
    const int layer = C == 1 ? rsel / P.hpk : 0;
    const int qi = C == 1 ? 0 : rsel / P.hpk;
    const int hq = hkv * P.hpk + rsel % P.hpk;
    int lo = W > 0 ? len - C + qi_lo - W + 1 : 0;
    lo = max(lo, max(0, len - R));
    const int hi = len - C + qi_hi - P.excl;        // excl: the fused step's token split has len-1
    const int base = lo & ~(kStep - 1);
    const int j0 = max(lo, base + s * P.split_len);
    const int j1 = min(hi + 1, base + (s + 1) * P.split_len);
    const int full_lo = max(j0, W > 0 ? len - C + qi_hi - W + 1 : 0);
    const int full_hi = min(j1 - 1, len - C + qi_lo - P.excl);
    const int p_row = len - C + qi;
    int klo = max(j0, W > 0 ? p_row - W + 1 : 0);
    int khi = min(j1 - 1, p_row - P.excl);
    if (!row_ok) { klo = 1; khi = 0; }
    const int nsteps = j0 < j1 ? ((j1 - 1) >> 5) - (j0 >> 5) + 1 : 0;
    const int st0 = j0 & ~(kStep - 1);

    // ---- q of this lane's row over this wave's columns, as MFMA B operands
    bf16x8 qb[KC];
    {
        const uint16_t* qrow = as_global(P.q[layer]) + ((((int64_t)b * P.Hq + hq) * C + qi) * D);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            u32x4 u = *reinterpret_cast<const u32x4*>(qrow + c0 + 32 * c + 8 * lg);
            if (!row_ok) u = (u32x4)0;
            qb[c] = __builtin_bit_cast(bf16x8, u);
        }
    }

    const int64_t kslot0 = (int64_t)bh * R;
    const uint32_t* __restrict__ kbase = as_global(P.k_codes) + kslot0 * KW + (c0 + 8 * lg) / 2;
    const uint32_t* __restrict__ vbase = as_global(P.v_codes) + ((int64_t)bh * (R / 8) * D + c0 + m) * 4;
    auto load = [&](BfRegs<D>& r, int st) {
        const int st_mod = st % R;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kk = 8 * (m >> 2) + 4 * t + (m & 3);
            const uint32_t* krow = kbase + (int64_t)wrap_slot(st_mod + kk, R) * KW;
#pragma unroll
            for (int c = 0; c < KC; ++c) r.k[t][c] = *reinterpret_cast<const u32x4*>(krow + 16 * c);
        }
        const uint32_t* vblk = vbase + (int64_t)(wrap_slot(st_mod + 8 * lg, R) >> 3) * D * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) r.v[dt] = *reinterpret_cast<const u32x4*>(vblk + 16 * dt * 4);
    };

    const float sl2e = P.scale_log2e;
    f32x4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // One step: partial scores -> LDS -> full scores -> online softmax -> PV.
    // Tile t row r of S^T holds key 8*(r/4) + 4*t + r%4, so lane group lg ends
    // with the scores of keys 8*lg .. 8*lg+7: the B operand of the PV MFMA.
    auto step = [&](const BfRegs<D>& r, int i) {
        const int st = st0 + i * kStep;
        const int par = i & 1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KC; ++c) acc = mfma_bf16(__builtin_bit_cast(bf16x8, r.k[t][c]), qb[c], acc);
            sm.spart[par][wave][t][lane] = acc;
        }
        __syncthreads();
        const bool full = st >= full_lo && st + kStep - 1 <= full_hi;
        float z[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = sm.spart[par][0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) acc += sm.spart[par][w][t][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = st + 8 * lg + 4 * t + e;
                z[4 * t + e] = (full || (key >= klo && key <= khi)) ? acc[e] * sl2e : -INFINITY;
            }
        }
        float mloc = z[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, z[k]);
        const float mt = max_across_groups(mloc);
        if (__any(mt > m_run + kBfRescaleSlack)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        uint16_t ph[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float e = __builtin_amdgcn_exp2f(z[k] - m_use);   // 0 for a masked key
            l_run += e;
            ph[k] = bf16_bits_rne(e);
        }
        const u32x4 pw = {ph[0] | ((uint32_t)ph[1] << 16), ph[2] | ((uint32_t)ph[3] << 16),
                          ph[4] | ((uint32_t)ph[5] << 16), ph[6] | ((uint32_t)ph[7] << 16)};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        // keys outside the item's range may sit in slots never written: their V
        // values are zeroed, so whatever bits they hold cannot reach O
        uint32_t vmask[4] = {~0u, ~0u, ~0u, ~0u};
        if (!full) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int key = st + 8 * lg + k;
                if (key < j0 || key >= j1) vmask[k >> 1] &= (k & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x4 v = r.v[dt];
            const u32x4 vm = {v.x & vmask[0], v.y & vmask[1], v.z & vmask[2], v.w & vmask[3]};
            O[dt] = mfma_bf16(__builtin_bit_cast(bf16x8, vm), pb, O[dt]);
        }
    };

    // Steps in pairs over two register sets: the loads of step i+1 are in
    // flight while step i is computed.  Loads are unconditional with the step
    // index clamped, so past the end the last step is read again.
    const int last = max(nsteps - 1, 0);
    auto stp = [&](int i) { return st0 + min(i, last) * kStep; };
    BfRegs<D> ra, rb;
    load(ra, stp(0));
    load(rb, stp(1));
    for (int i = 0; i < nsteps; i += 2) {
        step(ra, i);
        load(ra, stp(i + 2));
        if (i + 1 >= nsteps) break;
        step(rb, i + 1);
        load(rb, stp(i + 3));
    }

    // ---- lane (m, lg) holds O^T[c0 + 16*dt + 4*lg + e][row m]
    const float L = sum_across_groups(l_run);
    const int dcol = c0 + 4 * lg;
    if (!row_ok) return;
    if (S == 1) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* orow = as_global(P.out[layer]) + ((((int64_t)b * P.Hq + hq) * C + qi) * D);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = O[dt] * inv;
            uint2 w;
            w.x = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
            w.y = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
            *reinterpret_cast<uint2*>(orow + dcol + 16 * dt) = w;
        }
        return;
    }
    const int64_t ib = (int64_t)bh * P.n_rt + rt;
    const int64_t prow = (ib * S + s) * kRowTile + m;
    float* po = as_global(P.part) + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dcol + 16 * dt) = O[dt];
    if (wave == 0 && lg == 0) {
        float* pml = as_global(P.part) + (size_t)P.B * P.Hkv * P.n_rt * S * kRowTile * D + prow * 2;
        pml[0] = m_run;
        pml[1] = L;
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnParams P)
{
    __shared__ BfSmem sm;
    const int bid = blockIdx.x;
    int di = 0;
    while (di + 1 < P.n_desc && bid >= P.d[di + 1].item_begin) ++di;
    attn_bf16_body<D>(P.d[di], bid - P.d[di].item_begin, sm);
}

hipError_t launch_attn_bf16(const AttnParams& p, int total_items, hipStream_t stream)
{
    const dim3 grid(total_items), block(256);
    switch (p.d[0].D) {
    case 128: return launch_read(attn_bf16_kernel<128>, grid, block, p, stream);
    case 384: return launch_read(attn_bf16_kernel<384>, grid, block, p, stream);
    case 256: return launch_read(attn_bf16_kernel<256>, grid, block, p, stream);
    case 512: return launch_read(attn_bf16_kernel<512>, grid, block, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq

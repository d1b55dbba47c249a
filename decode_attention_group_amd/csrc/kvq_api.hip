// Host side of the C ABI declared in include/kvq.h: argument validation, launch
// planning (row tiles, split-KV), workspace sizing and thread-local errors.
// Nothing here allocates device memory.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kvq_internal.h"

#define KVQ_API extern "C" __attribute__((visibility("default")))

// Split partials of kvq_attn_decode_static, for callers that cannot allocate:
// one copy of this array per device, held until the process ends.  Host code
// never uses its name as an address: the device address comes from
// hipGetSymbolAddress, once per device (static_scratch below).
static __device__ __align__(256) unsigned char scratch[KVQ_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";
// kvq_mark_next_read: events the next attention call records around its main kernel
thread_local hipEvent_t g_mark_before = nullptr;
thread_local hipEvent_t g_mark_after = nullptr;

// armed between mark_before and mark_after: the events the read kernels take
thread_local hipEvent_t g_kstart = nullptr;
thread_local hipEvent_t g_kstop = nullptr;

void mark_before(hipStream_t)
{
    g_kstart = g_mark_before;
    g_kstop = g_mark_after;
    g_mark_before = nullptr;
}

void mark_after(hipStream_t) { g_kstart = g_kstop = nullptr; }

// Every attention call ends its marks (armed for one call only).
struct MarkScope {
    ~MarkScope() { g_mark_before = g_mark_after = g_kstart = g_kstop = nullptr; }
};

kvq_status fail(kvq_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kvq_status ok()
{
    g_err[0] = '\0';
    return KVQ_OK;
}

bool trace_on()
{
    static const int on = [] { const char* e = getenv("KVQ_TRACE"); return e && *e && *e != '0'; }();
    return on != 0;
}

kvq_status check_cache(const kvq_cache* c, const char* what)
{
    if (!c) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: cache descriptor is NULL", what);
    const bool bf16 = c->k_bits == 16 && c->v_bits == 16;
    if (!c->k_codes || !c->v_codes || (!bf16 && (!c->k_sb || !c->v_sb)))
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: a cache array pointer is NULL", what);
    if (c->group_size != KVQ_GROUP_SIZE)
        return fail(KVQ_ERR_UNSUPPORTED, "%s: group_size %d (only 64 is supported)", what, c->group_size);
    if (c->head_dim < 64 || c->head_dim > 512 || c->head_dim % 64 != 0)
        return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d (supported: multiples of 64 up to 512)", what, c->head_dim);
    if (bf16 && c->head_dim % 128 != 0)
        return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d on a bf16 cache (supported: 128, 256, 384, 512)", what,
                    c->head_dim);
    if (!bf16 && ((c->k_bits != 4 && c->k_bits != 8) || (c->v_bits != 4 && c->v_bits != 8)))
        return fail(KVQ_ERR_UNSUPPORTED, "%s: k_bits %d / v_bits %d (each 4 or 8, or both 16)", what, c->k_bits,
                    c->v_bits);
    if (c->batch < 1 || c->n_kv_heads < 1)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch %d and n_kv_heads %d must be >= 1", what, c->batch, c->n_kv_heads);
    // launch grids put (2x) batch and the KV heads on 16-bit grid dimensions
    if (c->batch > 32767 || c->n_kv_heads > 65535)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch %d or n_kv_heads %d too large", what, c->batch, c->n_kv_heads);
    // rows and blocks are read with 16-byte loads
    const uintptr_t ca = reinterpret_cast<uintptr_t>(c->k_codes) | reinterpret_cast<uintptr_t>(c->v_codes) |
                         reinterpret_cast<uintptr_t>(c->k_sb) | reinterpret_cast<uintptr_t>(c->v_sb);
    if (ca & 15) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: cache arrays must be 16-byte aligned", what);
    // a read loads the slots of a 32-key step as (step start mod R) + k, k < 32,
    // wrapped with one subtraction: in range for R >= 32
    if (c->capacity < KVQ_MIN_CAPACITY || c->capacity % KVQ_V_BLOCK != 0)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: capacity %d must be a multiple of 8 and at least %d", what,
                    c->capacity, KVQ_MIN_CAPACITY);
    if (c->window < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: window %d < 0", what, c->window);
    if (c->window > c->capacity)
        return fail(KVQ_ERR_CAPACITY, "%s: window %d exceeds capacity %d", what, c->window, c->capacity);
    if (c->capacity > (INT_MAX / 2))
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: capacity %d too large", what, c->capacity);
    // the kernels address one (sequence, KV head)'s codes with 32-bit word offsets
    if ((int64_t)c->capacity * c->head_dim * std::max(c->k_bits, c->v_bits) / 32 > INT_MAX)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: capacity %d x head_dim %d at %d bits exceeds 8 GiB of codes per "
                    "sequence and KV head", what, c->capacity, c->head_dim, std::max(c->k_bits, c->v_bits));
    return KVQ_OK;
}

int env_splits()
{
    const char* e = getenv("KVQ_SPLITS");
    return e ? atoi(e) : 0;
}

// One read of one cache by `n_layers` layers (decode/shared) or by a chunk of
// C queries (prefill).
struct ReadSpec {
    const kvq_cache* cache;
    int n_layers;
    const uint16_t* const* q;
    uint16_t* const* out;
    int Hq;
    float scale;
    const int32_t* len;
    int max_len;
    int C;             // 1: decode rows are layers x heads; > 1: prefill rows are queries x heads
    const float* k_new = nullptr;   // fused decode step: the step's K and V rows, appended by the read
    const float* v_new = nullptr;
};

kvq_status check_read(const ReadSpec& r, const char* what)
{
    kvq_status st = check_cache(r.cache, what);
    if (st != KVQ_OK) return st;
    const kvq_cache* c = r.cache;
    if (r.n_layers < 1 || r.n_layers > KVQ_MAX_SHARED_LAYERS)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_layers %d outside [1, %d]", what, r.n_layers, KVQ_MAX_SHARED_LAYERS);
    if (!r.q || !r.out) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q/out pointer array is NULL", what);
    for (int l = 0; l < r.n_layers; ++l) {
        if (!r.q[l] || !r.out[l]) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q or out of layer %d is NULL", what, l);
        // q rows are read with 16-byte loads, outputs written 8 bytes at a time
        if ((reinterpret_cast<uintptr_t>(r.q[l]) & 15) || (reinterpret_cast<uintptr_t>(r.out[l]) & 7))
            return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q of layer %d must be 16-byte and out 8-byte aligned", what, l);
    }
    if (!r.len) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: len is NULL", what);
    if (r.Hq < 1 || r.Hq % c->n_kv_heads != 0)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_q_heads %d is not a positive multiple of n_kv_heads %d",
                    what, r.Hq, c->n_kv_heads);
    if (!std::isfinite(r.scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: scale is not finite", what);
    if (r.C < 1) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: chunk %d < 1", what, r.C);
    if (r.max_len < r.C)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: max_len %d < %d queries per sequence", what, r.max_len, r.C);
    if (c->window == 0 && r.max_len > c->capacity)
        return fail(KVQ_ERR_CAPACITY, "%s: full-attention cache of capacity %d cannot hold max_len %d",
                    what, c->capacity, r.max_len);
    if (c->window > 0 && (int64_t)c->window + r.C - 1 > c->capacity)
        return fail(KVQ_ERR_CAPACITY, "%s: window %d + chunk %d - 1 exceeds capacity %d",
                    what, c->window, r.C, c->capacity);
    const int64_t rows = (int64_t)(r.C == 1 ? r.n_layers : r.C) * (r.Hq / c->n_kv_heads);
    if (rows > (1 << 24)) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: too many query rows", what);
    return KVQ_OK;
}

// Fill the descriptor's shape and split plan.  `target_wg` is the number of
// workgroups this read should aim for.  fold: a fused step's token (quantized
// cache) is taken by the last split of each item instead of a split of its own.
void plan_read(const ReadSpec& r, int target_wg, kvq::AttnDesc& d, bool fold = false)
{
    const kvq_cache* c = r.cache;
    std::memset(&d, 0, sizeof(d));
    d.k_codes = c->k_codes;
    d.v_codes = c->v_codes;
    d.k_sb = c->k_sb;
    d.v_sb = c->v_sb;
    for (int l = 0; l < r.n_layers && l < KVQ_MAX_SHARED_LAYERS; ++l) {   // sizing queries pass no pointers
        d.q[l] = r.q ? r.q[l] : nullptr;
        d.out[l] = r.out ? r.out[l] : nullptr;
    }
    d.len = r.len;
    d.B = c->batch;
    d.Hkv = c->n_kv_heads;
    d.Hq = r.Hq;
    d.R = c->capacity;
    d.W = c->window;
    d.C = r.C;
    d.D = c->head_dim;
    d.max_len = r.max_len;
    d.hpk = r.Hq / c->n_kv_heads;
    d.n_rows = (r.C == 1 ? r.n_layers : r.C) * d.hpk;
    d.n_layers = r.C == 1 ? r.n_layers : 1;
    d.n_rt = (d.n_rows + kvq::kRowTile - 1) / kvq::kRowTile;
    d.scale_log2e = r.scale * kvq::kLog2e;
    d.cfg = kvq::cfg_id(c->head_dim, c->k_bits, c->v_bits);

    // Keys one row tile can see, plus the alignment of its first step.
    int64_t vis = r.max_len;
    if (c->window > 0) {
        const int64_t span = r.C == 1 ? 1 : (kvq::kRowTile + d.hpk - 1) / d.hpk + 1;
        vis = std::min<int64_t>(vis, (int64_t)c->window + span);
    }
    const int64_t steps = (vis + 2 * kvq::kStep - 1) / kvq::kStep;
    const int64_t items = (int64_t)d.B * d.Hkv * d.n_rt;
    int64_t S = (target_wg + items - 1) / items;
    // a fused step's token: a split of its own per item (it counts against the
    // target), unless the last split takes it (fold)
    const bool tok_fold = r.k_new && fold && c->k_bits != 16;
    const bool tok_split = r.k_new && !tok_fold;
    if (tok_split) S = std::max<int64_t>(1, S - 1);
    // two steps per split where that still leaves 128 workgroups: a workgroup's
    // first step costs a full memory round trip, its second overlaps it
    // (measured on 8 sequences x 2 KV heads over a 512-key window: 11.3 us at 9
    // splits against 11.7 us at 18); below that, one step per split
    const int64_t min_steps_per_split = items * ((steps + 1) / 2) >= 128 ? 2 : 1;
    S = std::min<int64_t>(S, (steps + min_steps_per_split - 1) / min_steps_per_split);
    // a short read (a window of up to 32 steps) in about 192 workgroups at most:
    // past that, more splits cost more in partials and in the combine than their
    // parallel first loads gain (5 queries x 8 heads of B8 over a 512-key window,
    // 32 items: 13.7 us at 6 splits against 14.8 us at 9; the sliding decode, 16
    // items, sits on its plateau at 9-12 splits)
    if (steps <= 32) S = std::min<int64_t>(S, std::max<int64_t>(1, 192 / items));
    const int forced = env_splits();
    if (forced > 0) S = forced;
    const int64_t max_s = tok_split ? kvq::kMaxSplits - 1 : kvq::kMaxSplits;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(steps, max_s)));
    const int64_t steps_per = (steps + S - 1) / S;
    d.split_len = (int)(steps_per * kvq::kStep);
    d.S = (int)((steps + steps_per - 1) / steps_per);
    if (r.k_new) {
        d.k_new = r.k_new;
        d.v_new = r.v_new;
        d.excl = 1;
        d.tok_fold = tok_fold ? 1 : 0;
        if (tok_split) d.S += 1;
    }
    d.n_items = (int)(items * d.S);
}

// Kernel path of a chunk read:
//   decode: head_dim 128, or a short chunk over a short key range: the decode
//     kernel with per-row positions (each 16-row tile reads the keys; for a
//     window of a few hundred keys the re-reads are cheaper than the
//     alternatives: 15.6 us against 18.1 us for 5 queries x 8 heads of B8 over
//     a 512-key window);
//   codes:  head_dim 256/512, up to 64 rows per KV head over more than 2048
//     keys (speculative-verify windows on full layers): each workgroup holds
//     all the rows, so every key is read once, and dequantizes each step into
//     LDS once (prefill_codes.hip; 63 us against 98 us on the decode path for
//     5 queries x 8 heads of B4 over 32768 keys of head_dim 512).  Inside a
//     mixed launch such a read runs in a launch of its own (74 us against 90
//     us for the whole mixed read of three decoding layers plus a 5-query
//     verify over 16384 keys, B8, with traffic 1.18x the algorithmic bytes
//     against 3.07x);
//   band:   longer chunks: the chunk's key band is dequantized once into the
//     workspace as bf16, then 32 query rows per workgroup (prefill.hip).
// A bf16 cache takes the band path for chunks of more than 64 rows per KV head
// (its band is a copy), else its own split kernel (bf16_cache.hip).
enum class ChunkPath { kDecode, kCodes, kBand };

ChunkPath chunk_path(const kvq_cache* c, int n_q_heads, int chunk, int max_len)
{
    const bool big = chunk > 1 && kvq::chunk_kernels_for(c->head_dim);
    if (c->k_bits == 16) {                 // bf16 caches: the bf16 split kernel, or the band (no short-chunk kernel)
        const char* f = getenv("KVQ_PREFILL_PATH");
        if (f && *f) return big && f[0] == 'b' ? ChunkPath::kBand : ChunkPath::kDecode;
        return big && (int64_t)chunk * (n_q_heads / c->n_kv_heads) > kvq::kCodesPrefillRows ? ChunkPath::kBand
                                                                                           : ChunkPath::kDecode;
    }
    const int64_t rows = (int64_t)chunk * (n_q_heads / c->n_kv_heads);
    const char* e = getenv("KVQ_PREFILL_PATH");          // "band" / "codes" / "decode": force (measurement)
    if (e && *e) return !big ? ChunkPath::kDecode : e[0] == 'b' ? ChunkPath::kBand
                                                  : e[0] == 'c' ? ChunkPath::kCodes : ChunkPath::kDecode;
    if (!big || rows <= kvq::kRowTile) return ChunkPath::kDecode;
    if (rows > kvq::kCodesPrefillRows) return ChunkPath::kBand;
    const int64_t keys = c->window > 0 ? std::min<int64_t>((int64_t)c->window + chunk - 1, max_len) : max_len;
    return keys > 2048 ? ChunkPath::kCodes : ChunkPath::kDecode;
}

// Short-chunk (codes) kernel plan of one read: one workgroup per (b, kv head,
// 64-row block, split), n_items of them, in a launch of its own.
void plan_codes_desc(const ReadSpec& r, kvq::AttnDesc& d)
{
    plan_read(r, 1, d);                           // shape fields
    const kvq_cache* c = r.cache;
    const int n_rb = (d.n_rows + kvq::kCodesPrefillRows - 1) / kvq::kCodesPrefillRows;
    int64_t vis = r.max_len;
    if (c->window > 0)
        vis = std::min<int64_t>(vis, (int64_t)c->window + (kvq::kCodesPrefillRows + d.hpk - 1) / d.hpk);
    const int64_t steps = (vis + 2 * kvq::kStep - 1) / kvq::kStep;
    const int64_t items = (int64_t)d.B * d.Hkv * n_rb;
    // resident workgroups: two per CU for head_dim 256, one for 512 (its LDS)
    const int kTargetWg = d.D == 512 ? 256 : 512;
    int64_t S = (kTargetWg + items - 1) / items;
    const int forced = env_splits();
    if (forced > 0) S = forced;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(steps, kvq::kMaxSplits)));
    const int64_t steps_per = (steps + S - 1) / S;
    d.split_len = (int)(steps_per * kvq::kStep);
    d.S = (int)((steps + steps_per - 1) / steps_per);
    d.n_items = (int)(items * d.S);
    d.own_launch = 1;
    d.part_h = 1;
}

size_t plan_all(const ReadSpec* rs, int n, kvq::AttnParams& P, int& total_items)
{
    std::memset(&P, 0, sizeof(P));
    P.n_desc = n;
    double bytes[KVQ_MAX_SHARED_GROUPS];
    double total = 0.0;
    // A chunk read that the short-chunk kernel serves best (see chunk_path) runs
    // in a launch of its own, where every key is read once for all its rows; the
    // other reads share one launch and its workgroup budget.
    bool own[KVQ_MAX_SHARED_GROUPS];
    for (int i = 0; i < n; ++i)
        own[i] = rs[i].C > 1 && chunk_path(rs[i].cache, rs[i].Hq, rs[i].C, rs[i].max_len) == ChunkPath::kCodes;
    for (int i = 0; i < n; ++i) {
        bytes[i] = 0.0;
        if (own[i]) continue;
        const kvq_cache* c = rs[i].cache;
        const double per_key = c->head_dim * (c->k_bits + c->v_bits) / 8.0 + 4.0 * 2 * c->head_dim / 64;
        const double vis = c->window > 0 ? std::min(c->window, rs[i].max_len) : rs[i].max_len;
        bytes[i] = (double)c->batch * c->n_kv_heads * vis * per_key;
        total += bytes[i];
    }
    const int kTargetWg = 512;   // two 4-wave workgroups per CU on 256 CUs
    // A descriptor with at least as many work items (one split each) as its
    // share of the target keeps that many; the rest of the target is shared by
    // the others in proportion to their bytes, so that the launch stays within
    // what the chip holds at once (a second wave of workgroups would start the
    // longest items late).
    // A fused step's token takes a split of its own when its read launches alone
    // (the token's work runs beside the other splits); with several reads in the
    // launch the last split of each item takes it, so an unsplit read (a sliding
    // donor) stays without partials and a combine.
    int n_shared = 0;
    for (int i = 0; i < n; ++i) n_shared += own[i] ? 0 : 1;
    const bool fold = n_shared > 1;
    int fixed_wg = 0;
    double free_bytes = 0.0;
    bool fixed[KVQ_MAX_SHARED_GROUPS];
    for (int i = 0; i < n; ++i) {
        fixed[i] = false;
        if (own[i]) continue;
        const kvq_cache* c = rs[i].cache;
        const int rows = (rs[i].C == 1 ? rs[i].n_layers : rs[i].C) * (rs[i].Hq / c->n_kv_heads);
        // (a fused step's token as a split of its own takes one more workgroup per item)
        const int64_t items = (int64_t)c->batch * c->n_kv_heads * ((rows + kvq::kRowTile - 1) / kvq::kRowTile) *
                              (rs[i].k_new && !(fold && c->k_bits != 16) ? 2 : 1);
        fixed[i] = total > 0 && items >= kTargetWg * (bytes[i] / total);
        if (fixed[i]) fixed_wg += (int)std::min<int64_t>(items, kTargetWg);
        else free_bytes += bytes[i];
    }
    const int free_wg = std::max(kTargetWg / 4, kTargetWg - fixed_wg);
    total_items = 0;
    int comb = 0;
    size_t ws = 0;
    for (int i = 0; i < n; ++i) {
        kvq::AttnDesc& d = P.d[i];
        if (own[i]) {
            plan_codes_desc(rs[i], d);
            d.item_begin = 0;
        } else {
            const double share = fixed[i] ? 0.0 : (free_bytes > 0 ? bytes[i] / free_bytes : 1.0);
            const int target = std::max(1, (int)std::lround(free_wg * share));
            plan_read(rs[i], target, d, fold);
            d.item_begin = total_items;
            total_items += d.n_items;
        }
        d.comb_begin = comb;
        if (d.S > 1) comb += d.B * d.Hkv * d.n_rows * (d.D / 64);
        const size_t f = kvq::part_floats(d);
        ws = (ws + 255) & ~(size_t)255;
        if (f) ws += f * sizeof(float);
    }
    return ws;
}

void bind_workspace(kvq::AttnParams& P, void* workspace)
{
    size_t off = 0;
    for (int i = 0; i < P.n_desc; ++i) {
        const size_t f = kvq::part_floats(P.d[i]);
        off = (off + 255) & ~(size_t)255;
        P.d[i].part = f ? reinterpret_cast<float*>(static_cast<char*>(workspace) + off) : nullptr;
        off += f * sizeof(float);
    }
}

kvq_status run_reads(const ReadSpec* rs, int n, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const char* what)
{
    kvq::AttnParams P;
    int total_items = 0;
    const size_t need = plan_all(rs, n, P, total_items);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KVQ_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", what, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", what);
    bind_workspace(P, workspace);
    // the reads that share one launch, renumbered; the others launch alone
    kvq::AttnParams Ps;
    std::memset(&Ps, 0, sizeof(Ps));
    for (int i = 0; i < n; ++i)
        if (!P.d[i].own_launch) Ps.d[Ps.n_desc++] = P.d[i];
    bool same = true, big = true;
    for (int i = 0; i < Ps.n_desc; ++i) {
        same &= Ps.d[i].cfg == Ps.d[0].cfg;
        big &= kvq::chunk_kernels_for(Ps.d[i].D) && !kvq::cfg_is_bf16(Ps.d[i].cfg);
    }
    auto launch_one = [&](const kvq::AttnParams& p, int items) {
        if (kvq::cfg_is_bf16(p.d[0].cfg)) return kvq::launch_attn_bf16(p, items, stream);
        if (p.n_desc == 1 && p.d[0].k_new && !p.d[0].tok_fold) return kvq::launch_attn_step(p, items, stream);
        return kvq::launch_attn(p, items, false, stream);
    };
    if (trace_on())
        for (int i = 0; i < n; ++i)
            fprintf(stderr, "[kvq] %s desc %d%s: B=%d Hkv=%d Hq=%d D=%d R=%d W=%d C=%d rows=%d tiles=%d S=%d split=%d wg=%d\n",
                    what, i, P.d[i].own_launch ? " (short-chunk kernel)" : "", P.d[i].B, P.d[i].Hkv, P.d[i].Hq,
                    P.d[i].D, P.d[i].R, P.d[i].W, P.d[i].C, P.d[i].n_rows, P.d[i].n_rt, P.d[i].S,
                    P.d[i].split_len, P.d[i].n_items);
    hipError_t e = hipSuccess;
    mark_before(stream);
    if (Ps.n_desc == 0) {
        // every read runs in a launch of its own
    } else if (same) {
        e = launch_one(Ps, total_items);
    } else if (big) {
        e = kvq::launch_attn(Ps, total_items, true, stream);
    } else {
        // Mixed configurations outside the fused set: one launch per descriptor.
        for (int i = 0; i < Ps.n_desc && e == hipSuccess; ++i) {
            kvq::AttnParams one;
            std::memset(&one, 0, sizeof(one));
            one.n_desc = 1;
            one.d[0] = Ps.d[i];
            one.d[0].item_begin = 0;
            e = launch_one(one, Ps.d[i].n_items);
        }
    }
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        if (!P.d[i].own_launch) continue;
        kvq::AttnParams one;
        std::memset(&one, 0, sizeof(one));
        one.n_desc = 1;
        one.d[0] = P.d[i];
        e = kvq::launch_prefill_codes(one, P.d[i].n_items, stream);
    }
    mark_after(stream);
    if (e == hipSuccess) e = kvq::launch_combine(P, stream);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
kvq_status static_scratch(void** ptr, const char* what)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVQ_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", what, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVQ_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", what,
                        dev, hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return KVQ_OK;
}

}  // namespace

namespace kvq {
bool read_marks(hipEvent_t& start, hipEvent_t& stop)
{
    start = g_kstart;
    stop = g_kstop;
    g_kstart = nullptr;
    return start != nullptr || stop != nullptr;
}
}  // namespace kvq

KVQ_API const char* kvq_last_error(void) { return g_err; }

KVQ_API kvq_status kvq_mark_next_read(hipEvent_t before, hipEvent_t after)
{
    g_mark_before = before;
    g_mark_after = after;
    return ok();
}

// The launch parameters of an append of T tokens (T > 0); a non-OK status (with
// a message) when an argument is invalid.
static kvq_status append_params(const kvq_cache* cache, const float* k, const float* v, int32_t T,
                                const int32_t* pos0, const char* what, kvq::AppendParams& p, int& n_cand)
{
    if (!k || !v || !pos0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k, v or pos0 is NULL", what);
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k and v must be 16-byte aligned", what);
    p.k = k;
    p.v = v;
    p.k_codes = cache->k_codes;
    p.v_codes = cache->v_codes;
    p.k_sb = cache->k_sb;
    p.v_sb = cache->v_sb;
    p.pos0 = pos0;
    p.B = cache->batch;
    p.H = cache->n_kv_heads;
    p.T = T;
    p.D = cache->head_dim;
    p.R = cache->capacity;
    p.k_bits = cache->k_bits;
    p.v_bits = cache->v_bits;
    p.t_first = T > p.R ? T - p.R : 0;
    p.n_written = T - p.t_first;
    n_cand = std::min(p.R / 8, (p.n_written + 7) / 8 + 1);
    if (2 * (int64_t)p.B > 65535) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch %d too large", what, p.B);
    return KVQ_OK;
}

KVQ_API kvq_status kvq_append_quantize(const kvq_cache* cache, const float* k, const float* v,
                                       int32_t T, const int32_t* pos0, hipStream_t stream)
{
    const char* what = "kvq_append_quantize";
    kvq_status st = check_cache(cache, what);
    if (st != KVQ_OK) return st;
    if (T < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: T %d < 0", what, T);
    if (T == 0) return ok();
    kvq::AppendParams p;
    int n_cand = 0;
    st = append_params(cache, k, v, T, pos0, what, p, n_cand);
    if (st != KVQ_OK) return st;
    if (cache->k_bits == 16) {                    // bf16 cache: round and store, no quantizer
        if (trace_on())
            fprintf(stderr, "[kvq] %s (bf16): B=%d H=%d T=%d D=%d R=%d\n", what, p.B, p.H, T, p.D, p.R);
        const hipError_t e = kvq::launch_append_bf16(p, stream);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
        return ok();
    }
    if (trace_on())
        fprintf(stderr, "[kvq] %s: B=%d H=%d T=%d D=%d R=%d bits=%d/%d blocks=%d\n", what, p.B, p.H, T, p.D, p.R,
                p.k_bits, p.v_bits, n_cand);
    const hipError_t e = kvq::launch_append(p, n_cand, stream);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

KVQ_API kvq_status kvq_append_quantize_multi(const kvq_append_item* items, int32_t n_items, hipStream_t stream)
{
    const char* what = "kvq_append_quantize_multi";
    if (!items) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: items is NULL", what);
    if (n_items < 1 || n_items > KVQ_MAX_SHARED_GROUPS)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_items %d outside [1, %d]", what, n_items,
                    KVQ_MAX_SHARED_GROUPS);
    kvq::AppendMulti P;
    kvq::AppendParams bf[KVQ_MAX_SHARED_GROUPS];
    int n_bf = 0;
    int64_t blocks = 0;
    P.n = 0;
    for (int i = 0; i < n_items; ++i) {
        const kvq_append_item& it = items[i];
        kvq_status st = check_cache(it.cache, what);
        if (st != KVQ_OK) return st;
        if (it.T < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: item %d: T %d < 0", what, i, it.T);
        for (int j = 0; j < i; ++j)
            if (items[j].cache->k_codes == it.cache->k_codes || items[j].cache->v_codes == it.cache->v_codes)
                return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: items %d and %d write the same cache", what, j, i);
        if (it.T == 0) continue;
        kvq::AppendParams p;
        int n_cand = 0;
        st = append_params(it.cache, it.k, it.v, it.T, it.pos0, what, p, n_cand);
        if (st != KVQ_OK) return st;
        if (it.cache->k_bits == 16) {
            bf[n_bf++] = p;
            continue;
        }
        P.a[P.n] = p;
        P.n_cand[P.n] = n_cand;
        P.block_begin[P.n] = (int32_t)blocks;
        blocks += (int64_t)n_cand * p.H * 2 * p.B;
        if (blocks > INT_MAX) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: too many blocks in one launch", what);
        ++P.n;
    }
    P.block_begin[P.n] = (int32_t)blocks;
    if (trace_on())
        fprintf(stderr, "[kvq] %s: %d quantized caches in %lld blocks, %d bf16 caches\n", what, P.n,
                (long long)blocks, n_bf);
    if (P.n > 0) {
        const hipError_t e = kvq::launch_append_multi(P, stream);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    }
    for (int i = 0; i < n_bf; ++i) {
        const hipError_t e = kvq::launch_append_bf16(bf[i], stream);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    }
    return ok();
}

KVQ_API kvq_status kvq_append_norm_quantize(const kvq_cache* cache, const float* k, const float* v,
                                            int32_t T, const int32_t* pos0, const float* k_weight, float eps,
                                            const float* rope_cos, const float* rope_sin, int32_t rope_dims,
                                            int32_t rope_positions, float* k_out, float* v_out,
                                            hipStream_t stream)
{
    const char* what = "kvq_append_norm_quantize";
    kvq_status st = check_cache(cache, what);
    if (st != KVQ_OK) return st;
    if (T < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: T %d < 0", what, T);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", what);
    if (rope_dims < 0 || rope_dims % 2 != 0 || rope_dims > cache->head_dim)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: rope_dims %d must be even and in [0, head_dim %d]", what,
                    rope_dims, cache->head_dim);
    if (rope_dims > 0 && (!rope_cos || !rope_sin || rope_positions < 1))
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: a rotation needs both tables and rope_positions >= 1", what);
    if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k_out and v_out must be 16-byte aligned", what);
    if (T == 0) return ok();
    kvq::NormAppendParams P;
    int n_cand = 0;
    st = append_params(cache, k, v, T, pos0, what, P.a, n_cand);
    if (st != KVQ_OK) return st;
    P.k_weight = k_weight;
    P.eps = eps;
    P.rope_cos = rope_dims > 0 ? rope_cos : nullptr;
    P.rope_sin = rope_dims > 0 ? rope_sin : nullptr;
    P.rope_half = rope_dims / 2;
    P.rope_positions = rope_dims > 0 ? rope_positions : 0;
    P.k_out = k_out;
    P.v_out = v_out;
    if (trace_on())
        fprintf(stderr, "[kvq] %s: B=%d H=%d T=%d D=%d R=%d bits=%d/%d rope=%d blocks=%d\n", what, P.a.B, P.a.H, T,
                P.a.D, P.a.R, P.a.k_bits, P.a.v_bits, rope_dims, n_cand);
    const hipError_t e = kvq::launch_append_norm(P, n_cand, stream);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ReadSpecs of a mixed launch; a non-OK status (with a message) when a read is
// invalid.  sizing: only what the workspace query can check (no pointers).
static kvq_status mixed_specs(const kvq_read* reads, int32_t n, ReadSpec* rs, const char* what, bool sizing)
{
    if (!reads) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: reads is NULL", what);
    if (n < 1 || n > KVQ_MAX_SHARED_GROUPS)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_reads %d outside [1, %d]", what, n, KVQ_MAX_SHARED_GROUPS);
    for (int i = 0; i < n; ++i) {
        const kvq_read& g = reads[i];
        if (g.chunk < 1) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: read %d: chunk %d < 1", what, i, g.chunk);
        if (g.chunk > 1 && g.n_layers != 1)
            return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: read %d: a chunk of %d queries needs n_layers == 1",
                        what, i, g.chunk);
        rs[i] = ReadSpec{g.cache, g.n_layers, g.q, g.out, g.n_q_heads, g.scale, g.len, g.max_len, g.chunk};
        kvq_status st;
        if (sizing) {
            st = check_cache(g.cache, what);
            if (st == KVQ_OK && (g.n_layers < 1 || g.n_layers > KVQ_MAX_SHARED_LAYERS || g.n_q_heads < 1 ||
                                 g.n_q_heads % g.cache->n_kv_heads != 0 || g.max_len < g.chunk))
                st = KVQ_ERR_INVALID_ARGUMENT;
        } else {
            st = check_read(rs[i], what);
        }
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

KVQ_API size_t kvq_decode_workspace_bytes(const kvq_shared_group* groups, int32_t n_groups)
{
    if (!groups || n_groups < 1 || n_groups > KVQ_MAX_SHARED_GROUPS) return SIZE_MAX;
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    for (int i = 0; i < n_groups; ++i) {
        const kvq_shared_group& g = groups[i];
        rs[i] = ReadSpec{g.cache, g.n_layers, g.q, g.out, g.n_q_heads, g.scale, g.len, g.max_len, 1};
        // Pointer arrays are not needed for sizing.
        if (check_cache(g.cache, "kvq_decode_workspace_bytes") != KVQ_OK) return SIZE_MAX;
        if (g.n_layers < 1 || g.n_layers > KVQ_MAX_SHARED_LAYERS || g.n_q_heads < 1 ||
            g.n_q_heads % g.cache->n_kv_heads != 0 || g.max_len < 1)
            return SIZE_MAX;
    }
    kvq::AttnParams P;
    int total = 0;
    return plan_all(rs, n_groups, P, total);
}

// Band positions per (b, kv head): every position a query of the chunk can see,
// from a step-aligned start.
int64_t band_positions(const kvq_cache* c, int chunk, int max_len)
{
    const int64_t span = c->window > 0 ? std::min<int64_t>((int64_t)c->window + chunk - 1, max_len) : max_len;
    return (span + 2 * kvq::kStep - 1) / kvq::kStep * kvq::kStep;
}

// A bf16 cache's chunk is read by the attention kernel straight from the cache
// (no band copy) when every byte offset inside one (sequence, KV head) fits the
// kernel's unsigned 32-bit DMA offsets; KVQ_BF16_BAND=1 forces the band copy
// (measurement).
bool band_direct(int cfg, int R, int D)
{
    if (!kvq::cfg_is_bf16(cfg)) return false;
    const char* e = getenv("KVQ_BF16_BAND");
    if (e && e[0] == '1') return false;
    return (int64_t)R * D * 2 < ((int64_t)1 << 31);
}

size_t plan_prefill(const ReadSpec& r, kvq::AttnParams& P, int& total_items)
{
    std::memset(&P, 0, sizeof(P));
    P.n_desc = 1;
    plan_read(r, 1, P.d[0]);                      // shape fields
    kvq::AttnDesc& d = P.d[0];
    const kvq_cache* c = r.cache;
    const int n_rb = (d.n_rows + kvq::kPrefillRows - 1) / kvq::kPrefillRows;
    int64_t vis = r.max_len;
    if (c->window > 0)
        vis = std::min<int64_t>(vis, (int64_t)c->window + (kvq::kPrefillRows + d.hpk - 1) / d.hpk);
    const int64_t steps = (vis + 2 * kvq::kStep - 1) / kvq::kStep;
    const int64_t items = (int64_t)d.B * d.Hkv * n_rb;
    const int kTargetWg = 128;     // workgroups to reach before splitting keys (a split adds a combine)
    int64_t S = (kTargetWg + items - 1) / items;
    const int forced = env_splits();
    if (forced > 0) S = forced;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(steps, kvq::kMaxSplits)));
    const int64_t steps_per = (steps + S - 1) / S;
    d.split_len = (int)(steps_per * kvq::kStep);
    d.S = (int)((steps + steps_per - 1) / steps_per);
    d.n_items = (int)(items * d.S);
    d.item_begin = 0;
    d.comb_begin = 0;
    d.nk = (int)band_positions(c, r.C, r.max_len);
    total_items = d.n_items;
    // workspace: split partials, then the band tiles (K and V, bf16; four spare
    // tiles per sequence and KV head that a final prefetch may read)
    const size_t part = (kvq::part_floats(d) * sizeof(float) + 255) & ~(size_t)255;
    if (band_direct(d.cfg, d.R, d.D)) return part;
    return part + (size_t)d.B * d.Hkv * (d.nk + 4 * kvq::kStep) * d.D * 2 * sizeof(uint16_t);
}

// Quantized caches, chunks of more than 64 rows per KV head (head_dim 256/512):
// one workgroup per (b, kv head, 32-row block, split) of the fused kernel, which
// reads the codes itself; the workspace holds the split partials only.
size_t plan_qprefill(const ReadSpec& r, kvq::AttnParams& P, int& total_items)
{
    std::memset(&P, 0, sizeof(P));
    P.n_desc = 1;
    plan_read(r, 1, P.d[0]);                      // shape fields (n_rt counts 16-row tiles)
    kvq::AttnDesc& d = P.d[0];
    const kvq_cache* c = r.cache;
    const int n_rb = (d.n_rows + kvq::kQprefillRows - 1) / kvq::kQprefillRows;
    int64_t vis = r.max_len;
    if (c->window > 0)
        vis = std::min<int64_t>(vis, (int64_t)c->window + (kvq::kQprefillRows + d.hpk - 1) / d.hpk);
    const int64_t steps = (vis + 2 * kvq::kStep - 1) / kvq::kStep;
    const int64_t items = (int64_t)d.B * d.Hkv * n_rb;
    // one workgroup per CU (each holds a wave per SIMD); split keys only below that
    const int kTargetWg = 256;
    int64_t S = (kTargetWg + items - 1) / items;
    const int forced = env_splits();
    if (forced > 0) S = forced;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>((steps + 3) / 4, kvq::kMaxSplits)));
    const int64_t steps_per = (steps + S - 1) / S;
    d.split_len = (int)(steps_per * kvq::kStep);
    d.S = (int)((steps + steps_per - 1) / steps_per);
    d.n_items = (int)(items * d.S);
    total_items = d.n_items;
    return kvq::part_floats(d) * sizeof(float);
}

// Short-chunk kernel: one workgroup per (b, kv head, 64-row block, split); the
// workspace holds the split partials only.
size_t plan_codes(const ReadSpec& r, kvq::AttnParams& P, int& total_items)
{
    std::memset(&P, 0, sizeof(P));
    P.n_desc = 1;
    kvq::AttnDesc& d = P.d[0];
    plan_codes_desc(r, d);
    d.own_launch = 0;                             // the only descriptor of its launch
    total_items = d.n_items;
    return kvq::part_floats(d) * sizeof(float);
}

void bind_prefill_workspace(kvq::AttnParams& P, void* workspace)
{
    kvq::AttnDesc& d = P.d[0];
    char* base = static_cast<char*>(workspace);
    const size_t part = (kvq::part_floats(d) * sizeof(float) + 255) & ~(size_t)255;
    d.part = kvq::part_floats(d) ? reinterpret_cast<float*>(base) : nullptr;
    d.band = band_direct(d.cfg, d.R, d.D) ? nullptr : reinterpret_cast<uint16_t*>(base + part);
}

KVQ_API size_t kvq_prefill_workspace_bytes(const kvq_cache* cache, int32_t n_q_heads, int32_t chunk, int32_t max_len)
{
    if (check_cache(cache, "kvq_prefill_workspace_bytes") != KVQ_OK) return SIZE_MAX;
    if (n_q_heads < 1 || n_q_heads % cache->n_kv_heads != 0 || chunk < 1 || max_len < chunk) return SIZE_MAX;
    ReadSpec r{cache, 1, nullptr, nullptr, n_q_heads, 1.0f, nullptr, max_len, chunk};
    kvq::AttnParams P;
    int total = 0;
    switch (chunk_path(cache, n_q_heads, chunk, max_len)) {
    case ChunkPath::kBand: return kvq::cfg_is_bf16(kvq::cfg_id(cache->head_dim, cache->k_bits, cache->v_bits))
                                      ? plan_prefill(r, P, total) : plan_qprefill(r, P, total);
    case ChunkPath::kCodes: return plan_codes(r, P, total);
    default: return plan_all(&r, 1, P, total);
    }
}

KVQ_API kvq_status kvq_attn_decode(const kvq_cache* cache, const uint16_t* q, int32_t n_q_heads,
                                   const int32_t* len, int32_t max_len, float scale, uint16_t* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_attn_decode";
    const uint16_t* qs[1] = {q};
    uint16_t* os[1] = {out};
    ReadSpec r{cache, 1, qs, os, n_q_heads, scale, len, max_len, 1};
    kvq_status st = check_read(r, what);
    if (st != KVQ_OK) return st;
    return run_reads(&r, 1, workspace, workspace_bytes, stream, what);
}

KVQ_API kvq_status kvq_attn_decode_static(const kvq_cache* cache, const uint16_t* q, int32_t n_q_heads,
                                          const int32_t* len, int32_t max_len, float scale, uint16_t* out,
                                          hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_attn_decode_static";
    const uint16_t* qs[1] = {q};
    uint16_t* os[1] = {out};
    ReadSpec r{cache, 1, qs, os, n_q_heads, scale, len, max_len, 1};
    kvq_status st = check_read(r, what);
    if (st != KVQ_OK) return st;
    kvq::AttnParams P;
    int total = 0;
    const size_t need = plan_all(&r, 1, P, total);
    if (need > (size_t)KVQ_STATIC_SCRATCH_BYTES)
        return fail(KVQ_ERR_WORKSPACE, "%s: this read needs %zu bytes of split partials, more than the %d-byte "
                    "static scratch; use kvq_attn_decode with a workspace", what, need, KVQ_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
        st = static_scratch(&ws, what);
        if (st != KVQ_OK) return st;
    }
    return run_reads(&r, 1, ws, KVQ_STATIC_SCRATCH_BYTES, stream, what);
}

KVQ_API size_t kvq_decode_step_workspace_bytes(const kvq_cache* cache, int32_t n_q_heads, int32_t max_len)
{
    if (check_cache(cache, "kvq_decode_step_workspace_bytes") != KVQ_OK) return SIZE_MAX;
    if (n_q_heads < 1 || n_q_heads % cache->n_kv_heads != 0 || max_len < 1) return SIZE_MAX;
    static const float dummy = 0.0f;
    ReadSpec r{cache, 1, nullptr, nullptr, n_q_heads, 1.0f, nullptr, max_len, 1, &dummy, &dummy};
    kvq::AttnParams P;
    int total = 0;
    return plan_all(&r, 1, P, total);
}

KVQ_API kvq_status kvq_decode_step(const kvq_cache* cache, const float* k, const float* v,
                                   const uint16_t* q, int32_t n_q_heads,
                                   const int32_t* len, int32_t max_len, float scale,
                                   uint16_t* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_decode_step";
    const uint16_t* qs[1] = {q};
    uint16_t* os[1] = {out};
    ReadSpec r{cache, 1, qs, os, n_q_heads, scale, len, max_len, 1, k, v};
    kvq_status st = check_read(r, what);
    if (st != KVQ_OK) return st;
    if (!k || !v) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k or v is NULL", what);
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k and v must be 16-byte aligned", what);
    return run_reads(&r, 1, workspace, workspace_bytes, stream, what);
}

KVQ_API kvq_status kvq_attn_prefill_chunk(const kvq_cache* cache, const uint16_t* q, int32_t n_q_heads,
                                          int32_t chunk, const int32_t* len, int32_t max_len, float scale,
                                          uint16_t* out, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_attn_prefill_chunk";
    const uint16_t* qs[1] = {q};
    uint16_t* os[1] = {out};
    ReadSpec r{cache, 1, qs, os, n_q_heads, scale, len, max_len, chunk};
    kvq_status st = check_read(r, what);
    if (st != KVQ_OK) return st;
    const ChunkPath path = chunk_path(cache, n_q_heads, chunk, max_len);
    if (path == ChunkPath::kDecode) return run_reads(&r, 1, workspace, workspace_bytes, stream, what);
    kvq::AttnParams P;
    int total_items = 0;
    const bool quant_band = path == ChunkPath::kBand && cache->k_bits != 16;
    const size_t need = quant_band ? plan_qprefill(r, P, total_items)
                        : path == ChunkPath::kBand ? plan_prefill(r, P, total_items) : plan_codes(r, P, total_items);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KVQ_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", what, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", what);
    if (quant_band) {
        P.d[0].part = kvq::part_floats(P.d[0]) ? static_cast<float*>(workspace) : nullptr;
        if (trace_on())
            fprintf(stderr, "[kvq] %s quantized prefill kernel: B=%d Hkv=%d Hq=%d D=%d R=%d W=%d C=%d rows=%d S=%d "
                    "split=%d wg=%d\n", what, P.d[0].B, P.d[0].Hkv, P.d[0].Hq, P.d[0].D, P.d[0].R, P.d[0].W,
                    P.d[0].C, P.d[0].n_rows, P.d[0].S, P.d[0].split_len, total_items);
        mark_before(stream);
        hipError_t e = kvq::launch_qprefill(P, total_items, stream);
        mark_after(stream);
        if (e == hipSuccess) e = kvq::launch_combine(P, stream);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
        return ok();
    }
    if (path == ChunkPath::kCodes) {
        P.d[0].part = kvq::part_floats(P.d[0]) ? static_cast<float*>(workspace) : nullptr;
        if (trace_on())
            fprintf(stderr, "[kvq] %s short-chunk kernel: B=%d Hkv=%d Hq=%d D=%d C=%d rows=%d S=%d split=%d wg=%d\n",
                    what, P.d[0].B, P.d[0].Hkv, P.d[0].Hq, P.d[0].D, P.d[0].C, P.d[0].n_rows, P.d[0].S,
                    P.d[0].split_len, total_items);
        mark_before(stream);
        hipError_t e = kvq::launch_prefill_codes(P, total_items, stream);
        mark_after(stream);
        if (e == hipSuccess) e = kvq::launch_combine(P, stream);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
        return ok();
    }
    bind_prefill_workspace(P, workspace);
    if (trace_on())
        fprintf(stderr, "[kvq] %s prefill kernel: B=%d Hkv=%d Hq=%d D=%d R=%d W=%d C=%d rows=%d S=%d split=%d wg=%d band=%d\n",
                what, P.d[0].B, P.d[0].Hkv, P.d[0].Hq, P.d[0].D, P.d[0].R, P.d[0].W, P.d[0].C, P.d[0].n_rows,
                P.d[0].S, P.d[0].split_len, total_items, P.d[0].nk);
    hipError_t e = kvq::launch_band(P, stream);
    if (e == hipSuccess) {
        mark_before(stream);
        e = kvq::launch_prefill(P, total_items, stream);
        mark_after(stream);
    }
    if (e == hipSuccess) e = kvq::launch_combine(P, stream);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

KVQ_API size_t kvq_mixed_workspace_bytes(const kvq_read* reads, int32_t n_reads)
{
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    if (mixed_specs(reads, n_reads, rs, "kvq_mixed_workspace_bytes", true) != KVQ_OK) return SIZE_MAX;
    kvq::AttnParams P;
    int total = 0;
    return plan_all(rs, n_reads, P, total);
}

KVQ_API kvq_status kvq_attn_mixed(const kvq_read* reads, int32_t n_reads, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_attn_mixed";
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    kvq_status st = mixed_specs(reads, n_reads, rs, what, false);
    if (st != KVQ_OK) return st;
    return run_reads(rs, n_reads, workspace, workspace_bytes, stream, what);
}

KVQ_API kvq_status kvq_attn_decode_shared(const kvq_shared_group* groups, int32_t n_groups,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_attn_decode_shared";
    if (!groups) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: groups is NULL", what);
    if (n_groups < 1 || n_groups > KVQ_MAX_SHARED_GROUPS)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_groups %d outside [1, %d]", what, n_groups, KVQ_MAX_SHARED_GROUPS);
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    for (int i = 0; i < n_groups; ++i) {
        const kvq_shared_group& g = groups[i];
        rs[i] = ReadSpec{g.cache, g.n_layers, g.q, g.out, g.n_q_heads, g.scale, g.len, g.max_len, 1};
        kvq_status st = check_read(rs[i], what);
        if (st != KVQ_OK) return st;
    }
    return run_reads(rs, n_groups, workspace, workspace_bytes, stream, what);
}

// ReadSpecs of a fused shared step; a non-OK status (with a message) when an
// argument is invalid.  sizing: only what the workspace query can check.
static kvq_status step_shared_specs(const kvq_shared_group* groups, int32_t n, const float* const* k,
                                    const float* const* v, ReadSpec* rs, const char* what, bool sizing)
{
    static const float dummy = 0.0f;
    if (!groups) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: groups is NULL", what);
    if (n < 1 || n > KVQ_MAX_SHARED_GROUPS)
        return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: n_groups %d outside [1, %d]", what, n, KVQ_MAX_SHARED_GROUPS);
    if (!sizing && (!k || !v)) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: k or v is NULL", what);
    for (int i = 0; i < n; ++i) {
        const kvq_shared_group& g = groups[i];
        const float* ki = sizing ? &dummy : k[i];
        const float* vi = sizing ? &dummy : v[i];
        rs[i] = ReadSpec{g.cache, g.n_layers, g.q, g.out, g.n_q_heads, g.scale, g.len, g.max_len, 1, ki, vi};
        kvq_status st;
        if (sizing) {
            st = check_cache(g.cache, what);
            if (st == KVQ_OK && (g.n_layers < 1 || g.n_layers > KVQ_MAX_SHARED_LAYERS || g.n_q_heads < 1 ||
                                 g.n_q_heads % g.cache->n_kv_heads != 0 || g.max_len < 1))
                st = fail(KVQ_ERR_INVALID_ARGUMENT, "%s: group %d: invalid read", what, i);
        } else {
            st = check_read(rs[i], what);
        }
        if (st != KVQ_OK) return st;
        if (!sizing) {
            if (!ki || !vi) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: group %d: k or v is NULL", what, i);
            if ((reinterpret_cast<uintptr_t>(ki) | reinterpret_cast<uintptr_t>(vi)) & 15)
                return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: group %d: k and v must be 16-byte aligned", what, i);
        }
        // each group appends to its own cache: two groups on one cache would write
        // the same slot twice
        for (int j = 0; j < i; ++j)
            if (groups[j].cache->k_codes == g.cache->k_codes)
                return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: groups %d and %d share a cache", what, j, i);
    }
    return KVQ_OK;
}

KVQ_API size_t kvq_decode_step_shared_workspace_bytes(const kvq_shared_group* groups, int32_t n_groups)
{
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    if (step_shared_specs(groups, n_groups, nullptr, nullptr, rs, "kvq_decode_step_shared_workspace_bytes", true) !=
        KVQ_OK)
        return SIZE_MAX;
    kvq::AttnParams P;
    int total = 0;
    return plan_all(rs, n_groups, P, total);
}

KVQ_API kvq_status kvq_decode_step_shared(const kvq_shared_group* groups, int32_t n_groups, const float* const* k,
                                          const float* const* v, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream)
{
    MarkScope marks;
    const char* what = "kvq_decode_step_shared";
    ReadSpec rs[KVQ_MAX_SHARED_GROUPS];
    const kvq_status st = step_shared_specs(groups, n_groups, k, v, rs, what, false);
    if (st != KVQ_OK) return st;
    return run_reads(rs, n_groups, workspace, workspace_bytes, stream, what);
}

// Launch parameter blocks shared by the host API and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

struct AppendParams {
    const float* k;
    const float* v;
    uint32_t* k_codes;
    uint32_t* v_codes;
    uint32_t* k_sb;
    uint32_t* v_sb;
    const int32_t* pos0;
    int32_t B, H, T, D, R;
    int32_t k_bits, v_bits;
    int32_t t_first;      // first token written (T > R keeps the last R)
    int32_t n_written;    // tokens written per sequence
};

// Appends of several caches in one launch: cache i takes blocks
// [block_begin[i], block_begin[i+1]), n_cand[i] x H x 2B of them.
struct AppendMulti {
    AppendParams a[KVQ_MAX_SHARED_GROUPS];
    int32_t n_cand[KVQ_MAX_SHARED_GROUPS];
    int32_t block_begin[KVQ_MAX_SHARED_GROUPS + 1];
    int32_t n;
};

// The append with the keys' and values' norms and the keys' rotation in front.
struct NormAppendParams {
    AppendParams a;
    const float* k_weight;     // [D] or null (un-scaled)
    float eps;
    const float* rope_cos;     // [rope_positions][rope_half]
    const float* rope_sin;
    int32_t rope_half;         // rotated pairs per row (0: no rotation)
    int32_t rope_positions;
    float* k_out;              // [B][H][T][D] normed (rotated) rows, or null
    float* v_out;
};

// Rows of one (sequence, KV head) pair are the query rows that read it:
//   decode / shared: row = layer * hpk + h   (hpk = Hq / Hkv query heads per KV head)
//   prefill:         row = i * hpk + h       (i = query index in the chunk)
// Rows are processed in tiles of 16; a work item is (b, kv head, row tile, split).
constexpr int kRowTile = 16;
constexpr int kStep = 32;          // keys per inner step
constexpr int kMaxSplits = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnDesc {
    const uint32_t* k_codes;
    const uint32_t* v_codes;
    const uint32_t* k_sb;
    const uint32_t* v_sb;
    const uint16_t* q[KVQ_MAX_SHARED_LAYERS];
    uint16_t* out[KVQ_MAX_SHARED_LAYERS];
    const int32_t* len;
    const float* k_new;     // fused decode step: the step's fp32 K and V rows [B][Hkv][D]
    const float* v_new;     //   (null otherwise); split S-1 of every item takes that token
                            //   (see tok_fold)
    int32_t excl;           // 1: the attention splits leave out position len-1 (fused step)
    int32_t tok_fold;       // fused step on a quantized cache: 1 the last split takes the
                            //   token after its keys (no extra split), 0 a split of its own
    float* part;            // split partials (null when S == 1)
    uint16_t* band;         // prefill: dequantized band tiles, bf16 [B][Hkv][nk/32][64*D] (the
                            // LDS image of each 32-key step: K rows, then V^T rows, swizzled);
                            // null for a bf16 cache that the attention kernel reads in place
    int32_t nk;             // prefill: band positions held per (b, kv head), a multiple of 32
    int32_t B, Hkv, Hq, R, W, C, D;
    int32_t max_len;        // len[b] is clamped to [0, max_len]
    int32_t hpk, n_rows, n_rt;
    int32_t n_layers;       // layers whose queries share the read (1 for prefill)
    int32_t S, split_len;   // splits per (b, kv head, row tile) and keys per split
    int32_t item_begin;     // first workgroup of this descriptor
    int32_t n_items;        // B * Hkv * n_rt * S
    int32_t comb_begin;     // first combine workgroup of this descriptor (S > 1)
    float scale_log2e;
    int32_t cfg;            // kernel configuration id (head_dim, k_bits, v_bits)
    int32_t own_launch;     // host: a short chunk of a mixed launch, read by the codes
                            // kernel in a launch of its own (items counted from 0)
    int32_t part_h;         // split partials of o hold o / l as fp16 (the short-chunk kernel,
                            // whose V values are fp16 already); else o as fp32
};

struct AttnParams {
    AttnDesc d[KVQ_MAX_SHARED_GROUPS];
    int32_t n_desc;
};

// Configuration id: 0..31 quantized (head_dim 64..512 in steps of 64, k_bits,
// v_bits); 32 + head_dim/64 - 1 for bf16 caches.
constexpr int cfg_of(int D, int kb, int vb)
{
    return kb == 16 ? 32 + D / 64 - 1 : (D / 64 - 1) * 4 + (kb == 8 ? 2 : 0) + (vb == 8 ? 1 : 0);
}
inline int cfg_id(int D, int kb, int vb) { return cfg_of(D, kb, vb); }
inline bool cfg_is_bf16(int cfg) { return cfg >= 32; }
// The chunk kernels (band and short-chunk) and the two-configuration decode
// launch exist for the model's head_dims; every other read takes the decode kernel.
inline bool chunk_kernels_for(int D) { return D == 256 || D == 512; }

// Partial buffer of one descriptor: o [B*Hkv*n_rt][S][16][D] fp32 (or o / l as
// fp16 in the first half of that space, part_h), then (m, l) [B*Hkv*n_rt][S][16][2]
// fp32.
inline size_t part_floats(const AttnDesc& d)
{
    if (d.S <= 1) return 0;
    const size_t items = (size_t)d.B * d.Hkv * d.n_rt * d.S * kRowTile;
    return items * (size_t)d.D + items * 2;
}

// Measurement marks (kvq_mark_next_read).  While a call's marks are armed, its
// read kernels launch with the start event attached to the first and the stop
// event to each (the last one stands), on the kernels themselves
// (hipExtLaunchKernel): the pair brackets their execution, not the dispatch gaps
// around them.  read_marks hands out the armed events (the start once).
bool read_marks(hipEvent_t& start, hipEvent_t& stop);

template <class K>
hipError_t launch_read(K kernel, dim3 grid, dim3 block, const AttnParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<AttnParams*>(&p)};
    hipEvent_t start = nullptr, stop = nullptr;
    if (read_marks(start, stop))
        return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream, start, stop, 0);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

hipError_t launch_append(const AppendParams& p, int n_cand, hipStream_t stream);
hipError_t launch_append_bf16(const AppendParams& p, hipStream_t stream);
hipError_t launch_append_multi(const AppendMulti& p, hipStream_t stream);
hipError_t launch_append_norm(const NormAppendParams& p, int n_cand, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnParams& p, int total_items, hipStream_t stream);
hipError_t launch_attn(const AttnParams& p, int total_items, bool multi, hipStream_t stream);
// the fused decode step of one descriptor (its k_new set)
hipError_t launch_attn_step(const AttnParams& p, int total_items, hipStream_t stream);
hipError_t launch_combine(const AttnParams& p, hipStream_t stream);
// The chunk's band tiles (dequantized, or a bf16 copy) when the prefill kernel
// needs them; then the prefill kernel itself.
hipError_t launch_band(const AttnParams& p, hipStream_t stream);
hipError_t launch_prefill(const AttnParams& p, int total_items, hipStream_t stream);
hipError_t launch_prefill_codes(const AttnParams& p, int total_items, hipStream_t stream);
// Chunks over quantized caches: the fused kernel (32-row items, codes read in place).
hipError_t launch_qprefill(const AttnParams& p, int total_items, hipStream_t stream);
constexpr int kQprefillRows = 32;

// Query rows per prefill workgroup (two 16-row tiles).
constexpr int kPrefillRows = 32;
// Query rows per workgroup of the short-chunk kernel (4 waves x 16 rows): a chunk
// with at most this many rows per KV head reads each key once.
constexpr int kCodesPrefillRows = 64;

}  // namespace kvq

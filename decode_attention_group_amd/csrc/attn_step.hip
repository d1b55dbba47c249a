// The fused decode step of one descriptor (page 80 of the @mlx-bun/inference
// 0.0.0-stage -> 1.0.0 diff, gemma4/model.ts attentionTraining: appendWindow,
// then read.attend, in one launch): the split decode kernel built with the
// token as a split of its own (attn_impl.h), in a translation unit of its own
// so that it compiles beside the plain reads.
#include "attn_impl.h"

namespace kvq {

hipError_t launch_attn_step(const AttnParams& p, int total_items, hipStream_t stream)
{
    const dim3 grid(total_items);
    if (p.n_desc != 1 || p.d[0].k_new == nullptr || p.d[0].tok_fold) return hipErrorInvalidValue;
    switch (p.d[0].cfg) {
#define KVQ_CASE(D_, KB_, VB_) \
    case cfg_of(D_, KB_, VB_): \
        return launch_read(attn_kernel<D_, KB_, VB_, true, kTokSplit>, grid, dim3(64 * Shape<D_>::NW), p, stream);
#define KVQ_D(D_) KVQ_CASE(D_, 4, 4) KVQ_CASE(D_, 4, 8) KVQ_CASE(D_, 8, 4) KVQ_CASE(D_, 8, 8)
    KVQ_D(64) KVQ_D(128) KVQ_D(192) KVQ_D(256) KVQ_D(320) KVQ_D(384) KVQ_D(448) KVQ_D(512)
#undef KVQ_D
#undef KVQ_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq

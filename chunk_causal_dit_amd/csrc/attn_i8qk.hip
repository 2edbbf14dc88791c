// int8-QK variant of the round's attention (see include/wf.h). Workspace
// layout and launchers; the kernels land in this file.
#include "wf_internal.h"

namespace wf {

I8Layout i8_layout(const wf_kv_cache& kv, int n_inflight) {
  I8Layout L{};
  L.blocks_per_chunk = (kv.chunk_tokens + 127) / 128;
  return L;
}

hipError_t launch_attn_fwd_i8qk(const wf_kv_cache&, AttnParams&, void*, float, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace wf

// Internal launch interface of the 8-bit QK^T variant (MXFP8 keys): the
// kernels take the common parameter blocks plus the scale array of the
// MXFP8 key pool, whose codes travel in the k_pages field.
#pragma once

#include "wf_internal.h"

namespace wf {

// publish with K quantized to MXFP8: p.k_pages = E4M3 codes
// [pages][H][ps][D], k8_scales = E8M0 codes [pages][H][ps][D/32]
hipError_t launch_publish_mx(const PublishParams& p, void* k8_scales, hipStream_t stream);

// attention with the 8-bit QK^T: p.k_pages = E4M3 key codes, k8_scales as
// above; head_dim 128, bfloat16 Q / V / out
hipError_t launch_attn_mx(const AttnParams& p, const void* k8_scales, hipStream_t stream);

}  // namespace wf

// Internal launch interface of the QKV projection fused with the publish
// (qkv_gemm.hip), used by api.cpp.
#pragma once

#include "wf_internal.h"

namespace wf {

struct QkvParams {
  const uint16_t* x;          // [n_tok] rows of [hidden] (bf16)
  const uint16_t* w;          // [3*H*D][hidden] (bf16), one row per output feature
  const uint16_t* bias;       // nullable, [3*H*D]
  uint16_t* q_out;            // nullable: [n_tok] rows of [H][D]
  uint16_t* k_pages;          // [pages][H][ps][D]
  uint16_t* v_pages;          // [pages][H][D][ps]
  const int32_t* page_table;
  const int32_t* pos;         // [n_tok][3], nullable when !rope
  int* status;
  int64_t x_stride, q_stride; // elements between rows
  int32_t n_tok, hidden, dst_start, heads, ps_log2, num_pages;
  int32_t tok_tiles;          // ceil(n_tok / 256)
  int32_t feat_tiles;         // 128-feature tiles computed (2H without Q, 3H with)
  int32_t sec0;               // section of the first tile: 0 (Q) or 1 (K)
  int32_t rope;               // 0/1
  int32_t pair_axis[kMaxPairs];
  double pair_omega[kMaxPairs];
};

hipError_t launch_qkv_publish(const QkvParams& p, hipStream_t stream);

}  // namespace wf

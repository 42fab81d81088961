// Internal launch interface of the QKV projection fused with the publish
// (qkv_gemm.hip), used by api.cpp.
#pragma once

#include "wf_internal.h"

namespace wf {

constexpr int kQkvBlockFeat = 256;  // output features per block (two heads of 128)
constexpr int kQkvBlockTok = 256;   // tokens per block
#ifndef WF_QKV_FT
#define WF_QKV_FT 8
#endif
constexpr int kQkvFT = WF_QKV_FT;   // feature tiles per XCD chunk
constexpr int kQkvTT = 32 / kQkvFT; // token tiles per XCD chunk (32 blocks, one per CU)

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
  int32_t feat_tiles;         // ceil(computed heads / 2); computed heads: 2H without Q, 3H with
  int32_t sec0;               // section of the first computed head: 0 (Q) or 1 (K)
  int32_t rope;               // 0/1
  int32_t band0[4];           // first pair of the t, h, w sub-bands; band0[3] = D/2
  double pair_omega[kMaxPairs];
};

struct QkvTile {
  int ftile, ttile;
};

// Block -> (feature tile, token tile).  The hardware deals consecutive
// blocks to the 8 XCDs in turn, so block b runs on XCD x = b % 8 as the
// k-th block of that XCD, k = b / 8.  The work order is cut into chunks of
// 32 (kQkvFT feature tiles x kQkvTT token tiles): round r gives XCD x the
// chunk 8r + x, its 32 blocks k = 32r .. 32r+31 at once, so the blocks an
// XCD runs together share weight and hidden-state rows in its L2, and the 8
// XCDs work on 8 neighbouring chunks (the same token rows) at the same
// time, which keeps the rows they miss in the L2 few enough for the
// memory-side cache.  The blocks of the last, partial round and those past
// 8 * (nb / 8) take the rest of the work order in turn.
// The work order takes token tiles in groups of kQkvTT and, inside a group,
// feature tiles in chunks of kQkvFT, token tile fastest.
__host__ __device__ inline QkvTile qkv_tile(int b, int nb, int feat_tiles, int tok_tiles) {
  const int per = nb >> 3;            // blocks per XCD in the dealt part
  const int rounds = per >> 5;        // full rounds of 32 blocks per XCD
  int w = b;
  if (b < (per << 3)) {
    const int x = b & 7, k = b >> 3;
    w = (k < (rounds << 5)) ? (((k >> 5) << 8) + (x << 5) + (k & 31))
                            : ((rounds << 8) + ((k - (rounds << 5)) << 3) + x);
  }
  const int group_blocks = kQkvTT * feat_tiles;
  const int g = w / group_blocks;
  const int rem = w - g * group_blocks;
  const int tt_in_g = (tok_tiles - g * kQkvTT < kQkvTT) ? tok_tiles - g * kQkvTT : kQkvTT;
  const int chunk = rem / (kQkvFT * tt_in_g);
  const int idx = rem - chunk * kQkvFT * tt_in_g;
  const int f = idx / tt_in_g;
  return QkvTile{chunk * kQkvFT + f, g * kQkvTT + (idx - f * tt_in_g)};
}

hipError_t launch_qkv_publish(const QkvParams& p, hipStream_t stream);

}  // namespace wf

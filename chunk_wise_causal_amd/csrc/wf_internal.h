// Internal launch interface of libwf: kernel parameter blocks shared by the
// host API (api.cpp) and the kernels (publish.hip, attn_bf16.hip,
// attn_fp32.hip).  Parameter blocks travel as kernel arguments, so a launch
// captures everything it needs and concurrent calls never share state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

constexpr int kMaxGroups = 32;     // query groups (slots) per attention call
constexpr int kMaxRanges = 256;    // merged visible ranges over all groups
constexpr int kMaxPairs = 64;      // head_dim / 2 for head_dim <= 128

// ---- publish ---------------------------------------------------------------
struct PublishParams {
  const void* k;        // [n_tok] rows of [H][D]
  const void* v;
  void* q;              // nullable, rotated in place
  void* k_pages;        // [pages][H][ps][D]
  void* v_pages;        // [pages][H][D][ps]
  const int32_t* page_table;
  const int32_t* pos;   // [n_tok][3], nullable when !rope
  int* status;          // device status word
  int64_t k_stride, v_stride, q_stride;   // elements between token rows
  int32_t n_tok, dst_start;
  int32_t heads, head_dim, ps_log2, num_pages, num_logical_pages;
  int32_t tiles;            // 64-token tiles covering the published window
  int32_t heads_per_kblock;  // heads per K block (rotary factors shared)
  int32_t k_blocks;         // K blocks; V blocks (tiles * heads) follow
  int32_t rope;         // 0/1
  int32_t pair_axis[kMaxPairs];     // axis (0 t, 1 h, 2 w) of each pair
  double pair_omega[kMaxPairs];     // theta^(-2i/d_a) of each pair
  int32_t band0[4];                 // first pair of the t, h, w sub-bands; band0[3] = D/2
};

// ---- attention -----------------------------------------------------------
struct AttnParams {
  const void* q;
  void* out;
  float* lse;           // nullable, [H][lse_stride]
  const void* k_pages;
  const void* v_pages;
  const int32_t* page_table;
  int* status;
  int64_t q_stride, out_stride;      // elements between rows
  int32_t heads, ps_log2, num_pages, num_logical_pages;
  int32_t lse_stride;                // = q_slot_start[n_slots]
  float scale;                       // softmax scale
  float scale_log2;                  // scale * log2(e)
  int32_t n_groups;
  int32_t tiles_per_head;            // sum of query tiles of all groups
  // groups in work order (longest visible context first)
  int32_t grp_tile_end[kMaxGroups];  // cumulative query tiles, work order
  int32_t grp_row0[kMaxGroups];      // first query row
  int32_t grp_row1[kMaxGroups];      // one past the last query row
  int32_t grp_rng0[kMaxGroups];      // first visible range of the group
  int32_t grp_rng1[kMaxGroups];      // one past its last visible range
  int2 ranges[kMaxRanges];           // [lo, hi) logical key ranges, sorted
};

// Work items of the attention blocks.  An item is an index into the
// head-major list of (head, group, query tile).  The hardware deals blocks
// round-robin to the 8 XCDs, so XCD x runs blocks x, x+8, ... (n_x of them:
// nb/8, plus one for x < nb%8), in that order.
//
// xcd_run_item: XCD x takes the contiguous run [x*per, (x+1)*per) of the
// list (per = nb/8), which keeps the query tiles of a head on one XCD and
// its key/value tiles in that XCD's L2; within the run the items go longest
// first (group by group in work order, head by head, tile by tile).  Blocks
// past 8*per keep their own index.
__host__ __device__ __forceinline__ int xcd_run_item(const AttnParams& p, int b, int nb) {
  const int per = nb >> 3;
  if (b >= (per << 3)) return b;
  const int r0 = (b & 7) * per, r1 = r0 + per;
  const int T = p.tiles_per_head;
  const int h_lo = r0 / T, h_hi = (r1 - 1) / T;
  int k = b >> 3;
  for (int g = 0; g < p.n_groups; ++g) {
    const int gs = g ? p.grp_tile_end[g - 1] : 0, ge = p.grp_tile_end[g];
    for (int hd = h_lo; hd <= h_hi; ++hd) {
      const int lo = max(hd * T + gs, r0), hi = min(hd * T + ge, r1);
      const int cnt = max(hi - lo, 0);
      if (k < cnt) return lo + k;
      k -= cnt;
    }
  }
  return r0 + k;   // not reached: the run holds per items
}

// Items of group g (all heads) and XCD x's share of them: an eighth of every
// group but the last, contiguous in head-major order; the last (shortest)
// group fills the XCD up to its n_x blocks.
__host__ __device__ __forceinline__ int64_t group_items(const AttnParams& p, int g) {
  return (int64_t)(p.grp_tile_end[g] - (g ? p.grp_tile_end[g - 1] : 0)) * p.heads;
}
__host__ __device__ __forceinline__ int group_share(const AttnParams& p, int g, int x) {
  const int64_t n = group_items(p, g);
  return (int)((((int64_t)x + 1) * n >> 3) - (((int64_t)x * n) >> 3));
}
__host__ __device__ __forceinline__ int last_group_share(const AttnParams& p, int nb, int x) {
  int s = (nb >> 3) + (x < (nb & 7) ? 1 : 0);
  for (int g = 0; g + 1 < p.n_groups; ++g) s -= group_share(p, g, x);
  return s;
}

// xcd_work_item: every XCD takes its share of every group, groups in work
// order (longest visible context first), each share contiguous in
// head-major order (a few heads' tiles, whose key/value tiles stay in the
// XCD's L2).  Every XCD thus gets the same mix of long and short items,
// longest first.  When the last group is too small to even out the counts
// (tiny grids), the runs of xcd_run_item are used instead.
__host__ __device__ __forceinline__ int xcd_work_item(const AttnParams& p, int b, int nb) {
  const int G = p.n_groups;
  for (int x = 0; x < 8; ++x)
    if (last_group_share(p, nb, x) < 0) return xcd_run_item(p, b, nb);
  const int x = b & 7;
  int k = b >> 3;
  for (int g = 0; g < G; ++g) {
    const bool last = g + 1 == G;
    const int s = last ? last_group_share(p, nb, x) : group_share(p, g, x);
    if (k < s) {
      int o = 0;
      if (!last) {
        o = (int)(((int64_t)x * group_items(p, g)) >> 3);
      } else {
        for (int xx = 0; xx < x; ++xx) o += last_group_share(p, nb, xx);
      }
      const int j = o + k;
      const int gs = g ? p.grp_tile_end[g - 1] : 0;
      const int tg = p.grp_tile_end[g] - gs;
      const int head = j / tg;
      return head * p.tiles_per_head + gs + (j - head * tg);
    }
    k -= s;
  }
  return b;   // not reached: the shares hold every block
}

// launches (stream-ordered; return hipError_t of the launch)
hipError_t launch_publish(const PublishParams& p, int dtype, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int block_m,
                            hipStream_t stream);
hipError_t launch_attn_fp32(const AttnParams& p, int head_dim, int block_m,
                            hipStream_t stream);

// per-device status word (status.hip)
int* status_word_ptr(hipError_t* err);

// query-tile height of each attention kernel
constexpr int kBlockMBf16 = 256;
constexpr int kBlockMFp32 = 64;

}  // namespace wf

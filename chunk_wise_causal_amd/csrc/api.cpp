// Host side of libwf: argument validation, the slot-mask schedule, launches.
//
// Every check runs before the first HIP call, so a rejected call has no side
// effect and the checks can be exercised on a machine without a GPU.
//
// Source of the method: "Wave Forcing: Towards Speed-of-Light Streaming Video
// Generation", §3.1 (chunk-wise causal mask and context order) and §4.2
// (K/V published after QKV projection and RoPE into paged attention slots).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/wf.h"
#include "wf_internal.h"
#include "wf_mx.h"
#include "wf_qkv.h"
#include "wf_rotate.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return WF_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(WF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return ((1 << l) == v) ? l : -1;
}

// mx: the call reads or writes MXFP8 keys instead of pool->k_pages, which
// may then be NULL
int check_pool(const wf_kv_pool* pool, const wf_mx_keys* mx = nullptr) {
  if (!pool) return fail(WF_ERR_INVALID, "pool is NULL");
  if ((!mx && !pool->k_pages) || !pool->v_pages || !pool->page_table)
    return fail(WF_ERR_INVALID, "pool: k_pages, v_pages and page_table must be non-NULL");
  if (pool->dtype != WF_BF16 && pool->dtype != WF_FP32)
    return fail(WF_ERR_INVALID, "pool: dtype %d is not WF_BF16 or WF_FP32", pool->dtype);
  if (pool->num_heads < 1) return fail(WF_ERR_INVALID, "pool: num_heads must be >= 1");
  if (pool->num_pages < 1 || pool->num_logical_pages < 1)
    return fail(WF_ERR_INVALID, "pool: num_pages and num_logical_pages must be >= 1");
  if (pool->page_size < 16 || pool->page_size > 1024 || log2_exact(pool->page_size) < 0)
    return fail(WF_ERR_INVALID, "pool: page_size %d is not a power of two in [16, 1024]",
                pool->page_size);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(WF_ERR_UNSUPPORTED, "pool: head_dim %d not supported (64 or 128)",
                pool->head_dim);
  if (!aligned16(pool->k_pages) || !aligned16(pool->v_pages))
    return fail(WF_ERR_INVALID, "pool: page arrays must be 16-byte aligned");
  if (mx) {
    if (!mx->k8_pages || !mx->k8_scales)
      return fail(WF_ERR_INVALID, "mx keys: k8_pages and k8_scales must be non-NULL");
    if (!aligned16(mx->k8_pages) || !aligned16(mx->k8_scales))
      return fail(WF_ERR_INVALID, "mx keys: arrays must be 16-byte aligned");
    if (pool->dtype != WF_BF16 || pool->head_dim != 128)
      return fail(WF_ERR_UNSUPPORTED, "mx keys: built for bfloat16 pools with head_dim 128");
  }
  const int64_t elems = (int64_t)pool->num_pages * pool->num_heads * pool->page_size *
                        pool->head_dim;
  if (elems > (int64_t(1) << 40))
    return fail(WF_ERR_UNSUPPORTED, "pool: too large");
  return WF_OK;
}

int check_rope(const wf_kv_pool* pool, const wf_rope* rope, int32_t n_tok,
               const int32_t* pos_thw) {
  if (!rope) return WF_OK;
  if (rope->d_t < 0 || rope->d_h < 0 || rope->d_w < 0 || (rope->d_t & 1) || (rope->d_h & 1) ||
      (rope->d_w & 1))
    return fail(WF_ERR_INVALID, "rope: sub-band widths must be even and >= 0");
  if (rope->d_t + rope->d_h + rope->d_w != pool->head_dim)
    return fail(WF_ERR_INVALID, "rope: d_t + d_h + d_w = %d != head_dim %d",
                rope->d_t + rope->d_h + rope->d_w, pool->head_dim);
  if (!(rope->theta > 0.0) || !std::isfinite(rope->theta))
    return fail(WF_ERR_INVALID, "rope: theta must be finite and > 0");
  if (n_tok > 0 && !pos_thw) return fail(WF_ERR_INVALID, "pos_thw is NULL with rope");
  return WF_OK;
}

// frequencies of every pair: theta^(-2i/d_a), evaluated in double
void fill_pairs(const wf_rope* rope, int32_t* axis, double* omega) {
  const int d[3] = {rope->d_t, rope->d_h, rope->d_w};
  int pair = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < d[a] / 2; ++i, ++pair) {
      axis[pair] = a;
      omega[pair] = std::pow(rope->theta, (-2.0 * i) / (double)d[a]);
    }
}

int check_rows(const char* name, const void* ptr, int64_t stride, const wf_kv_pool* pool) {
  if (!ptr) return fail(WF_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(WF_ERR_INVALID, "%s must be 16-byte aligned", name);
  const int64_t row = (int64_t)pool->num_heads * pool->head_dim;
  if (stride < row)
    return fail(WF_ERR_INVALID, "%s_row_stride %lld < num_heads*head_dim %lld", name,
                (long long)stride, (long long)row);
  if (stride % 8 != 0)
    return fail(WF_ERR_INVALID, "%s_row_stride %lld is not a multiple of 8", name,
                (long long)stride);
  return WF_OK;
}

}  // namespace

namespace {

// One query group of an attention launch: its rows and its merged visible
// key ranges (sorted, non-adjacent).
struct GroupSpec {
  int row0, row1;
  std::vector<int2> ranges;
  int64_t vis;   // visible keys
};

// Append [lo, hi) to sorted ranges, merging with the last one when adjacent.
void push_range(std::vector<int2>& r, int lo, int hi) {
  if (!r.empty() && r.back().y == lo) r.back().y = hi;
  else r.push_back(make_int2(lo, hi));
}

// The launch shared by the slot and the generic entry points: groups are
// validated and their ranges merged by the caller; q and out were checked
// when any group has rows.
int launch_groups(const wf_kv_pool* pool, const std::vector<GroupSpec>& groups, const void* q,
                  int64_t q_row_stride, float scale, void* out, int64_t out_row_stride,
                  float* lse, int64_t lse_stride, hipStream_t stream,
                  const wf_mx_keys* mx = nullptr) {
  int n_ranges = 0;
  bool any_rows = false;
  for (const GroupSpec& g : groups) {
    n_ranges += (int)g.ranges.size();
    any_rows |= g.row1 > g.row0;
  }
  if (n_ranges > wf::kMaxRanges)
    return fail(WF_ERR_UNSUPPORTED, "%d visible ranges exceed the limit of %d", n_ranges,
                wf::kMaxRanges);
  if (!any_rows) return ok();

  wf::AttnParams p{};
  const bool bf16 = pool->dtype == WF_BF16;
  const int bm = bf16 ? wf::kBlockMBf16 : wf::kBlockMFp32;
  // longest visible context first (largest tiles start first), ties by group
  std::vector<int> order(groups.size());
  for (size_t g = 0; g < groups.size(); ++g) order[g] = (int)g;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return groups[a].vis > groups[b].vis; });
  int nr = 0, tiles = 0, k = 0;
  for (int gi : order) {
    const GroupSpec& g = groups[gi];
    const int rows = g.row1 - g.row0;
    if (rows == 0) continue;
    tiles += (rows + bm - 1) / bm;
    p.grp_tile_end[k] = tiles;
    p.grp_row0[k] = g.row0;
    p.grp_row1[k] = g.row1;
    p.grp_rng0[k] = nr;
    for (const int2& r : g.ranges) p.ranges[nr++] = r;
    p.grp_rng1[k] = nr;
    ++k;
  }
  p.n_groups = k;
  p.tiles_per_head = tiles;
  p.q = q;
  p.out = out;
  p.lse = lse;
  p.k_pages = pool->k_pages;
  p.v_pages = pool->v_pages;
  p.page_table = pool->page_table;
  p.q_stride = q_row_stride;
  p.out_stride = out_row_stride;
  p.heads = pool->num_heads;
  p.ps_log2 = log2_exact(pool->page_size);
  p.num_pages = pool->num_pages;
  p.num_logical_pages = pool->num_logical_pages;
  p.lse_stride = (int32_t)lse_stride;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int64_t blocks = (int64_t)tiles * pool->num_heads;
  if (blocks > 0x7fffffff) return fail(WF_ERR_UNSUPPORTED, "too many query tiles");

  hipError_t e;
  p.status = wf::status_word_ptr(&e);
  if (!p.status) return hip_fail(e, "status word");
  if (mx) {
    p.k_pages = mx->k8_pages;
    e = wf::launch_attn_mx(p, mx->k8_scales, stream);
  } else {
    e = bf16 ? wf::launch_attn_bf16(p, pool->head_dim, bm, stream)
             : wf::launch_attn_fp32(p, pool->head_dim, bm, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // namespace

extern "C" {

const char* wf_last_error(void) { return g_err.c_str(); }

const char* wf_version(void) { return "libwf 0.1.0 gfx950"; }

int wf_device_status(int32_t* status, int32_t clear) {
  if (!status) return fail(WF_ERR_INVALID, "status is NULL");
  hipError_t e;
  int* p = wf::status_word_ptr(&e);
  if (!p) return hip_fail(e, "status word");
  int v = 0;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  if ((e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "read status");
  if (clear) {
    const int zero = 0;
    if ((e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "clear status");
  }
  *status = v;
  return ok();
}

}  // extern "C"

namespace {

int publish_impl(const wf_kv_pool* pool, const wf_mx_keys* mx, const wf_rope* rope,
                 const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                 const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                 void* q_inout, int64_t q_row_stride, hipStream_t stream) {
  int rc = check_pool(pool, mx);
  if (rc) return rc;
  if (n_tok < 0) return fail(WF_ERR_INVALID, "n_tok %d < 0", n_tok);
  if (dst_logical_start < 0)
    return fail(WF_ERR_INVALID, "dst_logical_start %d < 0", dst_logical_start);
  const int64_t cap = (int64_t)pool->num_logical_pages * pool->page_size;
  if ((int64_t)dst_logical_start + n_tok > cap)
    return fail(WF_ERR_INVALID, "dst_logical_start + n_tok = %lld exceeds pool capacity %lld",
                (long long)dst_logical_start + n_tok, (long long)cap);
  wf::PublishParams p{};
  if ((rc = check_rope(pool, rope, n_tok, pos_thw))) return rc;
  if (q_inout && !rope) return fail(WF_ERR_INVALID, "q_inout requires rope");
  if (n_tok > 0) {
    if ((rc = check_rows("k", k, k_row_stride, pool))) return rc;
    if ((rc = check_rows("v", v, v_row_stride, pool))) return rc;
    if (q_inout && (rc = check_rows("q", q_inout, q_row_stride, pool))) return rc;
  }
  if (n_tok == 0) return ok();

  p.k = k;
  p.v = v;
  p.q = q_inout;
  p.k_pages = mx ? mx->k8_pages : pool->k_pages;
  p.v_pages = pool->v_pages;
  p.page_table = pool->page_table;
  p.pos = pos_thw;
  p.k_stride = k_row_stride;
  p.v_stride = v_row_stride;
  p.q_stride = q_inout ? q_row_stride : 0;
  p.n_tok = n_tok;
  p.dst_start = dst_logical_start;
  p.heads = pool->num_heads;
  p.head_dim = pool->head_dim;
  p.ps_log2 = log2_exact(pool->page_size);
  p.num_pages = pool->num_pages;
  p.num_logical_pages = pool->num_logical_pages;
  p.rope = rope ? 1 : 0;
  if (rope) {
    fill_pairs(rope, p.pair_axis, p.pair_omega);
    p.band0[0] = 0;
    p.band0[1] = rope->d_t / 2;
    p.band0[2] = (rope->d_t + rope->d_h) / 2;
    p.band0[3] = pool->head_dim / 2;
  }
  // 64-token tiles of the window; K blocks take groups of about 10 heads,
  // split evenly (the rotary factors of a tile are evaluated once per K
  // block), V blocks 256 features (bfloat16) or one head (float32)
  const int64_t tiles = ((int64_t)dst_logical_start + n_tok - 1) / 64 - dst_logical_start / 64 + 1;
  p.tiles = (int)tiles;
  // K blocks per tile: heads split into at most four groups of at least
  // four (measured: 4 groups of 10 at 40 heads, 3 groups of 4 at 12 heads;
  // more, smaller groups repeat the rotary factors, fewer leave a tail)
  const int kgroups = std::min(4, (pool->num_heads + 3) / 4);
  p.heads_per_kblock = (pool->num_heads + kgroups - 1) / kgroups;
  const int64_t v_per_tile = (mx || pool->dtype == WF_BF16)
                                 ? (pool->num_heads * pool->head_dim / 64 + 3) / 4
                                 : pool->num_heads;
  const int64_t blocks = tiles * kgroups + tiles * v_per_tile;
  if (blocks > 0x7fffffff) return fail(WF_ERR_UNSUPPORTED, "publish window too large");
  p.k_blocks = (int)(tiles * kgroups);

  hipError_t e;
  p.status = wf::status_word_ptr(&e);
  if (!p.status) return hip_fail(e, "status word");
  e = mx ? wf::launch_publish_mx(p, mx->k8_scales, stream)
         : wf::launch_publish(p, pool->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "publish launch");
  return ok();
}

}  // namespace

extern "C" {

int wf_kv_publish(const wf_kv_pool* pool, const wf_rope* rope, const void* k,
                  int64_t k_row_stride, const void* v, int64_t v_row_stride,
                  const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                  void* q_inout, int64_t q_row_stride, hipStream_t stream) {
  return publish_impl(pool, nullptr, rope, k, k_row_stride, v, v_row_stride, pos_thw, n_tok,
                      dst_logical_start, q_inout, q_row_stride, stream);
}

// The 8-bit QK^T variant's publish ([WF] §5.5): K quantized to MXFP8.
int wf_kv_publish_mx(const wf_kv_pool* pool, const wf_mx_keys* keys, const wf_rope* rope,
                     const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                     const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                     void* q_inout, int64_t q_row_stride, hipStream_t stream) {
  if (!keys) return fail(WF_ERR_INVALID, "keys is NULL");
  return publish_impl(pool, keys, rope, k, k_row_stride, v, v_row_stride, pos_thw, n_tok,
                      dst_logical_start, q_inout, q_row_stride, stream);
}

}  // extern "C"

namespace {

int chunk_attn_impl(const wf_kv_pool* pool, const wf_mx_keys* mx, const wf_segment* segs,
                    int32_t n_segs, const void* q, int64_t q_row_stride,
                    const int32_t* q_slot_start, int32_t n_slots, int32_t first_slot,
                    float scale, void* out, int64_t out_row_stride, float* lse,
                    hipStream_t stream) {
  int rc = check_pool(pool, mx);
  if (rc) return rc;
  if (!segs) return fail(WF_ERR_INVALID, "segs is NULL");
  if (n_segs < 1 || n_segs > 64) return fail(WF_ERR_INVALID, "n_segs %d not in [1, 64]", n_segs);
  if (!q_slot_start) return fail(WF_ERR_INVALID, "q_slot_start is NULL");
  if (n_slots < 1 || n_slots > wf::kMaxGroups)
    return fail(WF_ERR_INVALID, "n_slots %d not in [1, %d]", n_slots, wf::kMaxGroups);
  if (first_slot < 0 || first_slot > (1 << 30))
    return fail(WF_ERR_INVALID, "first_slot %d out of range", first_slot);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(WF_ERR_INVALID, "scale must be finite and > 0");
  const int64_t cap = (int64_t)pool->num_logical_pages * pool->page_size;
  std::vector<wf_segment> sorted(segs, segs + n_segs);
  for (int i = 0; i < n_segs; ++i) {
    const wf_segment& s = segs[i];
    if (s.kv_len < 1 || s.kv_start < 0 || (int64_t)s.kv_start + s.kv_len > cap)
      return fail(WF_ERR_INVALID, "segment %d [%d, +%d) outside the pool's %lld tokens", i,
                  s.kv_start, s.kv_len, (long long)cap);
  }
  std::sort(sorted.begin(), sorted.end(),
            [](const wf_segment& a, const wf_segment& b) { return a.kv_start < b.kv_start; });
  for (int i = 1; i < n_segs; ++i)
    if ((int64_t)sorted[i - 1].kv_start + sorted[i - 1].kv_len > sorted[i].kv_start)
      return fail(WF_ERR_INVALID, "segments overlap at token %d", sorted[i].kv_start);
  if (q_slot_start[0] < 0) return fail(WF_ERR_INVALID, "q_slot_start[0] < 0");
  for (int g = 0; g < n_slots; ++g)
    if (q_slot_start[g + 1] < q_slot_start[g])
      return fail(WF_ERR_INVALID, "q_slot_start is not non-decreasing at %d", g);
  for (int g = 0; g < n_slots; ++g) {
    bool own = false;
    for (int i = 0; i < n_segs; ++i) own |= (segs[i].slot == first_slot + g);
    if (!own)
      return fail(WF_ERR_INVALID, "query slot %d owns no segment", first_slot + g);
  }
  const int total_rows = q_slot_start[n_slots];
  const bool any_rows = total_rows > q_slot_start[0];
  if (any_rows) {
    if ((rc = check_rows("q", q, q_row_stride, pool))) return rc;
    if ((rc = check_rows("out", out, out_row_stride, pool))) return rc;
  }

  // ---- slot-mask schedule: merged visible ranges per group ([WF] §3.1) ----
  std::vector<GroupSpec> groups(n_slots);
  for (int g = 0; g < n_slots; ++g) {
    const int sl = first_slot + g;
    GroupSpec& G = groups[g];
    G.row0 = q_slot_start[g];
    G.row1 = q_slot_start[g + 1];
    G.vis = 0;
    for (const wf_segment& sg : sorted) {
      if (!(sg.slot < 0 || sg.slot >= sl)) continue;
      G.vis += sg.kv_len;
      push_range(G.ranges, sg.kv_start, sg.kv_start + sg.kv_len);
    }
  }
  return launch_groups(pool, groups, q, q_row_stride, scale, out, out_row_stride, lse,
                       total_rows, stream, mx);
}

}  // namespace

extern "C" {

int wf_chunk_attn(const wf_kv_pool* pool, const wf_segment* segs, int32_t n_segs,
                  const void* q, int64_t q_row_stride, const int32_t* q_slot_start,
                  int32_t n_slots, int32_t first_slot, float scale, void* out,
                  int64_t out_row_stride, float* lse, hipStream_t stream) {
  return chunk_attn_impl(pool, nullptr, segs, n_segs, q, q_row_stride, q_slot_start, n_slots,
                         first_slot, scale, out, out_row_stride, lse, stream);
}

// The 8-bit QK^T variant ([WF] §5.5): scores from MXFP8 queries and keys.
int wf_chunk_attn_mx(const wf_kv_pool* pool, const wf_mx_keys* keys, const wf_segment* segs,
                     int32_t n_segs, const void* q, int64_t q_row_stride,
                     const int32_t* q_slot_start, int32_t n_slots, int32_t first_slot,
                     float scale, void* out, int64_t out_row_stride, float* lse,
                     hipStream_t stream) {
  if (!keys) return fail(WF_ERR_INVALID, "keys is NULL");
  return chunk_attn_impl(pool, keys, segs, n_segs, q, q_row_stride, q_slot_start, n_slots,
                         first_slot, scale, out, out_row_stride, lse, stream);
}

int wf_group_attn(const wf_kv_pool* pool, const wf_kv_run* runs, int32_t n_runs,
                  const wf_query_group* groups, int32_t n_groups, const void* q,
                  int64_t q_row_stride, float scale, void* out, int64_t out_row_stride,
                  float* lse, int64_t lse_stride, hipStream_t stream) {
  int rc = check_pool(pool);
  if (rc) return rc;
  if (!runs) return fail(WF_ERR_INVALID, "runs is NULL");
  if (n_runs < 1 || n_runs > wf::kMaxRanges)
    return fail(WF_ERR_INVALID, "n_runs %d not in [1, %d]", n_runs, wf::kMaxRanges);
  if (!groups) return fail(WF_ERR_INVALID, "groups is NULL");
  if (n_groups < 1 || n_groups > wf::kMaxGroups)
    return fail(WF_ERR_INVALID, "n_groups %d not in [1, %d]", n_groups, wf::kMaxGroups);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(WF_ERR_INVALID, "scale must be finite and > 0");
  const int64_t cap = (int64_t)pool->num_logical_pages * pool->page_size;
  for (int i = 0; i < n_runs; ++i) {
    const wf_kv_run& r = runs[i];
    if (r.kv_len < 1 || r.kv_start < 0 || (int64_t)r.kv_start + r.kv_len > cap)
      return fail(WF_ERR_INVALID, "run %d [%d, +%d) outside the pool's %lld tokens", i,
                  r.kv_start, r.kv_len, (long long)cap);
  }
  int64_t max_row = 0;
  bool any_rows = false;
  std::vector<GroupSpec> specs(n_groups);
  for (int g = 0; g < n_groups; ++g) {
    const wf_query_group& G = groups[g];
    if (G.q_row_start < 0 || G.q_row_end < G.q_row_start)
      return fail(WF_ERR_INVALID, "group %d rows [%d, %d) invalid", g, G.q_row_start,
                  G.q_row_end);
    if (G.run_begin < 0 || G.run_end <= G.run_begin || G.run_end > n_runs)
      return fail(WF_ERR_INVALID, "group %d runs [%d, %d) not inside [0, %d) or empty", g,
                  G.run_begin, G.run_end, n_runs);
    std::vector<wf_kv_run> mine(runs + G.run_begin, runs + G.run_end);
    std::sort(mine.begin(), mine.end(),
              [](const wf_kv_run& a, const wf_kv_run& b) { return a.kv_start < b.kv_start; });
    GroupSpec& S = specs[g];
    S.row0 = G.q_row_start;
    S.row1 = G.q_row_end;
    S.vis = 0;
    for (size_t i = 0; i < mine.size(); ++i) {
      if (i && (int64_t)mine[i - 1].kv_start + mine[i - 1].kv_len > mine[i].kv_start)
        return fail(WF_ERR_INVALID, "runs of group %d overlap at token %d", g, mine[i].kv_start);
      S.vis += mine[i].kv_len;
      push_range(S.ranges, mine[i].kv_start, mine[i].kv_start + mine[i].kv_len);
    }
    max_row = std::max<int64_t>(max_row, G.q_row_end);
    any_rows |= G.q_row_end > G.q_row_start;
  }
  // each output row is written by one group only
  std::vector<std::pair<int, int>> rows;
  for (int g = 0; g < n_groups; ++g)
    if (groups[g].q_row_end > groups[g].q_row_start)
      rows.push_back({groups[g].q_row_start, groups[g].q_row_end});
  std::sort(rows.begin(), rows.end());
  for (size_t i = 1; i < rows.size(); ++i)
    if (rows[i - 1].second > rows[i].first)
      return fail(WF_ERR_INVALID, "query row ranges of two groups overlap at row %d",
                  rows[i].first);
  if (lse && (lse_stride < max_row || lse_stride > 0x7fffffff))
    return fail(WF_ERR_INVALID, "lse_stride %lld must cover row %lld and fit 32 bits",
                (long long)lse_stride, (long long)max_row);
  if (any_rows) {
    if ((rc = check_rows("q", q, q_row_stride, pool))) return rc;
    if ((rc = check_rows("out", out, out_row_stride, pool))) return rc;
  }
  return launch_groups(pool, specs, q, q_row_stride, scale, out, out_row_stride, lse,
                       lse ? lse_stride : 0, stream);
}

// History rotation ([WF] §3.1, bounded clean history then live store): the
// window's table entries rotate left by one chunk; pages do not move.
int wf_history_rotate(int32_t* page_table, int32_t num_logical_pages, int32_t page_size,
                      int32_t window_start, int32_t chunk_stride, int32_t n_chunks,
                      hipStream_t stream) {
  if (!page_table) return fail(WF_ERR_INVALID, "page_table is NULL");
  if ((reinterpret_cast<uintptr_t>(page_table) & 3u) != 0)
    return fail(WF_ERR_INVALID, "page_table must be 4-byte aligned");
  if (num_logical_pages < 1) return fail(WF_ERR_INVALID, "num_logical_pages must be >= 1");
  if (page_size < 16 || page_size > 1024 || log2_exact(page_size) < 0)
    return fail(WF_ERR_INVALID, "page_size %d is not a power of two in [16, 1024]", page_size);
  if (window_start < 0 || window_start % page_size != 0)
    return fail(WF_ERR_INVALID, "window_start %d is not a non-negative multiple of page_size",
                window_start);
  if (chunk_stride < page_size || chunk_stride % page_size != 0)
    return fail(WF_ERR_INVALID, "chunk_stride %d is not a positive multiple of page_size",
                chunk_stride);
  if (n_chunks < 1) return fail(WF_ERR_INVALID, "n_chunks must be >= 1");
  const int64_t first = window_start / page_size;
  const int64_t cp = chunk_stride / page_size;
  const int64_t n = cp * n_chunks;
  if (first + n > num_logical_pages)
    return fail(WF_ERR_INVALID, "window [%lld, %lld) pages exceeds num_logical_pages %d",
                (long long)first, (long long)(first + n), num_logical_pages);
  if (n > wf::kMaxRotatePages)
    return fail(WF_ERR_UNSUPPORTED, "window of %lld pages exceeds the limit of %d",
                (long long)n, wf::kMaxRotatePages);
  if (n_chunks == 1) return ok();
  const hipError_t e = wf::launch_rotate(page_table, (int)first, (int)n, (int)cp, stream);
  if (e != hipSuccess) return hip_fail(e, "rotation launch");
  return ok();
}

// The QKV projection with the publish fused into its epilogue ([WF] §4.2:
// K/V are published right after the projection and RoPE).
int wf_qkv_publish(const wf_kv_pool* pool, const wf_rope* rope, const void* x,
                   int64_t x_row_stride, int32_t hidden, const void* w_qkv, const void* bias,
                   const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                   void* q_out, int64_t q_row_stride, hipStream_t stream) {
  int rc = check_pool(pool);
  if (rc) return rc;
  if (pool->dtype != WF_BF16 || pool->head_dim != 128)
    return fail(WF_ERR_UNSUPPORTED, "qkv publish: built for bfloat16 pools with head_dim 128");
  if (n_tok < 0) return fail(WF_ERR_INVALID, "n_tok %d < 0", n_tok);
  if (dst_logical_start < 0)
    return fail(WF_ERR_INVALID, "dst_logical_start %d < 0", dst_logical_start);
  const int64_t cap = (int64_t)pool->num_logical_pages * pool->page_size;
  if ((int64_t)dst_logical_start + n_tok > cap)
    return fail(WF_ERR_INVALID, "dst_logical_start + n_tok = %lld exceeds pool capacity %lld",
                (long long)dst_logical_start + n_tok, (long long)cap);
  if (hidden < 64 || hidden % 64 != 0 || hidden > 65536)
    return fail(WF_ERR_UNSUPPORTED, "hidden %d is not a multiple of 64 in [64, 65536]", hidden);
  if ((rc = check_rope(pool, rope, n_tok, pos_thw))) return rc;
  if (n_tok > 0) {
    if (!x || !w_qkv) return fail(WF_ERR_INVALID, "x and w_qkv must be non-NULL");
    if (!aligned16(x) || !aligned16(w_qkv))
      return fail(WF_ERR_INVALID, "x and w_qkv must be 16-byte aligned");
    if (x_row_stride < hidden || x_row_stride % 8 != 0)
      return fail(WF_ERR_INVALID, "x_row_stride %lld must be >= hidden and a multiple of 8",
                  (long long)x_row_stride);
    if (x_row_stride > (int64_t(1) << 22))
      return fail(WF_ERR_UNSUPPORTED, "x_row_stride %lld exceeds 2^22", (long long)x_row_stride);
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u))
      return fail(WF_ERR_INVALID, "bias must be 2-byte aligned");
    if (q_out && (rc = check_rows("q", q_out, q_row_stride, pool))) return rc;
  }
  if (n_tok == 0) return ok();
  wf::QkvParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w_qkv);
  p.bias = static_cast<const uint16_t*>(bias);
  p.q_out = static_cast<uint16_t*>(q_out);
  p.k_pages = static_cast<uint16_t*>(pool->k_pages);
  p.v_pages = static_cast<uint16_t*>(pool->v_pages);
  p.page_table = pool->page_table;
  p.pos = pos_thw;
  p.x_stride = x_row_stride;
  p.q_stride = q_out ? q_row_stride : 0;
  p.n_tok = n_tok;
  p.hidden = hidden;
  p.dst_start = dst_logical_start;
  p.heads = pool->num_heads;
  p.ps_log2 = log2_exact(pool->page_size);
  p.num_pages = pool->num_pages;
  p.tok_tiles = (n_tok + wf::kQkvBlockTok - 1) / wf::kQkvBlockTok;
  p.sec0 = q_out ? 0 : 1;
  // blocks of two heads over the computed heads (2H without Q, 3H with)
  p.feat_tiles = ((3 - p.sec0) * pool->num_heads + 1) / 2;
  p.rope = rope ? 1 : 0;
  if (rope) {
    int32_t axis[wf::kMaxPairs];
    fill_pairs(rope, axis, p.pair_omega);
    p.band0[0] = 0;
    p.band0[1] = rope->d_t / 2;
    p.band0[2] = (rope->d_t + rope->d_h) / 2;
    p.band0[3] = pool->head_dim / 2;
  }
  if ((int64_t)p.feat_tiles * p.tok_tiles > 0x7fffffff)
    return fail(WF_ERR_UNSUPPORTED, "projection too large");
  hipError_t e;
  p.status = wf::status_word_ptr(&e);
  if (!p.status) return hip_fail(e, "status word");
  if ((e = wf::launch_qkv_publish(p, stream)) != hipSuccess)
    return hip_fail(e, "qkv publish launch");
  return ok();
}

}  // extern "C"

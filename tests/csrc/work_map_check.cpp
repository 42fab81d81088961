// Host check of the block -> work mappings: the attention work items
// (xcd_work_item and its fallback xcd_run_item in wf_internal.h) for a grid
// of nb = query tiles x heads blocks must be a permutation of [0, nb), so
// that every (head, group, query tile) is computed exactly once; the fused
// QKV projection's tiles (qkv_tile in wf_qkv.h) must cover every (feature
// tile, token tile) of the grid exactly once.  Exits non-zero and names the
// layout on the first failure.
#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

#include "wf_internal.h"
#include "wf_qkv.h"

using wf::AttnParams;

static bool check(const std::vector<int>& tiles, int heads, bool run_only, int* fallback) {
  AttnParams p{};
  p.n_groups = (int)tiles.size();
  p.heads = heads;
  int acc = 0;
  for (size_t g = 0; g < tiles.size(); ++g) p.grp_tile_end[g] = (acc += tiles[g]);
  p.tiles_per_head = acc;
  const int nb = acc * heads;
  bool fb = false;
  for (int x = 0; x < 8; ++x) fb |= wf::last_group_share(p, nb, x) < 0;
  *fallback += fb;
  std::vector<int> w(nb);
  for (int b = 0; b < nb; ++b)
    w[b] = run_only ? wf::xcd_run_item(p, b, nb) : wf::xcd_work_item(p, b, nb);
  std::sort(w.begin(), w.end());
  for (int i = 0; i < nb; ++i)
    if (w[i] != i) {
      std::printf("not a permutation: %zu groups, %d heads, %s\n", tiles.size(), heads,
                  run_only ? "runs" : "shares");
      return false;
    }
  return true;
}

static bool check_qkv(int feat_tiles, int tok_tiles) {
  const int nb = feat_tiles * tok_tiles;
  std::vector<char> seen(nb, 0);
  for (int b = 0; b < nb; ++b) {
    const wf::QkvTile t = wf::qkv_tile(b, nb, feat_tiles, tok_tiles);
    if (t.ftile < 0 || t.ftile >= feat_tiles || t.ttile < 0 || t.ttile >= tok_tiles ||
        seen[t.ftile * tok_tiles + t.ttile]++) {
      std::printf("qkv tiles not a permutation: %d feature x %d token tiles\n", feat_tiles,
                  tok_tiles);
      return false;
    }
  }
  return true;
}

int main() {
  int fallback = 0, n = 0;
  // fused QKV projection: every grid up to 64 x 40 tiles, and the 14B-like
  // ticks (60 or 40 feature tiles over 92 or 211 token tiles)
  for (int f = 1; f <= 64; ++f)
    for (int t = 1; t <= 40; ++t) {
      if (!check_qkv(f, t)) return 1;
      ++n;
    }
  for (int f : {20, 30, 40, 60})
    for (int t : {19, 92, 211}) {
      if (!check_qkv(f, t)) return 1;
      ++n;
    }
  // the query tiles per slot of the five workload shapes
  const std::vector<std::pair<std::vector<int>, int>> shapes = {
      {{1, 1}, 2}, {{19, 19, 19, 19}, 12}, {{19, 19, 19, 19, 19}, 12},
      {{19, 19, 19, 19}, 40}, {{43, 43, 43, 43, 43}, 40}};
  for (const auto& s : shapes) {
    for (bool run_only : {false, true}) {
      if (!check(s.first, s.second, run_only, &fallback)) return 1;
      ++n;
    }
  }
  std::mt19937 rng(7);
  for (int t = 0; t < 4000; ++t) {
    const int groups = 1 + (int)(rng() % 32), heads = 1 + (int)(rng() % 64);
    std::vector<int> tiles(groups);
    for (auto& v : tiles) v = 1 + (int)(rng() % 30);
    for (bool run_only : {false, true}) {
      if (!check(tiles, heads, run_only, &fallback)) return 1;
      ++n;
    }
  }
  std::printf("ok: %d layouts, %d of them on the run fallback\n", n, fallback);
  return 0;
}

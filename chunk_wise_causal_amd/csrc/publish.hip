// wf_kv_publish kernel: 3D RoPE on K (and optionally Q) and the paged scatter
// of K and V into the pool.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §4.2:
// K/V are published after the QKV projection and RoPE, straight into ordered
// paged attention slots, with no concatenation step.
//
// Memory-bound: every byte of K and V is read once and written once.  One
// launch runs two kinds of blocks, each shaped for what it moves:
//   K blocks  (64-token tile x a group of heads, in two passes of 32 tokens):
//             evaluate the rotary factors of the pass's tokens once
//             (double-precision angle and cos/sin, rounded to float) into
//             LDS, then for every head of the group
//             16-byte vector load -> rotate pairs in float (no fused
//             multiply-add) -> round to the storage type -> 16-byte store
//             into the K page row.  Registers are kept low (one head in
//             flight per thread) so that several blocks share a CU.
//   V blocks  (64-token tile x 256 features, bfloat16): every lane loads an
//             8-token x 8-feature block, transposes it in registers and
//             stores 8 runs of 8 consecutive tokens into the d-major V page
//             (16-byte stores), with no LDS staging and no barrier before
//             the stores.  For float32, a 64-token tile of one head is
//             staged in LDS and re-read by feature.
// Pool rows of both kinds are written with device-scope stores (st_device).
// Token tiles are aligned to 64 in logical space, so an 8-token run never
// crosses a page (pages hold >= 16 tokens).
#include <climits>
#include <type_traits>

#include "../../include/wf.h"
#include "wf_internal.h"
#include "wf_mx.h"
#include "wf_numerics.h"

namespace wf {
namespace {

constexpr int kTileTok = 64;
constexpr int kThreads = 256;

// rotate the pairs of one 16-byte vector in place (storage type T)
template <typename T>
__device__ __forceinline__ void rotate_vec(uint4& v, const float2* cs) {
  constexpr int EPV = 16 / sizeof(T);
  T* e = reinterpret_cast<T*>(&v);
#pragma unroll
  for (int j = 0; j < EPV / 2; ++j) {
    float y0, y1;
    if constexpr (sizeof(T) == 2) {
      rotate_pair(bf16_to_f32(e[2 * j]), bf16_to_f32(e[2 * j + 1]), cs[j], y0, y1);
      e[2 * j] = f32_to_bf16_rne(y0);
      e[2 * j + 1] = f32_to_bf16_rne(y1);
    } else {
      rotate_pair(e[2 * j], e[2 * j + 1], cs[j], y0, y1);
      e[2 * j] = y0;
      e[2 * j + 1] = y1;
    }
  }
}

// Streaming 16-byte loads and stores: every input byte is read once and every
// pool byte written once, so neither is kept for reuse (nontemporal).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void* ptr) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4*>(ptr)));
}

__device__ __forceinline__ void st_stream(void* ptr, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), static_cast<u32x4*>(ptr));
}

// 16-byte store at device scope (cache-policy bit sc1, no non-temporal
// bit): the pool rows go toward HBM without being kept in the L2 for reuse,
// and the memory side still merges neighbouring pieces.  For the K rows and
// the V runs of the bfloat16 publish this measured faster than streaming
// (non-temporal) stores (0.157 against 0.195 ms at the 14B-like tick) and
// than plain stores.  A vector store in inline assembly: no builtin takes a
// scope for a 16-byte store.
__device__ __forceinline__ void st_device(void* ptr, uint4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(ptr), "v"(__builtin_bit_cast(u32x4, v))
               : "memory");
}

// Quantize and store one rotated 8-element K vector of a bfloat16 head row
// (D = 128: 16 vectors per row in 16 consecutive lanes; a 32-feature block
// is 4 consecutive lanes, all active or all inactive together, like the
// row).  `dst` is the vector's element address in the bf16 K-pool layout
// (head 0) or null; the MXFP8 pools share that indexing, one byte per
// element for the codes and one scale byte per 32 elements.
__device__ __forceinline__ void mx_store(const PublishParams& p, void* k8_scales, uint4 v,
                                         const uint16_t* dst, int h, int ps) {
  constexpr int D = 128;
  const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(bf16_to_f32(e[j])));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const uint32_t sc = mx_scale_code(amax);
  const float mult = __uint_as_float((254u - sc) << 23);   // 2^(127 - sc), exact
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j >> 2] |= e4m3_code(bf16_to_f32(e[j]) * mult) << (8 * (j & 3));
  // the row's four scale codes, gathered by its first lane
  const int lane = threadIdx.x & 63, row0 = lane & ~15;
  uint32_t word = 0u;
#pragma unroll
  for (int bk = 0; bk < 4; ++bk) word |= (uint32_t)__shfl((int)sc, row0 + 4 * bk) << (8 * bk);
  if (!dst) return;
  const int64_t idx = (dst - static_cast<const uint16_t*>(p.k_pages)) + (int64_t)h * ps * D;
  uint8_t* codes = static_cast<uint8_t*>(p.k_pages) + idx;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(codes));
  if ((lane & 15) == 0)
    __builtin_nontemporal_store(word, static_cast<uint32_t*>(k8_scales) + idx / D);
}

// K blocks' factor table of a tile: the tile's token positions, the
// per-axis position ranges, the table row base of every pair and the
// (cos, sin) of every (pair, position) present, within the LDS of the
// per-element factors it replaces
template <int D>
struct KTable {
  // entries that fit the LDS of the per-element factors (32 tokens x D/2 pairs)
  static constexpr int CAP = (kTileTok / 2 * (D / 2) * 8 - kTileTok * 16 - 8 * 4 - (D / 2) * 4) / 8;
  int4 pos[kTileTok];
  int hdr[8];
  int rb[D / 2];
  float2 tab[CAP];
};

template <int D, typename T>
union PublishShared {
  // LDS row padding (elements): 8 bytes, so that the 8 rows one run reads
  // (8 apart) spread over more banks than with a 16-byte pad
  static constexpr int VPAD = 8 / sizeof(T);
  float2 cs[kTileTok / 2][D / 2];               // K blocks: rotary factors (32 tokens)
  KTable<D> kt;                                 // K blocks: the tile's factor table
  T vt[kTileTok][D + VPAD];                     // V blocks: staged rows
};

// physical page of every token of the tile (-1: outside the published window
// or a bad page-table entry, which also raises the status bit)
__device__ __forceinline__ void tile_pages(const PublishParams& p, int L0, int lo, int hi,
                                           int* page_of) {
  const int tid = threadIdx.x;
  if (tid < kTileTok) {
    const int L = L0 + tid;
    int page = -1;
    // host validation keeps L >> ps_log2 < num_logical_pages for published rows
    if (L >= lo && L < hi) {
      page = p.page_table[L >> p.ps_log2];
      if (page < 0 || page >= p.num_pages) {
        atomicOr(p.status, WF_STATUS_BAD_PAGE);
        page = -1;
      }
    }
    page_of[tid] = page;
  }
}

// A K block's rotation from a per-tile factor table.  On a frame grid the
// tile's 64 tokens take few distinct positions per axis, so the factors are
// evaluated once per (pair, position) present, the per-axis position ranges
// of the tile's in-window tokens, instead of once per (token, pair); every
// head of the group then rotates with table lookups in one pass of 64
// tokens.  The factors are the same double-precision evaluation rounded to
// float, so the results do not change.  Returns false (nothing done but
// reading the positions) when the ranges do not fit the table.
template <int D, bool BF16, bool HAS_Q, bool MX>
__device__ __forceinline__ bool k_block_table(const PublishParams& p, void* k8_scales,
                                              KTable<D>& kt, const int* page_of, int L0, int lo,
                                              int hi, int h0, int h1) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPV = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = D / EPV;               // vectors per head row
  constexpr int NP = D / 2;
  constexpr int PER = kTileTok * VPR / kThreads;   // vectors per thread per head
  const int tid = threadIdx.x;
  const int ps = 1 << p.ps_log2;
  if (tid < kTileTok) {
    // wave 0 holds the tile's tokens: positions and per-axis ranges of the
    // in-window ones (an empty tile leaves hi < lo)
    const int L = L0 + tid;
    const bool in = L >= lo && L < hi;
    int4 v = make_int4(0, 0, 0, 0);
    if (in) {
      const int64_t t = L - p.dst_start;
      v = make_int4(p.pos[t * 3], p.pos[t * 3 + 1], p.pos[t * 3 + 2], 0);
    }
    kt.pos[tid] = v;
    int lo3[3], hi3[3];
    const int a0[3] = {v.x, v.y, v.z};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      int mn = in ? a0[a] : INT_MAX, mx = in ? a0[a] : INT_MIN;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        mn = min(mn, __shfl_xor(mn, m));
        mx = max(mx, __shfl_xor(mx, m));
      }
      lo3[a] = mn;
      hi3[a] = mx;
    }
    if (tid == 0) {
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        kt.hdr[a] = lo3[a];
        kt.hdr[3 + a] = hi3[a];
      }
    }
  }
  __syncthreads();   // positions, ranges and page_of visible
  int64_t rng[3], off[4];
  int mn[3];
  off[0] = 0;
  bool fits = true;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    mn[a] = kt.hdr[a];
    rng[a] = (int64_t)kt.hdr[3 + a] - kt.hdr[a] + 1;
    fits &= rng[a] >= 1;
    off[a + 1] = off[a] + (int64_t)(p.band0[a + 1] - p.band0[a]) * rng[a];
  }
  if (!fits || off[3] > KTable<D>::CAP) {   // uniform over the block
    __syncthreads();   // every thread has read the ranges before the caller reuses the LDS
    return false;
  }
  {
    const int o1 = (int)off[1], o2 = (int)off[2], r0 = (int)rng[0], r1 = (int)rng[1],
              r2 = (int)rng[2];
    if (tid < NP) {
      const int a = (tid >= p.band0[1]) + (tid >= p.band0[2]);
      const int oa = a == 0 ? 0 : (a == 1 ? o1 : o2);
      const int ra_ = a == 0 ? r0 : (a == 1 ? r1 : r2);
      const int ma = a == 0 ? mn[0] : (a == 1 ? mn[1] : mn[2]);
      const int b0 = a == 0 ? 0 : (a == 1 ? p.band0[1] : p.band0[2]);
      kt.rb[tid] = oa + (tid - b0) * ra_ - ma;
    }
    for (int e = tid; e < (int)off[3]; e += kThreads) {
      const int a = (e >= o1) + (e >= o2);
      const int oa = a == 0 ? 0 : (a == 1 ? o1 : o2);
      const int ra_ = a == 0 ? r0 : (a == 1 ? r1 : r2);
      const int ma = a == 0 ? mn[0] : (a == 1 ? mn[1] : mn[2]);
      const int b0 = a == 0 ? 0 : (a == 1 ? p.band0[1] : p.band0[2]);
      const int within = e - oa;
      const int pr = b0 + within / ra_;
      kt.tab[e] = rotary_factors(ma + within % ra_, p.pair_omega[pr]);
    }
  }
  __syncthreads();   // the table visible
  // vectors of this thread: idx = tid + kThreads * i -> (token ti, vector c);
  // each pair's table entry is fixed for the tile, every head adds a uniform
  // offset to the row pointers (h*D in the rows, h*ps*D in the pages)
  const T* __restrict__ kin = static_cast<const T*>(p.k);
  T* qio = static_cast<T*>(p.q);
  T* __restrict__ kpg = static_cast<T*>(p.k_pages);
  const T* src[PER];
  T* qptr[PER];
  T* dst[PER];
  int ent[PER][EPV / 2];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + kThreads * i;
    const int ti = idx / VPR, c = idx % VPR;
    const int L = L0 + ti;
    const int64_t t = L - p.dst_start;
    const bool in = L >= lo && L < hi;
    const int page = in ? page_of[ti] : -1;
    src[i] = in ? kin + t * p.k_stride + c * EPV : nullptr;
    qptr[i] = (in && HAS_Q) ? qio + t * p.q_stride + c * EPV : nullptr;
    dst[i] = page >= 0 ? kpg + ((int64_t)page * p.heads * ps + (L & (ps - 1))) * D + c * EPV
                       : nullptr;
    const int4 pz = kt.pos[ti];
#pragma unroll
    for (int j = 0; j < EPV / 2; ++j) {
      const int pr = c * (EPV / 2) + j;
      const int a = (pr >= p.band0[1]) + (pr >= p.band0[2]);
      ent[i][j] = kt.rb[pr] + (a == 0 ? pz.x : (a == 1 ? pz.y : pz.z));
    }
  }
  for (int h = h0; h < h1; ++h) {
    uint4 kv[PER], qv[HAS_Q ? PER : 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!src[i]) continue;
      kv[i] = ld_stream(src[i] + (int64_t)h * D);
      if constexpr (HAS_Q) qv[i] = *reinterpret_cast<const uint4*>(qptr[i] + (int64_t)h * D);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!src[i]) continue;
      float2 cs[EPV / 2];
#pragma unroll
      for (int j = 0; j < EPV / 2; ++j) cs[j] = kt.tab[ent[i][j]];
      rotate_vec<T>(kv[i], cs);
      if constexpr (HAS_Q) {
        rotate_vec<T>(qv[i], cs);
        *reinterpret_cast<uint4*>(qptr[i] + (int64_t)h * D) = qv[i];
      }
      if constexpr (MX) {
        mx_store(p, k8_scales, kv[i], dst[i], h, ps);
      } else {
        if (dst[i]) st_device(dst[i] + (int64_t)h * ps * D, kv[i]);
      }
    }
  }
  return true;
}

template <int D, bool BF16, bool HAS_Q, bool MX>
__device__ __forceinline__ void k_block(
    const PublishParams& p, void* k8_scales, int b,
    PublishShared<D, typename std::conditional<BF16, uint16_t, float>::type>& sm,
    int* page_of) {
  static_assert(!MX || (BF16 && D == 128), "MXFP8 keys: bfloat16, head_dim 128");
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPV = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = D / EPV;               // vectors per head row
  constexpr int HALF = kTileTok / 2;         // tokens per factor pass
  constexpr int PER = HALF * VPR / kThreads; // vectors per thread per head and pass
  const int tid = threadIdx.x;
  const int ps = 1 << p.ps_log2;
  const int tile = b % p.tiles, grp = b / p.tiles;
  const int L0 = (p.dst_start / kTileTok + tile) * kTileTok;
  const int lo = max(L0, p.dst_start);
  const int hi = min(L0 + kTileTok, p.dst_start + p.n_tok);
  const int h0 = grp * p.heads_per_kblock;
  const int h1 = min(p.heads, h0 + p.heads_per_kblock);
  const T* __restrict__ kin = static_cast<const T*>(p.k);
  T* qio = static_cast<T*>(p.q);
  T* __restrict__ kpg = static_cast<T*>(p.k_pages);

  tile_pages(p, L0, lo, hi, page_of);
  if (p.rope && k_block_table<D, BF16, HAS_Q, MX>(p, k8_scales, sm.kt, page_of, L0, lo, hi, h0,
                                                    h1))
    return;
  // otherwise (positions spread too widely for the table): factors per
  // element, in two passes of 32 tokens that keep them at half the LDS of
  // the staged V rows, so K and V blocks reach the same occupancy
  for (int half = 0; half < 2; ++half) {
    const int T0 = L0 + half * HALF;
    if (half) __syncthreads();   // every thread is done with the previous factors
    if (p.rope) {
      for (int idx = tid; idx < HALF * (D / 2); idx += kThreads) {
        const int ti = idx / (D / 2), pr = idx % (D / 2);
        const int L = T0 + ti;
        if (L < lo || L >= hi) continue;
        const int t = L - p.dst_start;
        sm.cs[ti][pr] = rotary_factors(p.pos[(int64_t)t * 3 + p.pair_axis[pr]], p.pair_omega[pr]);
      }
    }
    __syncthreads();   // factors (and, in the first pass, page_of) visible
    // vectors of this thread: idx = tid + kThreads * i -> (token ti, vector c);
    // source and destination bases are fixed for the pass, each head adds a
    // uniform offset (h*D in the rows, h*ps*D in the pages)
    const T* src[PER];
    T* qptr[PER];
    T* dst[PER];
    int fidx[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + kThreads * i;
      const int ti = idx / VPR, c = idx % VPR;
      const int L = T0 + ti;
      const int64_t t = L - p.dst_start;
      const bool in = L >= lo && L < hi;
      const int page = in ? page_of[half * HALF + ti] : -1;
      src[i] = in ? kin + t * p.k_stride + c * EPV : nullptr;
      qptr[i] = (in && HAS_Q) ? qio + t * p.q_stride + c * EPV : nullptr;
      dst[i] = page >= 0 ? kpg + ((int64_t)page * p.heads * ps + (L & (ps - 1))) * D + c * EPV
                         : nullptr;
      fidx[i] = ti * (D / 2) + c * (EPV / 2);
    }
    const float2* cs = &sm.cs[0][0];
    for (int h = h0; h < h1; ++h) {
      uint4 kv[PER], qv[HAS_Q ? PER : 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (!src[i]) continue;
        kv[i] = ld_stream(src[i] + (int64_t)h * D);
        if constexpr (HAS_Q) qv[i] = *reinterpret_cast<const uint4*>(qptr[i] + (int64_t)h * D);
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (!src[i]) continue;
        if (p.rope) {
          rotate_vec<T>(kv[i], cs + fidx[i]);
          if constexpr (HAS_Q) {
            rotate_vec<T>(qv[i], cs + fidx[i]);
            *reinterpret_cast<uint4*>(qptr[i] + (int64_t)h * D) = qv[i];
          }
        }
        if constexpr (MX) {
          mx_store(p, k8_scales, kv[i], dst[i], h, ps);
        } else {
          if (dst[i]) st_device(dst[i] + (int64_t)h * ps * D, kv[i]);
        }
      }
    }
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void v_block(
    const PublishParams& p, int b,
    PublishShared<D, typename std::conditional<BF16, uint16_t, float>::type>& sm,
    int* page_of) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int VPR = D / EPV;
  constexpr int PER = kTileTok * VPR / kThreads;        // staged vectors per thread
  constexpr int RUNS = D * (kTileTok / 8) / kThreads;   // 8-token runs per thread
  const int tid = threadIdx.x;
  const int ps = 1 << p.ps_log2;
  const int tile = b % p.tiles, h = b / p.tiles;
  const int L0 = (p.dst_start / kTileTok + tile) * kTileTok;
  const int lo = max(L0, p.dst_start);
  const int hi = min(L0 + kTileTok, p.dst_start + p.n_tok);
  const T* __restrict__ vin = static_cast<const T*>(p.v);
  T* __restrict__ vpg = static_cast<T*>(p.v_pages);

  tile_pages(p, L0, lo, hi, page_of);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + kThreads * i;
    const int ti = idx / VPR, c = idx % VPR;
    const int L = L0 + ti;
    if (L < lo || L >= hi) continue;
    const int64_t t = L - p.dst_start;
    const uint4 val = ld_stream(vin + t * p.v_stride + (int64_t)h * D + c * EPV);
    reinterpret_cast<uint2*>(&sm.vt[ti][c * EPV])[0] = make_uint2(val.x, val.y);
    reinterpret_cast<uint2*>(&sm.vt[ti][c * EPV])[1] = make_uint2(val.z, val.w);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RUNS; ++i) {
    const int idx = tid + kThreads * i;
    const int d = idx / (kTileTok / 8), r8 = idx % (kTileTok / 8);
    const int ti0 = r8 * 8;
    const int L = L0 + ti0;
    if (L + 8 <= lo || L >= hi) continue;
    int page = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (L + e >= lo && L + e < hi) page = page_of[ti0 + e];
    if (page < 0) continue;
    T* dst = vpg + (((int64_t)page * p.heads + h) * D + d) * ps + (L & (ps - 1));
    T run[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) run[e] = sm.vt[ti0 + e][d];
    if (L >= lo && L + 8 <= hi) {
#pragma unroll
      for (int v = 0; v < 8 / EPV; ++v)
        st_stream(reinterpret_cast<uint4*>(dst) + v, reinterpret_cast<const uint4*>(run)[v]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (L + e >= lo && L + e < hi) dst[e] = run[e];
    }
  }
}

// V block without LDS (bfloat16): 64 tokens x 256 features (2 heads of 128
// or 4 of 64).  Wave w takes a 64-feature block of one head; lane (c, g)
// loads the 16-byte vectors c (features 8c..8c+7 of the block) of tokens
// 8g..8g+7, transposes the 8 x 8 block in registers and stores 8 runs of 8
// consecutive tokens, one per feature, into the d-major V page.  An aligned
// run of 8 tokens lies in one page (pages hold at least 16), so each lane
// reads its own page entry: no shared page list and no barrier.
template <int D>
__device__ __forceinline__ void v_block_reg(const PublishParams& p, int tile, int vb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fb = vb * (kThreads / 64) + wave;          // 64-feature block
  const int h = fb / (D / 64), f0 = (fb % (D / 64)) * 64;
  const int c = lane & 7, g = lane >> 3;
  const int ps = 1 << p.ps_log2;
  const int L0 = (p.dst_start / kTileTok + tile) * kTileTok;
  const int lo = max(L0, p.dst_start);
  const int hi = min(L0 + kTileTok, p.dst_start + p.n_tok);
  const bool live = h < p.heads;
  const uint16_t* __restrict__ vin = static_cast<const uint16_t*>(p.v);
  uint16_t* __restrict__ vpg = static_cast<uint16_t*>(p.v_pages);
  const int Lg = L0 + 8 * g;
  uint4 r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int L = Lg + j;
    r[j] = make_uint4(0, 0, 0, 0);
    if (live && L >= lo && L < hi)
      r[j] = ld_stream(vin + (int64_t)(L - p.dst_start) * p.v_stride + (int64_t)h * D + f0 + 8 * c);
  }
  if (!live || Lg + 8 <= lo || Lg >= hi) return;
  // host validation keeps L >> ps_log2 < num_logical_pages for published rows
  const int page = p.page_table[max(Lg, lo) >> p.ps_log2];
  if (page < 0 || page >= p.num_pages) {
    atomicOr(p.status, WF_STATUS_BAD_PAGE);
    return;
  }
  uint16_t* dst = vpg + (((int64_t)page * p.heads + h) * D + f0 + 8 * c) * ps + (Lg & (ps - 1));
  const bool full = Lg >= lo && Lg + 8 <= hi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // run e: feature 8c+e of tokens 8g..8g+7 (element e of each r[j])
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = (&r[2 * k].x)[e >> 1], b = (&r[2 * k + 1].x)[e >> 1];
      w[k] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    uint16_t* d = dst + (int64_t)e * ps;
    if (full) {
      // a run is 16 bytes of a feature row of the page; the blocks of
      // neighbouring tiles fill the rest of that row at about the same time
      st_device(d, make_uint4(w[0], w[1], w[2], w[3]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (Lg + j >= lo && Lg + j < hi) d[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    }
  }
}

// at least 5 waves per SIMD; the variants that also rotate Q need more
// registers and take 4
template <int D, bool BF16, bool HAS_Q, bool MX>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(HAS_Q ? 4 : 5)))
void publish_kernel(const PublishParams p, void* k8_scales) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  __shared__ __attribute__((aligned(16))) PublishShared<D, T> sm;
  __shared__ int page_of[kTileTok];
  const int b = blockIdx.x;
  if (b < p.k_blocks) {
    k_block<D, BF16, HAS_Q, MX>(p, k8_scales, b, sm, page_of);
  } else {
    const int vb = b - p.k_blocks;
    if constexpr (BF16) v_block_reg<D>(p, vb % p.tiles, vb / p.tiles);
    else v_block<D, BF16>(p, vb, sm, page_of);
  }
}

template <int D, bool BF16>
void launch_typed(const PublishParams& p, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.q)
    hipLaunchKernelGGL((publish_kernel<D, BF16, true, false>), grid, block, 0, stream, p, nullptr);
  else
    hipLaunchKernelGGL((publish_kernel<D, BF16, false, false>), grid, block, 0, stream, p,
                       nullptr);
}

}  // namespace

// V blocks per 64-token tile: bfloat16 blocks take 256 features (4 waves of
// 64), float32 blocks one head
static int v_blocks_per_tile(const PublishParams& p, bool bf16) {
  return bf16 ? (p.heads * p.head_dim / 64 + 3) / 4 : p.heads;
}

hipError_t launch_publish_mx(const PublishParams& p, void* k8_scales, hipStream_t stream) {
  const int v_blocks = p.tiles * v_blocks_per_tile(p, true);
  dim3 grid(p.k_blocks + v_blocks), block(kThreads);
  if (p.q)
    hipLaunchKernelGGL((publish_kernel<128, true, true, true>), grid, block, 0, stream, p,
                       k8_scales);
  else
    hipLaunchKernelGGL((publish_kernel<128, true, false, true>), grid, block, 0, stream, p,
                       k8_scales);
  return hipGetLastError();
}

hipError_t launch_publish(const PublishParams& p, int dtype, hipStream_t stream) {
  const bool bf16 = dtype == WF_BF16;
  const int v_blocks = p.tiles * v_blocks_per_tile(p, bf16);
  dim3 grid(p.k_blocks + v_blocks), block(kThreads);
  if (p.head_dim == 128) {
    if (bf16) launch_typed<128, true>(p, grid, block, stream);
    else launch_typed<128, false>(p, grid, block, stream);
  } else {
    if (bf16) launch_typed<64, true>(p, grid, block, stream);
    else launch_typed<64, false>(p, grid, block, stream);
  }
  return hipGetLastError();
}

}  // namespace wf

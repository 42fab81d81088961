// Shared core of the chunk-wise causal attention forward kernels
// (attn_bf16.hip: bfloat16 QK^T; attn_mx.hip: MXFP8 QK^T).  Everything but
// the score product lives here: the tile walk over the merged visible key
// ranges, the V^T loads, the masks, the online softmax, O += P V, the
// two-group pipeline and the kernel body.  A kernel supplies a score policy
// S (see ScoreBf16 and ScoreMx) with its K-tile loads, its S^T = K Q^T
// product and scheduling hint, its query operands and its LDS slot sizes.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §3.1:
// a query of denoising slot s attends to the anchor, the clean history, the
// live store and every slot j >= s (itself included, with full attention
// inside the chunk).  The host turns that rule into a list of merged visible
// key ranges per slot; the kernel walks only the key tiles those ranges
// touch, so tiles the mask removes entirely are never loaded or multiplied.
//
// Work unit: one block = (head, slot, 256-row query tile), 8 waves of 64
// lanes, each wave owning 32 query rows; every K/V tile brought into LDS
// serves all 256 rows, which halves the L2 -> CU traffic of 128-row tiles.
// Per 64-key tile:
//   S^T = K Q^T   the policy's product: A = K rows from LDS, B = the query
//                 operands held in registers for the whole kernel.  The
//                 transposed product puts one query in every lane (lanes l
//                 and l+32 share it), so row max / row sum need a single
//                 cross-half exchange.
//   mask          only on tiles cut by a range boundary: keys outside the
//                 range become -inf; their K/V rows are never read from HBM
//                 (filled in LDS: K with NaN, which the row max skips, V with
//                 zeros), so stale or NaN memory cannot leak.
//   softmax       online, base 2, with the running max raised only when a
//                 row's tile max exceeds it by more than 2^8 (the exact
//                 result is unchanged: numerator and denominator share the
//                 stale max, and 2^8 keeps every term finite).  The max of
//                 tile j+1 is taken while O += P(j) V(j) runs, so the
//                 probabilities of a tile never wait for a reduction.  The
//                 denominator sums the bf16-rounded probabilities that
//                 multiply V, so the weights applied to V are normalized
//                 exactly.
//   O^T += V^T P^T  A = V^T read from the d-major V pages via LDS, B = P^T
//                 straight from the S^T accumulators: the K rows of S^T are
//                 loaded in the order sigma(i) (bits 2 and 3 of the row index
//                 swapped) so that each lane's 8 probabilities of a k-step
//                 are 8 consecutive keys, matching a 16-byte V^T read.  The
//                 row sums of P ride along on the matrix core: one 16x16x32
//                 product per k-step of the same P^T fragment against a
//                 constant 0/1 selector leaves each lane its query's sum.
//
// Pipeline: a ring of four LDS slots each for K and V (and the policy's
// extra slots), filled by direct global->LDS loads (global_load_lds_dwordx4)
// four and two tiles ahead.  Per tile, S(j+1) = K(j+1) Q^T is issued while
// the softmax of tile j runs, and the max of S(j+1) is taken while
// O += P(j) V(j) runs.  Half of the waves run half a tile behind the other
// half (one of each on every SIMD), so the vector work of one overlaps the
// matrix work of the other.  One barrier per tile.  Tiles cut by a range
// boundary, spread over several pages or naming a bad page take a register
// path that fills what lies outside the window.
//
// Block ids are remapped so that each XCD (blocks are dealt round-robin over
// the 8 XCDs) receives a contiguous run of the work list: the query tiles of
// one head and slot then share that XCD's L2 while streaming the same keys.
#pragma once

#include "../../include/wf.h"
#include "wf_internal.h"

namespace wf {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;       // waves per block, 32 query rows each
constexpr int BM = 32 * NW; // query rows per block
constexpr int BN = 64;      // keys per tile
constexpr int NT = 64 * NW; // threads per block
constexpr int LT = NT / 2;  // threads that issue the K/V tile loads (waves 0..NW/2-1)
constexpr int NS = 4;       // ring slots of K, V and the policy's extra data
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xhalf_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// row of the K tile feeding S^T row i: bits 2 and 3 swapped
__device__ __forceinline__ int sigma(int i) {
  return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// V^T column swizzle (16-byte chunk units): chunk c of feature row d sits at
// column c ^ vswz(d), so the A-operand reads of 16 consecutive lanes hit
// distinct banks
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 1); }

// Physical page for a page-table entry, or -1 (and `bad` set) for an entry
// outside the pool; integer arithmetic only, so that a uniform entry stays
// in scalar registers.  The status word is written once, after the key loop.
__device__ __forceinline__ int check_page(const AttnParams& p, int page, int& bad) {
  const int out = (unsigned)page >= (unsigned)p.num_pages;
  bad |= out;
  return out ? -1 : page;
}

// Per-lane lookup (register path: the token may differ between lanes).
__device__ __forceinline__ int lookup_page(const AttnParams& p, int L, int& bad) {
  return check_page(p, p.page_table[L >> p.ps_log2], bad);
}

// Wave-uniform page-table read through the constant address space: the
// table is read-only for the kernel, so the compiler emits a scalar load it
// can issue early and wait for exactly.  (A generic read becomes a vector
// load, and consuming one needs vmcnt(0), which would drain every in-flight
// tile load of the ring.)
typedef const __attribute__((address_space(4))) int32_t* const_table_ptr;

__device__ __forceinline__ int table_entry(const AttnParams& p, int logical_page) {
  return ((const_table_ptr)p.page_table)[logical_page];
}

// Position of the tile walk over the merged visible ranges of one group:
// the tile's first key kt, its range [rlo, rhi) and the physical page of
// the tile (pages of >= BN keys), read a step before the tile is loaded.
struct Walk {
  int ri;     // current range; == rng1 once past the last tile
  int kt;
  int rlo;
  int rhi;
  int page;
};

// One key tile as the loads and the mask see it, in three scalar registers:
// ktc = first key | 1 when the tile is cut by its range (ktc < 0: past the
// end of the walk), ri = its range, page = its physical page (-1 when the
// tile spans several pages or its page entry is bad).
struct Tile {
  int ktc;
  int ri;
  int page;
};

// BP: pages hold at least BN keys, so a 64-aligned tile lies in one page
// (otherwise every tile takes the register path, with per-lane lookups).
template <bool BP>
__device__ __forceinline__ void walk_page(const AttnParams& p, Walk& w) {
  if (BP) w.page = table_entry(p, w.kt >> p.ps_log2);
}

template <bool BP>
__device__ __forceinline__ Walk walk_first(const AttnParams& p, int rng0) {
  const int2 r = p.ranges[rng0];
  Walk w{rng0, r.x & ~(BN - 1), r.x, r.y, -1};
  walk_page<BP>(p, w);
  return w;
}

template <bool BP>
__device__ __forceinline__ void walk_next(const AttnParams& p, int rng1, Walk& w) {
  w.kt += BN;
  if (w.kt >= w.rhi) {
    if (++w.ri >= rng1) return;
    const int2 r = p.ranges[w.ri];
    w.rlo = r.x;
    w.rhi = r.y;
    w.kt = r.x & ~(BN - 1);
  }
  walk_page<BP>(p, w);
}

// The tile at the walk position; its page entry is checked here, once.
// The cut flag is integer arithmetic (sign bits), not a boolean, so that it
// stays in scalar registers.
template <bool BP>
__device__ __forceinline__ Tile walk_tile(const AttnParams& p, int rng1, const Walk& w,
                                          int& bad) {
  if (w.ri >= rng1) return Tile{-1, 0, -1};
  const int page = BP ? check_page(p, w.page, bad) : -1;
  const int cut = (int)(((uint32_t)(w.kt - w.rlo) | (uint32_t)(w.rhi - (w.kt + BN))) >> 31);
  return Tile{w.kt | cut, w.ri, page};
}

__device__ __forceinline__ int tile_kt(const Tile& t) { return t.ktc & ~(BN - 1); }
__device__ __forceinline__ bool tile_cut(const Tile& t) { return t.ktc & 1; }

// visible keys [lo, hi) of a tile
__device__ __forceinline__ void tile_window(const AttnParams& p, const Tile& t, int& lo,
                                            int& hi) {
  const int2 r = p.ranges[t.ri];
  lo = max(tile_kt(t), r.x);
  hi = min(tile_kt(t) + BN, r.y);
}

// every key of the tile visible and on one good page: the direct-load path
__device__ __forceinline__ bool tile_full(const Tile& t) {
  return ((t.page >> 31) | (t.ktc & 1)) == 0;
}

// Direct global->LDS load, 16 bytes per lane (global_load_lds_dwordx4, the
// scalar-base form): lane i writes LDS bytes [M0 + 16 i, +16) with
// M0 = wave_lds + OFF.  Issued as inline assembly so that the compiler does
// not model it: with this LDS-DMA form in the loop its wait bookkeeping
// drains every later LDS read with lgkmcnt(0), which serializes the
// A-operand fragment reads.  The caller's explicit vmcnt waits track
// completion.  The wait states cover an SGPR base written by a VALU
// instruction just before (a memory instruction reading it needs 5) and the
// M0 write read by the LDS-DMA load (1).
template <uint32_t OFF>
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t wave_lds) {
  asm volatile(
      "s_nop 4\n\t"
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(wave_lds), "i"(OFF)
      : "memory", "m0", "scc");
}

// The PER chunks of one loading thread: chunk i goes to this wave's 1 KB
// run i*LT/64 runs further on.
template <uint32_t SLOT, int I, int PER>
__device__ __forceinline__ void dma_chunks(const char* base, const uint32_t* off,
                                           uint32_t wave_lds) {
  if constexpr (I < PER) {
    dma16<SLOT + I * (LT / 64) * 1024>(base, off[I], wave_lds);
    dma_chunks<SLOT, I + 1, PER>(base, off, wave_lds);
  }
}

// Block-constant addressing of the V^T loads, which the first LT threads
// issue (the waves that run ahead; see Loop).
template <int D>
struct VLoad {
  static constexpr int PER = D * (BN / 8) / LT;   // 16-byte chunks per thread
  const char* v_head;       // V pages + head offset (bytes)
  int64_t page_bytes;
  uint32_t voff[PER];       // per-lane byte offsets of this thread's chunks
  uint32_t wave_lds;        // LDS byte address of this wave's first chunk
};

// ---- global -> LDS: the V^T tile [D][BN] of one head -----------------------
// A full tile goes by direct loads (PER per thread, left in flight).  Any
// other tile takes the register path, and a tile past the end of the walk
// loads nothing; both end with every older vector load complete, so a step
// never has more than its own direct loads outstanding.  (The K loads of the
// policies follow the same contract.)
template <int D, bool BP, uint32_t SLOT>
__device__ __forceinline__ void load_v(const AttnParams& p, const VLoad<D>& lc, int head,
                                       const Tile& t, uint16_t* __restrict__ lds, int& bad) {
  constexpr int PER = VLoad<D>::PER;
  const int ps = 1 << p.ps_log2;
  if (tile_full(t)) {
    const char* base =
        lc.v_head + (int64_t)t.page * lc.page_bytes + (int64_t)(tile_kt(t) & (ps - 1)) * 2;
    dma_chunks<SLOT, 0, PER>(base, lc.voff, lc.wave_lds);
    return;
  }
  if (t.ktc >= 0) {
    const int tid = threadIdx.x;
    const uint16_t* __restrict__ vpg = static_cast<const uint16_t*>(p.v_pages);
    uint16_t* vbuf = lds + SLOT / 2;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    int lo, hi;
    tile_window(p, t, lo, hi);
#pragma unroll 1
    for (int i = 0; i < PER; ++i) {
      const int q = i * LT + tid;
      const int d = q >> 3, col = (q & 7) ^ vswz(d);
      const int L = tile_kt(t) + col * 8;   // first of the chunk's 8 keys
      uint4 val = zero;
      if (L + 8 > lo && L < hi) {
        // an 8-key run never crosses a page (page_size >= 16, runs 8-aligned)
        const int page = BP ? t.page : lookup_page(p, max(L, lo), bad);
        if (page >= 0) {
          val = *reinterpret_cast<const uint4*>(
              vpg + (((int64_t)page * p.heads + head) * D + d) * ps + (L & (ps - 1)));
          if (L < lo || L + 8 > hi) {
            uint16_t* e = reinterpret_cast<uint16_t*>(&val);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (L + j < lo || L + j >= hi) e[j] = 0;
          }
        }
      }
      *reinterpret_cast<uint4*>(vbuf + q * 8) = val;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Tile geometry shared by both products
template <int D>
struct Frag {
  static constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  static constexpr int SB = BN / 32;  // 32-key blocks of S^T
  static constexpr int PK = BN / 16;  // k-steps of O^T += V^T P^T
};

// Row max of a score tile in log2 units, scaled by sl2 (both halves of the
// row combined).
template <int D>
__device__ __forceinline__ float tile_max(const f32x16* s, float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < Frag<D>::SB; ++sb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
  return xhalf_max(mx) * sl2;
}

// bf16 probabilities of one tile for running max m (their row sums are
// taken on the matrix core with the P V product, see pv)
template <int D>
__device__ __forceinline__ void probs(const f32x16* s, float sl2, float m, bf16x8* pb) {
  const float neg_m = -m;
#pragma unroll
  for (int t = 0; t < Frag<D>::PK; ++t) {
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * j], sl2, neg_m)),
                       __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * j + 1], sl2, neg_m))};
      const bf16x2 b = __builtin_convertvector(x, bf16x2);
      pk[j] = __builtin_bit_cast(uint32_t, b);
    }
    pb[t] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  }
}

// Row-sum selector: the A operand of a 16x16x32 product whose B operand is
// the P^T fragment of a k-step.  Read as a 16x16x32 B operand, lane
// 16g + n of that fragment holds 8 keys of query n + 16 (g % 2); row m of
// the selector is 1 on the k-groups g with g % 2 == (m / 4) % 2, so every
// output register of lane l is the sum of the k-step's 16 probabilities of
// query l % 32, the query the lane holds in S^T and O^T.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
  const int m = lane & 15, g = lane >> 4;
  const uint32_t w = ((g & 1) == ((m >> 2) & 1)) ? 0x3f803f80u : 0u;   // bf16 1.0 pairs
  return __builtin_bit_cast(bf16x8, make_uint4(w, w, w, w));
}

// O^T += V^T P^T, and l += the row sums of the same bf16 probabilities on
// the matrix core (one 16x16x32 product per k-step against the selector)
template <int D>
__device__ __forceinline__ void pv(const uint16_t* __restrict__ vbuf, const int* vaddr,
                                   const bf16x8* pb, f32x16* o, const bf16x8& sel, f32x4& lacc) {
#pragma unroll
  for (int t = 0; t < Frag<D>::PK; ++t) {
#pragma unroll
    for (int db = 0; db < Frag<D>::DB; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vbuf + vaddr[t] + 32 * db * BN);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
    }
    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[t], lacc, 0, 0, 0);
  }
}

// Scheduling hint for the block of O += P(j) V(j) and the max of S(j+1):
// V^T fragment reads run a few products ahead and each MFMA is followed by
// one vector instruction of the max.
template <int D>
__device__ __forceinline__ void interleave_pv_max() {
  constexpr int NM = Frag<D>::PK * (Frag<D>::DB + 1);   // MFMAs of the product and row sums
  constexpr int AHEAD = 3;
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    if (k + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Keys of a tile cut by a range boundary that lie outside [w_lo, w_hi) get
// score -inf (their K/V rows were zero-filled, never read from memory).
template <int D>
__device__ __forceinline__ void mask_tile(f32x16* s, int kt, int w_lo, int w_hi, int hg) {
  // register r of block sb holds key kt + 8hg + c with c = 32sb + 16(r/8) + r%8;
  // it is visible iff c - lo lies in [0, hi - lo) (one unsigned compare)
  const int lo = w_lo - (kt + 8 * hg);
  const unsigned span = (unsigned)(w_hi - w_lo);
#pragma unroll
  for (int sb = 0; sb < Frag<D>::SB; ++sb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * sb + 16 * (r >> 3) + (r & 7);
      if ((unsigned)(c - lo) >= span) s[sb][r] = -INFINITY;
    }
}

// Second half of tile j: O += P(j) V(j) while the max of S(j+1) is taken.
// The running max is raised (wave-uniformly) only when some row's max
// exceeds it by more than the slack; the caller then rescales O and l.
template <int D>
__device__ __forceinline__ bool pv_max(const uint16_t* __restrict__ vbuf, const int* vaddr,
                                       const bf16x8* pb, f32x16* o, const bf16x8& sel,
                                       f32x4& lacc, const f32x16* s_nxt, float m_run, float sl2,
                                       float& m_new) {
  pv<D>(vbuf, vaddr, pb, o, sel, lacc);
  const float mt = tile_max<D>(s_nxt, sl2);
  interleave_pv_max<D>();
  m_new = fmaxf(m_run, mt);
  return __builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0;
}

// Raise the running max to m_new: O and l scale by 2^(m_run - m_new).
template <int D>
__device__ __forceinline__ void rescale(f32x16* o, f32x4& lacc, float& m_run, float m_new) {
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  lacc *= alpha;
#pragma unroll
  for (int i = 0; i < Frag<D>::DB; ++i) o[i] *= alpha;
  m_run = m_new;
}

// Ring of NS = 4 LDS slots for K and 4 for V (and 4 of the policy's extra
// data), and two wave groups half a tile apart.  Per tile j every wave runs
// [S(j+1) + softmax(j)] then [O += P(j) V(j) + max of S(j+1)]; waves
// 0..NW/2-1 ("leading") take the step's barrier after the second half, waves
// NW/2.. ("lagging") before it, carrying P(j) in registers across the
// barrier.  Between two barriers a leading wave thus runs softmax(j) then
// P(j) V(j) while a lagging wave runs P(j-1) V(j-1) then softmax(j); the two
// waves sharing a SIMD are one of each group, so while one issues the
// softmax's vector work the other keeps the matrix pipe busy.
// Step j starts by issuing K(j+3) into the slot of K(j-1) and V(j+2) into
// the slot of V(j-2), both read by every wave before the previous barrier.
// Only the leading waves issue loads: they finish their half-tiles early and
// would otherwise idle at the barrier, while the lagging waves' softmax is
// the critical path.  The barrier of step j must publish K(j+2) and V(j+1),
// issued in earlier steps: each loading wave waits until no more than this
// step's direct loads are outstanding (vector loads complete in order), then
// the barrier publishes them to all waves.
// The walk runs once per step and yields tile j+4; the tiles in between are
// kept in a four-entry ring in scalar registers (tl), indexed like the K
// slots, from which the loads, the masks and the end test read.  A leading
// wave walks after its P V block, a lagging wave at the step start (after
// its own P V): either way the walk's scalar work stays out of the softmax
// block that bounds the step (walking at the step start in the leading
// waves measured 1-2 % slower).
//
// LDS layout: NS K slots of S::KSLOT<D> bytes, NS V^T slots, NS extra slots
// of S::XSLOT<D> bytes.
template <class S, int D, bool BP>
struct Loop {
  static constexpr uint32_t KSLOT = S::template KSLOT<D>;
  static constexpr uint32_t VSLOT = D * BN * 2;
  static constexpr uint32_t XSLOT = S::template XSLOT<D>;
  static constexpr uint32_t VBASE = NS * KSLOT;
  static constexpr uint32_t XBASE = NS * (KSLOT + VSLOT);
  static constexpr uint32_t LDS_BYTES = NS * (KSLOT + VSLOT + XSLOT);
  // direct loads per loading thread and step: the policy's K loads, V^T
  static constexpr int DMAS = S::template KDMAS<D> + VLoad<D>::PER;
  using Ctx = typename S::template Ctx<D>;

  struct Args {
    const AttnParams& p;
    const Ctx& kc;      // the policy's K loads and score operands
    const VLoad<D>& lc;
    uint16_t* lds;
    int head, rng1, hg;
    float sl2;
    const int* vaddr;
    bf16x8 sel;         // row-sum selector (rowsum_selector)
  };

  static __device__ __forceinline__ const uint16_t* vslot(const uint16_t* lds, int i) {
    return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(lds) + VBASE +
                                             i * VSLOT);
  }

  // First half of tile j: S(j+1) = K(j+1) Q^T (from K slot NK) is issued
  // while the softmax of S(j) runs, producing the bf16 probabilities pb of
  // tile j.  The running max already bounds tile j (it was raised, if
  // needed, while the previous tile's product ran), so the probabilities are
  // at most 2^kRescaleSlack and need no max of their own: one straight-line
  // block of MFMAs and vector work.
  template <int NK>
  static __device__ __forceinline__ void softmax_qk(const Args& a, const f32x16* s_cur,
                                                    f32x16* s_nxt, float m_run, bf16x8* pb) {
    S::template qk<D, NK * KSLOT, XBASE + NK * XSLOT>(a.lds, a.kc, s_nxt);
    probs<D>(s_cur, a.sl2, m_run, pb);
#pragma unroll
    for (int t = 0; t < Frag<D>::PK; ++t) asm volatile("" ::"v"(pb[t]));
    S::template interleave_qk_softmax<D>();
  }

  // Step j with J = j mod NS.  Scores of tile j are in s_cur.  Returns false
  // after the softmax of the last tile (its P V runs after the loop).  On
  // the last tile the S(j+1) product runs on whatever the K slot holds and
  // is discarded (cheaper than a branch in the scheduled block).
  template <int J, bool LAG>
  static __device__ __forceinline__ bool step(const Args& a, Walk& wk, Tile* tl, int& bad_u,
                                              int& bad_v, int& last, f32x16* s_cur,
                                              f32x16* s_nxt, bf16x8* pb, f32x16* o,
                                              float& m_run, f32x4& lacc) {
    const Tile tj = tl[J];   // tile j: its window masks S(j)
    // the page read issued by the last step lands here, before any LDS read
    // is in flight: a pending scalar load inside the compute block would
    // force lgkmcnt(0) at every fragment read
    asm volatile("" ::"s"(wk.page));
    constexpr int JK = (J + 3) % NS;   // the slot of K(j-1) and K(j+3)
    if (!LAG) {
      S::template load_k<D, BP, JK * KSLOT, XBASE + JK * XSLOT>(a.p, a.kc, a.lc.wave_lds, a.head,
                                                                 tl[JK], a.lds, bad_v);
      load_v<D, BP, VBASE + ((J + 2) % NS) * VSLOT>(a.p, a.lc, a.head, tl[(J + 2) % NS], a.lds,
                                                    bad_v);
    } else {
      tl[J] = walk_tile<BP>(a.p, a.rng1, wk, bad_u);   // tile j+4
      walk_next<BP>(a.p, a.rng1, wk);
    }
    if (tile_cut(tj)) {
      int lo, hi;
      tile_window(a.p, tj, lo, hi);
      mask_tile<D>(s_cur, tile_kt(tj), lo, hi, a.hg);
    }
    softmax_qk<(J + 1) % NS>(a, s_cur, s_nxt, m_run, pb);
    if (tl[(J + 1) % NS].ktc < 0) {
      last = J;   // P(j) V(j) of the last tile runs after the loop
      return false;
    }
    const uint16_t* vb = vslot(a.lds, J);
    float m_new;
    if (!LAG) {
      if (pv_max<D>(vb, a.vaddr, pb, o, a.sel, lacc, s_nxt, m_run, a.sl2, m_new))
        rescale<D>(o, lacc, m_run, m_new);
      tl[J] = walk_tile<BP>(a.p, a.rng1, wk, bad_u);   // tile j+4
      walk_next<BP>(a.p, a.rng1, wk);
    }
    // a bare barrier: __syncthreads() would also drain every outstanding
    // load (its fence waits for vmcnt(0)), emptying the ring each step
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // register-path LDS stores
    if (!LAG) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMAS) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (LAG && pv_max<D>(vb, a.vaddr, pb, o, a.sel, lacc, s_nxt, m_run, a.sl2, m_new))
      rescale<D>(o, lacc, m_run, m_new);
    return true;
  }

  template <bool LAG>
  static __device__ __forceinline__ void run(const Args& a, int rng0, f32x16* o, float& m_run,
                                             f32x4& lacc, int& bad_u, int& bad_v) {
    // prologue: the walk's first four tiles, K(0..2), V(0..1), then S(0)
    // and the first running max (step 0 loads K(3))
    Walk wk = walk_first<BP>(a.p, rng0);
    Tile tl[NS];
#define WF_PRO_K(I)                                                                   \
  tl[I] = walk_tile<BP>(a.p, a.rng1, wk, bad_u);                                      \
  walk_next<BP>(a.p, a.rng1, wk);                                                     \
  if (!LAG && (I) < NS - 1)                                                           \
    S::template load_k<D, BP, (I) * KSLOT, XBASE + (I) * XSLOT>(a.p, a.kc, a.lc.wave_lds, \
                                                                 a.head, tl[I], a.lds, bad_v);
    WF_PRO_K(0)
    WF_PRO_K(1)
    WF_PRO_K(2)
    WF_PRO_K(3)
#undef WF_PRO_K
    if (!LAG) {
      load_v<D, BP, VBASE>(a.p, a.lc, a.head, tl[0], a.lds, bad_v);
      load_v<D, BP, VBASE + VSLOT>(a.p, a.lc, a.head, tl[1], a.lds, bad_v);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[Frag<D>::SB], sb[Frag<D>::SB];
    S::template qk<D, 0, XBASE>(a.lds, a.kc, sa);
    if (tile_cut(tl[0])) {
      int lo, hi;
      tile_window(a.p, tl[0], lo, hi);
      mask_tile<D>(sa, tile_kt(tl[0]), lo, hi, a.hg);
    }
    // finite floor: a row with no visible key in the first tile keeps exact
    // zero probabilities instead of -inf - -inf
    m_run = fmaxf(tile_max<D>(sa, a.sl2), -1e30f);
    // both wave groups enter the loop together (the lagging group falls
    // half a tile behind at its first barrier)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8 pb[Frag<D>::PK];
    int last = 0;
    while (true) {
#define WF_STEP(J, SC, SN)                                                                   \
  if (!step<J, LAG>(a, wk, tl, bad_u, bad_v, last, SC, SN, pb, o, m_run, lacc)) break;
      WF_STEP(0, sa, sb)
      WF_STEP(1, sb, sa)
      WF_STEP(2, sa, sb)
      WF_STEP(3, sb, sa)
#undef WF_STEP
    }
    pv<D>(vslot(a.lds, last), a.vaddr, pb, o, a.sel, lacc);
    // no LDS-DMA may still be in flight when the block ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

// The kernel body: work item, the policy's operands (S::setup), the loop of
// both wave groups, the bad-page status, and O = O^T / l with the LSE.
// X is the policy's extra kernel argument (the MXFP8 key scales).
template <class S, int D, bool BP>
__device__ __forceinline__ void attn_body(const AttnParams& p, const typename S::Extra& x,
                                          uint16_t* lds) {
  using L = Loop<S, D, BP>;
  constexpr int DB = Frag<D>::DB, PK = Frag<D>::PK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hg = lane >> 5;

  // ---- work item: XCD-contiguous runs, longest first within each --------
  const int w = xcd_work_item(p, blockIdx.x, gridDim.x);
  const int head = w / p.tiles_per_head;
  const int tw = w - head * p.tiles_per_head;
  int grp = 0;
  while (tw >= p.grp_tile_end[grp]) ++grp;
  const int qtile = tw - (grp ? p.grp_tile_end[grp - 1] : 0);
  const int row_end = p.grp_row1[grp];
  const int qrow = p.grp_row0[grp] + qtile * BM + wave * 32 + ql;
  const bool qvalid = qrow < row_end;
  const int rng0 = p.grp_rng0[grp], rng1 = p.grp_rng1[grp];

  // per-lane LDS element offsets of the V^T A-operand reads
  int vaddr[PK];
  {
    const int vu = hg ^ vswz(ql);
#pragma unroll
    for (int t = 0; t < PK; ++t) vaddr[t] = ql * BN + ((2 * t) ^ vu) * 8;
  }

  // the policy's score operands and K load addressing (query fragments,
  // A-operand offsets, key pages) for loading thread lq of the leading waves
  const int lq = (wave % (LT / 64)) * 64 + lane;
  const uint32_t wave_lds =
      (uint32_t)(uintptr_t)lds + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  typename S::template Ctx<D> kc;
  S::template setup<D>(p, x, head, qrow, qvalid, wave, ql, hg, lq, wave_lds, lds, kc);

  // block-constant V^T load addressing: feature row d0 + i*LT/8 of a loading
  // thread keeps the swizzle of row d0 (a multiple of 16 rows further)
  VLoad<D> lc;
  {
    const int ps = 1 << p.ps_log2;
    lc.v_head = static_cast<const char*>(p.v_pages) + (int64_t)head * ps * D * 2;
    lc.page_bytes = (int64_t)p.heads * ps * D * 2;
    static_assert((LT / 8) % 16 == 0, "chunk rows keep their swizzle");
    const int d0 = lq >> 3, vcol = (lq & 7) ^ vswz(d0);
#pragma unroll
    for (int i = 0; i < VLoad<D>::PER; ++i)
      lc.voff[i] = (uint32_t)((d0 + i * (LT / 8)) * ps + vcol * 8) * 2u;
    lc.wave_lds = wave_lds;
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run;               // running max of scale*log2(e)*<q,k>
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};   // row sums of P (every register: the lane's query)
  int bad_u = 0, bad_v = 0;  // bad page entries: wave-uniform and per-lane
  const typename L::Args args{p, kc, lc, lds, head, rng1, hg, p.scale_log2, vaddr,
                              rowsum_selector(lane)};
  // waves NW/2.. run half a tile behind (see Loop)
  if (wave >= NW / 2)
    L::template run<true>(args, rng0, o, m_run, lacc, bad_u, bad_v);
  else
    L::template run<false>(args, rng0, o, m_run, lacc, bad_u, bad_v);
  // one status write per wave that met a bad page entry (per-lane lookups
  // of the register path included)
  if ((bad_u | (__builtin_amdgcn_ballot_w64(bad_v != 0) != 0)) && lane == 0)
    atomicOr(p.status, WF_STATUS_BAD_PAGE);

  // ---- epilogue: O = O^T / l, LSE ------------------------------------------
  const float l = lacc[0];
  const float inv = 1.0f / l;
  if (qvalid) {
    uint16_t* op = static_cast<uint16_t*>(p.out) + (int64_t)qrow * p.out_stride + head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // registers 4j..4j+3 of block db: d = 32db + 8j + 4hg + 0..3
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * j + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hg) = v;
      }
    if (p.lse && hg == 0)
      p.lse[(int64_t)head * p.lse_stride + qrow] = (m_run + __log2f(l)) * kLn2;
  }
}

}  // namespace attn
}  // namespace wf

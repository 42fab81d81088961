// wf_chunk_attn, bfloat16: slot-masked flash-attention forward over the paged
// K/V pool on CDNA4 matrix cores.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §3.1:
// a query of denoising slot s attends to the anchor, the clean history, the
// live store and every slot j >= s (itself included, with full attention
// inside the chunk).  The host turns that rule into a list of merged visible
// key ranges per slot; this kernel walks only the key tiles those ranges
// touch, so tiles the mask removes entirely are never loaded or multiplied.
//
// Work unit: one block = (head, slot, 256-row query tile), 8 waves of 64
// lanes, each wave owning 32 query rows; every K/V tile brought into LDS
// serves all 256 rows, which halves the L2 -> CU traffic of 128-row tiles.
// Per 64-key tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T held
//                 in registers for the whole kernel.  The transposed product
//                 puts one query in every lane (lanes l and l+32 share it),
//                 so row max / row sum need a single cross-half exchange.
//   mask          only on tiles cut by a range boundary: keys outside the
//                 range become -inf; their K/V rows are never read from HBM
//                 (zero-filled in LDS), so stale or NaN memory cannot leak.
//   softmax       online, base 2, with the running max raised only when a
//                 row's tile max exceeds it by more than 2^8 (the exact
//                 result is unchanged: numerator and denominator share the
//                 stale max, and 2^8 keeps every term finite).  The
//                 denominator sums the bf16-rounded probabilities that
//                 multiply V (v_dot2 against 1.0), so the weights applied to
//                 V are normalized exactly.
//   O^T += V^T P^T  A = V^T read from the d-major V pages via LDS, B = P^T
//                 straight from the S^T accumulators: the K rows of S^T are
//                 loaded in the order sigma(i) (bits 2 and 3 of the row index
//                 swapped) so that each lane's 8 probabilities of a k-step
//                 are 8 consecutive keys, matching a 16-byte V^T read.
//
// Pipeline: K runs one tile ahead of V in two LDS double buffers.  While the
// softmax of tile j runs on the VALU, the MFMAs of S(j+1) = K(j+1) Q^T are
// already issued; the direct global->LDS loads (global_load_lds_dwordx4) of
// K(j+2) and V(j+1) are in flight during both.  One barrier per tile.  Tiles
// cut by a range boundary, spread over several pages or naming a bad page
// take a register path that zero-fills what lies outside the window.
//
// LDS layout: 16-byte chunks XOR-swizzled by row so that the A-operand reads
// of 8 (or 16) consecutive lanes hit distinct banks: K chunk c of row r sits
// at column c ^ kswz(r); V^T chunk c of feature row d at column c ^ vswz(d).
//
// Block ids are remapped so that each XCD (blocks are dealt round-robin over
// the 8 XCDs) receives a contiguous run of the work list: the query tiles of
// one head and slot then share that XCD's L2 while streaming the same keys.
#include "../../include/wf.h"
#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 8;       // waves per block, 32 query rows each
constexpr int BM = 32 * NW; // query rows per block
constexpr int BN = 64;      // keys per tile
constexpr int NT = 64 * NW; // threads per block
constexpr int kStages = 4;  // LDS ring slots for K and for V
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

// column swizzles (16-byte chunk units)
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return ((((r & 7) ^ ((r >> 1) & 4)) | (r & 8)) & (D / 8 - 1));
}
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 1); }

// Physical page of logical token L, or -1 (and `bad` set) for an entry
// outside the pool.  The status word is written once, after the key loop.
__device__ __forceinline__ int check_page(const AttnParams& p, int page, int& bad) {
  if (page < 0 || page >= p.num_pages) {
    bad = 1;
    return -1;
  }
  return page;
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

// Position of the tile walk over the merged visible ranges of one group.
// The bounds of the current range and the physical page of the tile are
// kept with it, so advancing is arithmetic plus one scalar read, issued a
// step before the tile is loaded.
struct Cursor {
  int ri;     // current range; == rng1 once past the last tile
  int kt;     // first key of the tile (multiple of BN)
  int rlo;    // range [rlo, rhi)
  int rhi;
  int page;   // physical page of the tile when pages hold >= BN keys
};

__device__ __forceinline__ void cursor_page(const AttnParams& p, Cursor& c) {
  if (p.ps_log2 >= 6) c.page = table_entry(p, c.kt >> p.ps_log2);
}

__device__ __forceinline__ Cursor cursor_first(const AttnParams& p, int rng0) {
  const int2 r = p.ranges[rng0];
  Cursor c{rng0, r.x & ~(BN - 1), r.x, r.y, -1};
  cursor_page(p, c);
  return c;
}

__device__ __forceinline__ Cursor cursor_next(const AttnParams& p, int rng1, Cursor c) {
  c.kt += BN;
  if (c.kt >= c.rhi) {
    ++c.ri;
    if (c.ri >= rng1) return c;
    const int2 r = p.ranges[c.ri];
    c.rlo = r.x;
    c.rhi = r.y;
    c.kt = r.x & ~(BN - 1);
  }
  cursor_page(p, c);
  return c;
}

// keys [lo, hi) of the tile at cursor c that lie in its range
__device__ __forceinline__ void cursor_window(const AttnParams& p, Cursor c, int& lo, int& hi) {
  lo = max(c.kt, c.rlo);
  hi = min(c.kt + BN, c.rhi);
}

// A wave-uniform pointer, placed in scalar registers (so that a load of
// base + per-lane 32-bit offset uses the scalar-base addressing form)
__device__ __forceinline__ const char* uniform_ptr(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Direct global->LDS load, 16 bytes per lane (global_load_lds_dwordx4, the
// scalar-base form): lane i writes LDS bytes [lds_dst + 16 i, +16).  Issued
// as inline assembly so that the compiler does not model it: with this
// LDS-DMA form in the loop its wait bookkeeping drains every later LDS read
// with lgkmcnt(0), which serializes the A-operand fragment reads.  The
// caller's explicit vmcnt waits track completion.  The wait states cover a
// base just written by v_readfirstlane (VALU write of an SGPR read by a
// memory instruction) and the M0 write read by the LDS-DMA load.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst);
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(m0)
      : "memory", "m0");
}

// ---- global -> LDS: the K tile [BN][D] of one head ------------------------
// Returns the number of direct global->LDS loads this thread issued, or 0
// when the register path ran (it waits for every older load as well).
template <int D>
__device__ __forceinline__ int load_k(const AttnParams& p, int head, Cursor c,
                                      uint16_t* __restrict__ kbuf, int& bad) {
  constexpr int CPR = D / 8;               // chunks per K row
  constexpr int PER = BN * CPR / NT;       // chunks per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ps = 1 << p.ps_log2;
  int lo, hi;
  cursor_window(p, c, lo, hi);
  const int kt = c.kt;
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(p.k_pages);
  const bool one_page = p.ps_log2 >= 6;    // a 64-aligned tile lies in one page
  const int tile_page = one_page ? check_page(p, c.page, bad) : -1;
  if (one_page && tile_page >= 0 && lo == kt && hi == kt + BN) {
    // chunk i of this thread is row r0 + i*NT/CPR (a multiple of 16 rows
    // further, so the same swizzled column): one lane offset serves every
    // chunk, and the per-chunk step goes into the uniform (scalar) base
    const char* kb = reinterpret_cast<const char*>(
        kpg + (((int64_t)tile_page * p.heads + head) * ps + (kt & (ps - 1))) * D);
    const int q = wave * 64 + lane;
    const int r0 = q / CPR, col = (q % CPR) ^ kswz<D>(r0);
    const uint32_t loff = (uint32_t)(r0 * D + col * 8) * 2u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const char* base = uniform_ptr(kb + i * (NT / CPR) * D * 2);
      dma16(base, loff, kbuf + (i * NW + wave) * 64 * 8);
    }
    return PER;
  }
  // rare (tile cut by a range boundary, or pages smaller than a tile): one
  // chunk at a time, to keep register pressure off the hot loop
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll 1
  for (int i = 0; i < PER; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    const int r = q / CPR, col = (q % CPR) ^ kswz<D>(r);
    const int L = kt + r;
    uint4 val = zero;
    if (L >= lo && L < hi) {
      const int page = one_page ? tile_page : lookup_page(p, L, bad);
      if (page >= 0)
        val = *reinterpret_cast<const uint4*>(
            kpg + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * D + col * 8);
    }
    *reinterpret_cast<uint4*>(kbuf + q * 8) = val;
  }
  return 0;
}

// ---- global -> LDS: the V^T tile [D][BN] of one head -----------------------
template <int D>
__device__ __forceinline__ int load_v(const AttnParams& p, int head, Cursor c,
                                      uint16_t* __restrict__ vbuf, int& bad) {
  constexpr int PER = D * (BN / 8) / NT;   // chunks per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ps = 1 << p.ps_log2;
  int lo, hi;
  cursor_window(p, c, lo, hi);
  const int kt = c.kt;
  const uint16_t* __restrict__ vpg = static_cast<const uint16_t*>(p.v_pages);
  const bool one_page = p.ps_log2 >= 6;
  const int tile_page = one_page ? check_page(p, c.page, bad) : -1;
  if (one_page && tile_page >= 0 && lo == kt && hi == kt + BN) {
    // chunk i of this thread is feature row d0 + i*NT/8 (same swizzle):
    // one lane offset, the per-chunk step in the uniform base
    const char* vb = reinterpret_cast<const char*>(
        vpg + ((int64_t)tile_page * p.heads + head) * D * ps + (kt & (ps - 1)));
    const int q = wave * 64 + lane;
    const int d0 = q >> 3, col = (q & 7) ^ vswz(d0);
    const uint32_t loff = (uint32_t)(d0 * ps + col * 8) * 2u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const char* base = uniform_ptr(vb + (int64_t)i * (NT / 8) * ps * 2);
      dma16(base, loff, vbuf + (i * NW + wave) * 64 * 8);
    }
    return PER;
  }
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll 1
  for (int i = 0; i < PER; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    const int d = q >> 3, col = (q & 7) ^ vswz(d);
    const int L = kt + col * 8;              // first of the chunk's 8 keys
    uint4 val = zero;
    if (L + 8 > lo && L < hi) {
      // an 8-key run never crosses a page (page_size >= 16, runs 8-aligned)
      const int page = one_page ? tile_page : lookup_page(p, max(L, lo), bad);
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
  return 0;
}

template <int D>
struct Frag {
  static constexpr int DK = D / 16;   // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  static constexpr int SB = BN / 32;  // 32-key blocks of S^T
  static constexpr int PK = BN / 16;  // k-steps of O^T += V^T P^T
};

// S^T of one tile: s[sb] for keys 32sb.. of the K slot
template <int D>
__device__ __forceinline__ void qk(const uint16_t* __restrict__ kbuf, const int* kaddr,
                                   const bf16x8* qf, f32x16* s) {
#pragma unroll
  for (int sb = 0; sb < Frag<D>::SB; ++sb) {
    s[sb] = f32x16{};
#pragma unroll
    for (int i = 0; i < Frag<D>::DK; ++i) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf + kaddr[i] + 32 * sb * D);
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i], s[sb], 0, 0, 0);
    }
  }
}

// bf16 probabilities of one tile for running max m, and their sum (over the
// rounded values, via v_dot2 against 1.0)
template <int D>
__device__ __forceinline__ void probs(const f32x16* s, float sl2, float m, bf16x8* pb,
                                      float* lsum) {
  const float neg_m = -m;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  lsum[0] = 0.f;
  lsum[1] = 0.f;
#pragma unroll
  for (int t = 0; t < Frag<D>::PK; ++t) {
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * j], sl2, neg_m)),
                       __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * j + 1], sl2, neg_m))};
      const bf16x2 b = __builtin_convertvector(x, bf16x2);
      pk[j] = __builtin_bit_cast(uint32_t, b);
      lsum[j & 1] = __builtin_amdgcn_fdot2_f32_bf16(b, ones, lsum[j & 1], false);
    }
    pb[t] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  }
}

template <int D>
__device__ __forceinline__ void pv(const uint16_t* __restrict__ vbuf, const int* vaddr,
                                   const bf16x8* pb, f32x16* o) {
#pragma unroll
  for (int t = 0; t < Frag<D>::PK; ++t)
#pragma unroll
    for (int db = 0; db < Frag<D>::DB; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vbuf + vaddr[t] + 32 * db * BN);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
    }
}

// Instruction-scheduling hint for the block that issues the S(j+1) MFMAs and
// the softmax of tile j: K reads run a few ahead, and every MFMA is followed
// by a share of the VALU work, so the matrix pipe and the VALU run together.
template <int D>
__device__ __forceinline__ void interleave_qk_softmax() {
  constexpr int NM = Frag<D>::SB * Frag<D>::DK;   // MFMAs of S(j+1)
  constexpr int AHEAD = 3;
  constexpr int VPM = 7;                           // VALU per MFMA
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
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

// One tile: S(j+1) = K(j+1) Q^T is issued while the softmax of S(j) runs,
// then O += V(j)^T P(j)^T.  The running max is raised (wave-uniformly) only
// when some row's tile max exceeds it by more than the slack; that decision
// is a select, so the probabilities are computed in the same straight-line
// block as the S(j+1) MFMAs, and only the rare rescale of O and l branches.
template <int D>
__device__ __forceinline__ void compute_tile(const uint16_t* __restrict__ kb_next,
                                             const uint16_t* __restrict__ vb_cur,
                                             const int* kaddr, const int* vaddr,
                                             const bf16x8* qf, f32x16* s_cur, f32x16* s_nxt,
                                             f32x16* o, float& m_run, float* l_acc,
                                             float sl2) {
  constexpr int SB = Frag<D>::SB, PK = Frag<D>::PK, DB = Frag<D>::DB;
  qk<D>(kb_next, kaddr, qf, s_nxt);
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[sb][r]);
  const float mt = xhalf_max(mx) * sl2;
  const bool raise = __builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0;
  const float m_new = raise ? fmaxf(m_run, mt) : m_run;
  bf16x8 pb[PK];
  float lsum[2];
  probs<D>(s_cur, sl2, m_new, pb, lsum);
  // pin the probabilities above the rescale branch: without a use here the
  // compiler sinks them below it, out of the block of the S(j+1) MFMAs
#pragma unroll
  for (int t = 0; t < PK; ++t) asm volatile("" ::"v"(pb[t]));
  asm volatile("" ::"v"(lsum[0]), "v"(lsum[1]));
  interleave_qk_softmax<D>();
  if (raise) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_acc[0] *= alpha;
    l_acc[1] *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  l_acc[0] += lsum[0];
  l_acc[1] += lsum[1];
  pv<D>(vb_cur, vaddr, pb, o);
}

// s_waitcnt vmcnt(n) for a wave-uniform n; values beyond the table wait for
// more than needed, which is always safe
__device__ __forceinline__ void wait_vmcnt(int n) {
  if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Ring of NS LDS slots for K and NS for V.  At tile j the slots hold
// K(j+1..j+NS) and V(j..j+NS-1); step j issues K(j+NS) into the slot of K(j)
// and V(j+NS-1) into the slot of V(j-1), both read by every wave before the
// previous barrier, so each load has NS-1 steps to land.  The end of step j
// needs only K(j+2) and V(j+1), issued NS-2 steps earlier: it waits until
// no more than the direct loads issued since then are outstanding (vector
// loads complete in order), then one barrier publishes them to all waves.
template <int D, int NS>
struct Loop {
  static constexpr int KT = BN * D;   // elements of one K tile slot
  static constexpr int VT = D * BN;   // elements of one V^T tile slot

  // Step j with J = j mod NS.  Scores of tile j are in s_cur.  Returns false
  // after the last tile.  On the last tile the S(j+1) product runs on
  // whatever the K slot holds and is discarded (cheaper than a branch in
  // the scheduled block).
  template <int J>
  static __device__ __forceinline__ bool step(const AttnParams& p, uint16_t* lds, int head,
                                              int rng1, Cursor& cc, Cursor& ck, Cursor& cv,
                                              int& n_prev, int& n_cur, int& bad,
                                              const int* kaddr, const int* vaddr,
                                              const bf16x8* qf, f32x16* s_cur, f32x16* s_nxt,
                                              f32x16* o, float& m_run, float* l_acc, int hg,
                                              float sl2) {
    uint16_t* kb = lds;
    uint16_t* vb = lds + NS * KT;
    n_prev = n_cur;
    n_cur = 0;
    if (ck.ri < rng1) {
      const int n = load_k<D>(p, head, ck, kb + J * KT, bad);
      if (n) n_cur += n;
      else n_prev = n_cur = 0;
      ck = cursor_next(p, rng1, ck);
    }
    if (cv.ri < rng1) {
      const int n = load_v<D>(p, head, cv, vb + ((J + NS - 1) % NS) * VT, bad);
      if (n) n_cur += n;
      else n_prev = n_cur = 0;
      cv = cursor_next(p, rng1, cv);
    }
    // let the page-table reads of the next step land here (scalar-cache
    // hits): the use pins them above the compute block, where a pending
    // scalar load would force lgkmcnt(0) at every LDS read
    asm volatile("" ::"s"(ck.page), "s"(cv.page));
    int w_lo, w_hi;
    cursor_window(p, cc, w_lo, w_hi);
    if (w_lo > cc.kt || w_hi < cc.kt + BN) mask_tile<D>(s_cur, cc.kt, w_lo, w_hi, hg);
    compute_tile<D>(kb + ((J + 1) % NS) * KT, vb + J * VT, kaddr, vaddr, qf, s_cur, s_nxt, o,
                    m_run, l_acc, sl2);
    cc = cursor_next(p, rng1, cc);
    if (cc.ri >= rng1) return false;
    // a bare barrier: __syncthreads() would also drain every outstanding
    // load (its fence waits for vmcnt(0)), emptying the ring each step
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // register-path LDS stores
    wait_vmcnt(NS >= 4 ? n_prev + n_cur : (NS == 3 ? n_cur : 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    return true;
  }

  static __device__ __forceinline__ void run(const AttnParams& p, uint16_t* lds, int head,
                                             int rng0, int rng1, const int* kaddr,
                                             const int* vaddr, const bf16x8* qf, f32x16* o,
                                             float& m_run, float* l_acc, int hg, float sl2,
                                             int& bad) {
    uint16_t* kb = lds;
    uint16_t* vb = lds + NS * KT;
    // prologue: K(0..NS-1) and V(0..NS-2), then S(0)
    Cursor cc = cursor_first(p, rng0);
    Cursor ck = cc, cv = cc;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (ck.ri < rng1) {
        load_k<D>(p, head, ck, kb + i * KT, bad);
        ck = cursor_next(p, rng1, ck);
      }
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      if (cv.ri < rng1) {
        load_v<D>(p, head, cv, vb + i * VT, bad);
        cv = cursor_next(p, rng1, cv);
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[Frag<D>::SB], sb[Frag<D>::SB];
    qk<D>(kb, kaddr, qf, sa);
    // step 0 loads K(NS) into the slot of K(0): every wave must have read
    // K(0) first (write-after-read across waves)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int n_prev = 0, n_cur = 0;
    while (true) {
#define WF_STEP(J, SC, SN)                                                                   \
  if (J < NS && !step<J % NS>(p, lds, head, rng1, cc, ck, cv, n_prev, n_cur, bad, kaddr,     \
                              vaddr, qf, SC, SN, o, m_run, l_acc, hg, sl2))                  \
    break;
      WF_STEP(0, sa, sb)
      WF_STEP(1, sb, sa)
      WF_STEP(2, sa, sb)
      WF_STEP(3, sb, sa)
#undef WF_STEP
      static_assert(NS == 2 || NS == 4, "the unrolled ring assumes an even slot count <= 4");
    }
    // no LDS-DMA may still be in flight when the block ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

template <int D, int NS>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const AttnParams p) {
  constexpr int DK = Frag<D>::DK, DB = Frag<D>::DB, PK = Frag<D>::PK;
  constexpr int KT = Loop<D, NS>::KT, VT = Loop<D, NS>::VT;
  __shared__ __attribute__((aligned(16))) uint16_t lds[NS * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, hg = lane >> 5;

  // ---- work item: XCD-contiguous remap of the block id --------------------
  const int nb = gridDim.x, b = blockIdx.x;
  const int per = nb >> 3;
  const int w = (b < (per << 3)) ? ((b & 7) * per + (b >> 3)) : b;
  const int head = w / p.tiles_per_head;
  const int tw = w - head * p.tiles_per_head;
  int grp = 0;
  while (tw >= p.grp_tile_end[grp]) ++grp;
  const int qtile = tw - (grp ? p.grp_tile_end[grp - 1] : 0);
  const int row_end = p.grp_row1[grp];
  const int qrow = p.grp_row0[grp] + qtile * BM + wave * 32 + ql;
  const bool qvalid = qrow < row_end;
  const int rng0 = p.grp_rng0[grp], rng1 = p.grp_rng1[grp];

  // lane (query ql, half hg) holds d = 16i+8hg..+8 of its query
  bf16x8 qf[DK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (int64_t)qrow * p.q_stride +
                         head * D + 8 * hg;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * i) : make_uint4(0, 0, 0, 0);
      qf[i] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // per-lane LDS element offsets of the A-operand reads
  int kaddr[DK], vaddr[PK];
  {
    const int kr = sigma(ql);
    const int ku = hg ^ kswz<D>(kr);
#pragma unroll
    for (int i = 0; i < DK; ++i) kaddr[i] = kr * D + ((2 * i) ^ ku) * 8;
    const int vu = hg ^ vswz(ql);
#pragma unroll
    for (int t = 0; t < PK; ++t) vaddr[t] = ql * BN + ((2 * t) ^ vu) * 8;
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*<q,k>
  float l_acc[2] = {0.f, 0.f};
  int bad = 0;
  Loop<D, NS>::run(p, lds, head, rng0, rng1, kaddr, vaddr, qf, o, m_run, l_acc, hg,
                   p.scale_log2, bad);
  if (bad && threadIdx.x == 0) atomicOr(p.status, WF_STATUS_BAD_PAGE);

  // ---- epilogue: O = O^T / l, LSE ------------------------------------------
  const float l = xhalf_sum(l_acc[0] + l_acc[1]);
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

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int block_m,
                            hipStream_t stream) {
  if (block_m != BM) return hipErrorInvalidValue;
  dim3 grid(p.tiles_per_head * p.heads), block(NT);
  if (head_dim == 128) hipLaunchKernelGGL((attn_fwd_bf16<128, kStages>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((attn_fwd_bf16<64, kStages>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace wf

// wf_qkv_publish kernel: the QKV projection of a chunk's hidden states on
// bf16 MFMA, with the publish fused into its epilogue.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §4.2:
// K/V are published right after the QKV projection and RoPE.  Fusing the
// publish into the projection's epilogue means the projected K and V are
// rotated and scattered into the paged pool straight from the accumulators:
// they are never written to HBM as a dense tensor and read back.
//
// Product: C^T[f][t] = sum_k W[f][k] x[t][k] for output feature f and token
// t, v_mfma_f32_32x32x16_bf16 with A = W rows and B = x rows (both
// contiguous in k).  The transposed product puts one token in every lane and
// a run of 4 consecutive features in 4 consecutive accumulator registers, so
// a RoPE pair (2i, 2i+1) is two registers of one lane.
//
// Block: 256 features (two heads) x 256 tokens, 8 waves of 128 features (one
// head) x 64 tokens, eight 32x32 accumulators per wave (two waves per SIMD).
// Per k-step of 16 a wave reads 6 fragments for 8 products.  k-tiles of 32
// go straight from global memory into a four-slot LDS ring
// (global_load_lds_dwordx4, three tiles in flight, 32 KB per tile), issued
// by one wave per SIMD while the other keeps the matrix pipe fed; 16-byte
// chunks of the 64-byte rows XOR-swizzled so that the fragment reads of 16
// consecutive rows hit distinct banks; one barrier per k-tile.  Per CU and
// clock the block needs 32 bytes of L2 traffic at the full matrix rate, half
// of what a 128 x 256 block needs, against the ~64 B/clk an MI355X CU fills
// from its L2.  Blocks are dealt to the XCDs in contiguous runs of 4 feature
// x 8 token tiles (qkv_tile in wf_qkv.h).
//
// Rotary factors: for the video layout a block's 256 tokens take few
// distinct positions per axis, so the block evaluates the factors once per
// (pair, position) present - the per-axis position ranges of its tokens -
// into an LDS table while its first tiles load; the epilogue then looks them
// up.  Positions spread too widely for the table fall back to evaluating the
// factors per element (same values, more time).
//
// Epilogue per element: + bias, round to bf16 (the unfused projection's
// output), then for Q and K the rotation of wf_kv_publish (double-precision
// angle and cos/sin rounded to float, float products and sums without fused
// multiply-add, round to bf16).  The results are staged in the ring's LDS,
// one wave's 64 tokens of one head at a time, and re-read in the output's own
// order, so that every global store is 16 bytes: Q rows, K page rows (256
// contiguous bytes per token) and V page columns (8 consecutive tokens of a
// feature, d-major).
#include "../../include/wf.h"
#include "wf_numerics.h"
#include "wf_qkv.h"

namespace wf {
namespace {

constexpr int BM = kQkvBlockFeat;          // 256 features per block
constexpr int BN = kQkvBlockTok;           // 256 tokens per block
constexpr int D = 128;                     // head_dim
constexpr int TK = 32;                     // hidden elements per k-tile
constexpr int NTH = 512;                   // 8 waves: 2 heads x 4 token quarters
constexpr int NSL = 4;                     // LDS ring slots
constexpr int ROWB = TK * 2;               // bytes per tile row: 64
constexpr int A_BYTES = BM * ROWB;         // 16 KB of W rows per tile
constexpr int B_BYTES = BN * ROWB;         // 16 KB of x rows per tile
constexpr int SLOT = A_BYTES + B_BYTES;    // 32 KB
constexpr int RING = NSL * SLOT;           // 128 KB
#ifndef WF_QKV_LW
#define WF_QKV_LW 4
#endif
constexpr int LW = WF_QKV_LW;                 // waves that issue the tile loads (one per SIMD)
constexpr int A_DMA = A_BYTES / (LW * 64 * 16);  // 16-byte loads per loading thread per tile: 4
constexpr int B_DMA = B_BYTES / (LW * 64 * 16);  // 4
constexpr int DMAS = A_DMA + B_DMA;
constexpr int NPAIR = D / 2;
// past the ring: the positions of the block's tokens (int4 per token), the
// per-wave position minima/maxima, the per-pair table row bases, then the
// (cos, sin) table; the whole LDS is 160 KB
constexpr int POS_OFF = RING;                  // int4[BN]
constexpr int HDR_OFF = POS_OFF + BN * 16;     // int[32]: 4 waves x (3 minima, 3 maxima)
constexpr int RB_OFF = HDR_OFF + 32 * 4;       // int[NPAIR]
constexpr int TAB_OFF = RB_OFF + NPAIR * 4;
constexpr int LDS_BYTES = 160 * 1024;
constexpr int TAB_CAP = (LDS_BYTES - TAB_OFF) / 8;
static_assert(A_DMA * LW * 1024 == A_BYTES && B_DMA * LW * 1024 == B_BYTES && 16 % DMAS == 0,
              "whole 1 KB runs per loading wave; loads spread evenly over a tile's 16 products");
static_assert(2 * 64 * D * 2 <= RING && 2 * D * BN * 2 <= RING, "staging fits in the ring");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Direct global->LDS load, 16 bytes per lane: lane i writes LDS bytes
// [M0 + 16 i, +16) with M0 = lds + OFF (inline assembly, so that the
// compiler's wait bookkeeping leaves the fragment reads alone; completion is
// tracked by the explicit vmcnt waits).  The wait states cover an SGPR base
// written just before (5) and the M0 write (1).
template <uint32_t OFF>
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 4\n\t"
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds), "i"(OFF)
      : "memory", "m0", "scc");
}

// Fragments of one k-tile for a wave: A = W rows 128 wm + 32 i + ql (i < 4),
// B = x rows 64 wn + 32 j + ql (j < 2), for the two k-steps; `ra` and `rb`
// are the lane's row bases in the slot, xo[ks] its swizzled chunk offset.
struct Frags {
  bf16x8 a[2][4], b[2][2];
};

// one fragment read of the 12 of a tile (n < 12): k-step n / 6, then
// A 0..3, B 0..1
template <int N>
__device__ __forceinline__ void read_frag(Frags& f, const char* slot, int ra, int rb,
                                          const int* xo) {
  constexpr int ks = N / 6, r = N % 6;
  if constexpr (r < 4)
    f.a[ks][r] = *reinterpret_cast<const bf16x8*>(slot + ra + xo[ks] + r * 32 * ROWB);
  else
    f.b[ks][r - 4] = *reinterpret_cast<const bf16x8*>(slot + rb + xo[ks] + (r - 4) * 32 * ROWB);
}

// product n of the 16 of a tile: k-step n / 8, accumulator (i, j) = n % 8
template <int N>
__device__ __forceinline__ void mma(const Frags& f, f32x16 (&acc)[4][2]) {
  constexpr int ks = N / 8, i = (N % 8) / 2, j = N % 2;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][i], f.b[ks][j], acc[i][j], 0, 0, 0);
}

// A wave-uniform pointer, held in scalar registers: the base operand of the
// direct loads must be a scalar register pair, which the compiler cannot
// choose on its own once it has placed the value in vector registers.
__device__ __forceinline__ const char* uniform_ptr(const char* q) {
  const uint64_t u = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// the scheduler keeps the source order across this point
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = min(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ int axis_of(const QkvParams& p, int pr) {
  return (pr >= p.band0[1]) + (pr >= p.band0[2]);
}

// Loads of tile m into ring slot m % 4 (M0 base `dst` = this wave's 1 KB
// of the slot).  Tiles past the last one re-load the last tile into a slot
// no step reads again, so every step issues the same loads and the wait
// counts are constants.
// load n of a loading thread's DMAS per tile: W rows first, then x rows;
// instruction u of loading wave lw fills the 1 KB run LW u + lw of its
// operand
template <int N>
__device__ __forceinline__ void dma_n(const char* wbase, const char* xbase, int kb,
                                      const uint32_t* aoff, const uint32_t* boff, uint32_t dst) {
  if constexpr (N < A_DMA)
    dma16<N * LW * 1024>(wbase + kb, aoff[N], dst);
  else
    dma16<A_BYTES + (N - A_DMA) * LW * 1024>(xbase + kb, boff[N - A_DMA], dst);
}

template <int N = 0>
__device__ __forceinline__ void dma_all(const char* wbase, const char* xbase, int kb,
                                        const uint32_t* aoff, const uint32_t* boff, uint32_t dst) {
  if constexpr (N < DMAS) {
    dma_n<N>(wbase, xbase, kb, aoff, boff, dst);
    dma_all<N + 1>(wbase, xbase, kb, aoff, boff, dst);
  }
}

__device__ __forceinline__ void load_tile_at(const char* wbase, const char* xbase, int m,
                                             int ktiles, const uint32_t* aoff,
                                             const uint32_t* boff, uint32_t wave_lds) {
  const int kb = min(m, ktiles - 1) * TK * 2;
  const uint32_t dst = wave_lds + (uint32_t)(m % NSL) * SLOT;
  dma_all(wbase, xbase, kb, aoff, boff, dst);
}

// the 16 products of the tile whose fragments are in `cur`
__device__ __forceinline__ void mma_all(const Frags& cur, f32x16 (&acc)[4][2]) {
  mma<0>(cur, acc); mma<1>(cur, acc); mma<2>(cur, acc); mma<3>(cur, acc);
  mma<4>(cur, acc); mma<5>(cur, acc); mma<6>(cur, acc); mma<7>(cur, acc);
  mma<8>(cur, acc); mma<9>(cur, acc); mma<10>(cur, acc); mma<11>(cur, acc);
  mma<12>(cur, acc); mma<13>(cur, acc); mma<14>(cur, acc); mma<15>(cur, acc);
}

// Step kt < ktiles - 1 of the k-loop (B = kt % 2: fragment buffer B holds
// tile kt, the other one receives tile kt+1).  Tile kt+1 is done for a
// loading thread when only the loads of tiles kt+2 and kt+3 are in flight,
// and this wave's reads of tile kt are done; after the barrier tile kt+1 is
// visible and tile kt's slot is free for tile kt+4.  Only the loading waves
// (LD, one per SIMD) issue loads: a direct-to-LDS load holds its wave at
// issue, and the other wave of the SIMD keeps the matrix pipe fed meanwhile.
// The loads go one every 16 / DMAS products, so that the CU's load path sees
// an even stream instead of a burst after the barrier; the 12 fragment reads
// of tile kt+1 go in between the first products.
template <bool LD, int M>
__device__ __forceinline__ void after_mma(const char* wbase, const char* xbase, int kb,
                                          const uint32_t* aoff, const uint32_t* boff,
                                          uint32_t dst, Frags& nxt, const char* nslot, int ra,
                                          int rb, const int* xo) {
  constexpr int EVERY = 16 / DMAS;
  if constexpr (LD && M % EVERY == 0) dma_n<M / EVERY>(wbase, xbase, kb, aoff, boff, dst);
  constexpr int R = M < 3 ? 2 * M : (M >= 4 && M < 7 ? 2 * (M - 1) : -1);   // reads 0..11
  if constexpr (R >= 0) {
    read_frag<R>(nxt, nslot, ra, rb, xo);
    read_frag<R + 1>(nxt, nslot, ra, rb, xo);
  }
}

template <int B, bool LD>
__device__ __forceinline__ void k_step(int kt, int ktiles, const char* lds, const char* wbase,
                                       const char* xbase, const uint32_t* aoff,
                                       const uint32_t* boff, uint32_t wave_lds, int ra, int rb,
                                       const int* xo, Frags (&fr)[2], f32x16 (&acc)[4][2]) {
  const Frags& cur = fr[B];
  Frags& nxt = fr[B ^ 1];
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * DMAS) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const char* nslot = lds + ((kt + 1) % NSL) * SLOT;
  const int kb = min(kt + NSL, ktiles - 1) * TK * 2;
  const uint32_t dst = wave_lds + (uint32_t)(kt % NSL) * SLOT;
#define WF_QKV_MMA(M)                                                                 \
  fence();                                                                            \
  mma<M>(cur, acc);                                                                   \
  fence();                                                                            \
  after_mma<LD, M>(wbase, xbase, kb, aoff, boff, dst, nxt, nslot, ra, rb, xo);
  WF_QKV_MMA(0) WF_QKV_MMA(1) WF_QKV_MMA(2) WF_QKV_MMA(3)
  WF_QKV_MMA(4) WF_QKV_MMA(5) WF_QKV_MMA(6) WF_QKV_MMA(7)
  WF_QKV_MMA(8) WF_QKV_MMA(9) WF_QKV_MMA(10) WF_QKV_MMA(11)
  WF_QKV_MMA(12) WF_QKV_MMA(13) WF_QKV_MMA(14) WF_QKV_MMA(15)
#undef WF_QKV_MMA
}

// The k-loop from the barrier that publishes tile 0 to the products of the
// last tile: steps 0 .. ktiles-2 (tile m's fragments in buffer m % 2), then
// the products of the last tile; ktiles = hidden / 32 is even.
template <bool LD>
__device__ __forceinline__ void k_loop(int ktiles, const char* lds, const char* wbase,
                                       const char* xbase, const uint32_t* aoff,
                                       const uint32_t* boff, uint32_t wave_lds, int ra, int rb,
                                       const int* xo, f32x16 (&acc)[4][2]) {
  Frags fr[2];
  // tile 0: visible after the loading threads' loads of it are done and the barrier
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMAS) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (LD) load_tile_at(wbase, xbase, NSL - 1, ktiles, aoff, boff, wave_lds);
  read_frag<0>(fr[0], lds, ra, rb, xo);
  read_frag<1>(fr[0], lds, ra, rb, xo);
  read_frag<2>(fr[0], lds, ra, rb, xo);
  read_frag<3>(fr[0], lds, ra, rb, xo);
  read_frag<4>(fr[0], lds, ra, rb, xo);
  read_frag<5>(fr[0], lds, ra, rb, xo);
  read_frag<6>(fr[0], lds, ra, rb, xo);
  read_frag<7>(fr[0], lds, ra, rb, xo);
  read_frag<8>(fr[0], lds, ra, rb, xo);
  read_frag<9>(fr[0], lds, ra, rb, xo);
  read_frag<10>(fr[0], lds, ra, rb, xo);
  read_frag<11>(fr[0], lds, ra, rb, xo);
  for (int kt = 0; kt < ktiles - 2; kt += 2) {
    k_step<0, LD>(kt, ktiles, lds, wbase, xbase, aoff, boff, wave_lds, ra, rb, xo, fr, acc);
    k_step<1, LD>(kt + 1, ktiles, lds, wbase, xbase, aoff, boff, wave_lds, ra, rb, xo, fr, acc);
  }
  k_step<0, LD>(ktiles - 2, ktiles, lds, wbase, xbase, aoff, boff, wave_lds, ra, rb, xo, fr, acc);
  mma_all(fr[1], acc);
}

// Phase 2 of the epilogue for a Q (SEC 0) or K (SEC 1) head, iteration it:
// the lane's 16-byte chunk c of token 64 wn + 4 it + lane / 16 is read from
// the stage, rotated (MODE 0: no rotation, 1: factors from the block's
// table, 2: factors evaluated per element) and stored to its Q row or K page
// row.
template <int MODE, int SEC>
__device__ __forceinline__ void qk_store(const QkvParams& p, int it, int lane, int wn, int t0,
                                         int pg, int c, const int* ax, const int* rbq,
                                         const char* stage, const int4* post,
                                         const float2* tab, int head, int ps, int& bad) {
  const int tk = 4 * it + (lane >> 4);
  const int tt = 64 * wn + tk;
  const int t = t0 + tt;
  const int page = __shfl(pg, tk);   // every lane active here
  if (t >= p.n_tok) return;
  uint4 v = *reinterpret_cast<const uint4*>(stage + tt * 256 + (((c ^ tt) & 15) << 4));
  if (MODE != 0) {
    const int4 pz = post[tt];
    uint32_t* wv = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pv = ax[q] == 0 ? pz.x : (ax[q] == 1 ? pz.y : pz.z);
      const float2 cs =
          MODE == 1 ? tab[rbq[q] + pv] : rotary_factors(pv, p.pair_omega[4 * c + q]);
      float y0, y1;
      rotate_pair(__uint_as_float(wv[q] << 16), __uint_as_float(wv[q] & 0xffff0000u), cs, y0,
                  y1);
      wv[q] = pack_bf16x2(y0, y1);
    }
  }
  if (SEC == 0) {
    *reinterpret_cast<uint4*>(p.q_out + (int64_t)t * p.q_stride + head * D + c * 8) = v;
  } else {
    const int L = p.dst_start + t;
    if ((unsigned)page >= (unsigned)p.num_pages) {
      bad = 1;
      return;
    }
    *reinterpret_cast<uint4*>(p.k_pages + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * D +
                              c * 8) = v;
  }
}

// The epilogue of a wave whose head is in section SEC (0 Q, 1 K, 2 V), one
// copy per section so that neither phase branches on it.  Phase 1: the
// wave's 64 tokens of its head, + bias and rounded to bf16 (the unfused
// projection's output), into the stage (the ring's LDS).  Phase 2: the wave
// re-reads its own part in the output's order; Q and K are rotated there
// (the accumulators are dead by then), and every global store is 16 bytes.
// bias2[4 i + q4] holds the bias of the lane's features 32 i + 8 q4 + 4 hg
// .. + 3 (bf16 pairs).
template <int SEC>
__device__ __forceinline__ void epilogue(const QkvParams& p, const f32x16 (&acc)[4][2],
                                         const uint2* bias2, int lane, int ql, int hg, int wn,
                                         int t0, int pg, bool use_tab, const int* rbt,
                                         char* stage, const int4* post, const float2* tab,
                                         int head, int ps, int& bad) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // features fl .. fl+3 of the head: registers 4 q4 .. 4 q4 + 3
      const int fl = 32 * i + 8 * q4 + 4 * hg;
      const uint2 b2 = bias2[4 * i + q4];
      const float bv[4] = {__uint_as_float(b2.x << 16), __uint_as_float(b2.x & 0xffff0000u),
                           __uint_as_float(b2.y << 16), __uint_as_float(b2.y & 0xffff0000u)};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t lo = pack_bf16x2(acc[i][j][4 * q4] + bv[0], acc[i][j][4 * q4 + 1] + bv[1]);
        const uint32_t hi =
            pack_bf16x2(acc[i][j][4 * q4 + 2] + bv[2], acc[i][j][4 * q4 + 3] + bv[3]);
        const int tt = 64 * wn + 32 * j + ql;   // token of the block
        if (SEC < 2) {
          // [token][feature] rows of 256 bytes, 16-byte chunks swizzled by token
          *reinterpret_cast<uint2*>(stage + tt * 256 + ((((fl >> 3) ^ tt) & 15) << 4) +
                                    (hg << 3)) = make_uint2(lo, hi);
        } else {
          // [feature][token] rows of 512 bytes
          uint16_t* col = reinterpret_cast<uint16_t*>(stage + fl * (BN * 2) + tt * 2);
          col[0] = (uint16_t)lo;
          col[BN] = (uint16_t)(lo >> 16);
          col[2 * BN] = (uint16_t)hi;
          col[3 * BN] = (uint16_t)(hi >> 16);
        }
      }
    }
  // the wave re-reads only what it wrote: LDS operations of one wave complete
  // in order, and the wait keeps the compiler from moving the reads up
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  if (SEC < 2) {
    // 64 tokens x 16 chunks of 8 features: lane -> (token, chunk); the
    // chunk c = lane % 16 is the same in every iteration, and with it the
    // lane's 4 pairs, their axes and table rows
    const int c = lane & 15;
    int ax[4] = {0, 0, 0, 0}, rbq[4] = {0, 0, 0, 0};
    if (p.rope) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ax[q] = axis_of(p, 4 * c + q);
        if (use_tab) rbq[q] = rbt[4 * c + q];
      }
    }
    // the rotation mode picks one of three copies of the loop: unrolled for
    // no rotation and for table factors, rolled for per-element factors
    if (!p.rope) {
#pragma unroll
      for (int it = 0; it < 16; ++it)
        qk_store<0, SEC>(p, it, lane, wn, t0, pg, c, ax, rbq, stage, post, tab, head, ps, bad);
    } else if (use_tab) {
#pragma unroll
      for (int it = 0; it < 16; ++it)
        qk_store<1, SEC>(p, it, lane, wn, t0, pg, c, ax, rbq, stage, post, tab, head, ps, bad);
    } else {
#pragma unroll 1
      for (int it = 0; it < 16; ++it)
        qk_store<2, SEC>(p, it, lane, wn, t0, pg, c, ax, rbq, stage, post, tab, head, ps, bad);
    }
  } else {
    // 128 features x 8 runs of 8 tokens: lane -> (feature, run)
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane;
      const int fr = idx >> 3, tt = 64 * wn + 8 * (idx & 7);
      const int t = t0 + tt;
      const int L = p.dst_start + t;
      const char* src = stage + fr * (BN * 2) + tt * 2;
      const int page = __shfl(pg, 8 * (idx & 7));   // every lane active here
      if (t + 8 <= p.n_tok && (L & 7) == 0) {
        // 8 consecutive tokens of one page (pages hold a multiple of 8)
        if ((unsigned)page >= (unsigned)p.num_pages) {
          bad = 1;
          continue;
        }
        *reinterpret_cast<uint4*>(p.v_pages + (((int64_t)page * p.heads + head) * D + fr) * ps +
                                  (L & (ps - 1))) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int u = 0; u < 8 && t + u < p.n_tok; ++u) {
          const int Lu = L + u;
          const int pgu = p.page_table[Lu >> p.ps_log2];
          if ((unsigned)pgu >= (unsigned)p.num_pages) {
            bad = 1;
            continue;
          }
          p.v_pages[(((int64_t)pgu * p.heads + head) * D + fr) * ps + (Lu & (ps - 1))] =
              reinterpret_cast<const uint16_t*>(src)[u];
        }
      }
    }
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTH, NTH)))
void qkv_gemm_publish(const QkvParams p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  int* hdr = reinterpret_cast<int*>(lds + HDR_OFF);
  int* rbt = reinterpret_cast<int*>(lds + RB_OFF);
  const int4* post = reinterpret_cast<const int4*>(lds + POS_OFF);
  float2* tab = reinterpret_cast<float2*>(lds + TAB_OFF);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int ql = lane & 31, hg = lane >> 5;

  // ---- block -> (two heads, 256 tokens) --------------------------------------
  const QkvTile tl = qkv_tile(blockIdx.x, gridDim.x, p.feat_tiles, p.tok_tiles);
  const int t0 = tl.ttile * BN;
  const int n_heads = (3 - p.sec0) * p.heads;     // heads computed: [K | V] or [Q | K | V]
  const int gh0 = p.sec0 * p.heads + 2 * tl.ftile;  // global head of wm = 0 (section-major)
  const int gh_last = 3 * p.heads - 1;
  const int wrow0 = gh0 * D;                        // first W row of the block

  // ---- load addressing (loading waves lw = 0 .. LW-1): instruction u of a
  // loading thread fills LDS row r = 16 (LW u + lw) + lane / 4 of its operand,
  // physical chunk lane % 4, which holds the logical chunk
  // (lane % 4) ^ ((r >> 2) & 3) of row r.  Rows past the last head or token
  // re-read the last one (their results are never stored), so no load leaves
  // w or x.
  const char* wbase = uniform_ptr(reinterpret_cast<const char*>(p.w + (int64_t)wrow0 * p.hidden));
  const char* xbase = uniform_ptr(reinterpret_cast<const char*>(p.x + (int64_t)t0 * p.x_stride));
  const bool loader = wave < LW;
  const int lw = wave % LW;
  uint32_t aoff[A_DMA], boff[B_DMA];
#pragma unroll
  for (int u = 0; u < A_DMA; ++u) {
    const int r = 16 * (LW * u + lw) + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    const int wr = min(wrow0 + r, (gh_last + 1) * D - 1) - wrow0;
    aoff[u] = (uint32_t)(wr * p.hidden * 2 + lc * 16);
  }
#pragma unroll
  for (int u = 0; u < B_DMA; ++u) {
    const int r = 16 * (LW * u + lw) + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    const int xr = min(t0 + r, p.n_tok - 1) - t0;
    boff[u] = (uint32_t)(xr * (int)p.x_stride * 2 + lc * 16);
  }
  const uint32_t wave_lds = (uint32_t)(uintptr_t)lds + (uint32_t)lw * 1024u;

  const int ktiles = p.hidden / TK;
  // tiles 0 .. 2
  if (loader) {
    load_tile_at(wbase, xbase, 0, ktiles, aoff, boff, wave_lds);
    load_tile_at(wbase, xbase, 1, ktiles, aoff, boff, wave_lds);
    load_tile_at(wbase, xbase, 2, ktiles, aoff, boff, wave_lds);
  }

  // ---- rotary factor table (while the first tiles load) ---------------------
  // the block needs it if its first head is Q or K (heads are section-major)
  const bool rot_block = p.rope && gh0 < 2 * p.heads;
  bool use_tab = false;
  int mn[3] = {0, 0, 0};
  if (rot_block) {
    if (tid < BN) {
      // rows past the last token repeat it: min and max unchanged
      const int64_t t = min(t0 + tid, p.n_tok - 1);
      const int4 v = make_int4(p.pos[t * 3], p.pos[t * 3 + 1], p.pos[t * 3 + 2], 0);
      reinterpret_cast<int4*>(lds + POS_OFF)[tid] = v;
      const int lo0 = wave_min(v.x), lo1 = wave_min(v.y), lo2 = wave_min(v.z);
      const int hi0 = wave_max(v.x), hi1 = wave_max(v.y), hi2 = wave_max(v.z);
      if (lane == 0) {
        hdr[wave * 6 + 0] = lo0;
        hdr[wave * 6 + 1] = lo1;
        hdr[wave * 6 + 2] = lo2;
        hdr[wave * 6 + 3] = hi0;
        hdr[wave * 6 + 4] = hi1;
        hdr[wave * 6 + 5] = hi2;
      }
    }
    __syncthreads();
    int64_t rng[3], off[4];
    off[0] = 0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      int lo = hdr[a], hi = hdr[3 + a];
#pragma unroll
      for (int w = 1; w < BN / 64; ++w) {
        lo = min(lo, hdr[w * 6 + a]);
        hi = max(hi, hdr[w * 6 + 3 + a]);
      }
      mn[a] = lo;
      rng[a] = (int64_t)hi - lo + 1;
      off[a + 1] = off[a] + (int64_t)(p.band0[a + 1] - p.band0[a]) * rng[a];
    }
    use_tab = off[3] <= TAB_CAP;
    if (use_tab) {
      // entry off[a] + (pr - band0[a]) * rng[a] + (pos - mn[a]) = rb[pr] + pos;
      // the per-axis values are picked with selects (a runtime index into a
      // small array would put it in scratch memory)
      const int o1 = (int)off[1], o2 = (int)off[2], r0 = (int)rng[0], r1 = (int)rng[1],
                r2 = (int)rng[2];
      if (tid < NPAIR) {
        const int a = axis_of(p, tid);
        const int oa = a == 0 ? 0 : (a == 1 ? o1 : o2);
        const int ra_ = a == 0 ? r0 : (a == 1 ? r1 : r2);
        const int ma = a == 0 ? mn[0] : (a == 1 ? mn[1] : mn[2]);
        const int b0 = a == 0 ? p.band0[0] : (a == 1 ? p.band0[1] : p.band0[2]);
        rbt[tid] = oa + (tid - b0) * ra_ - ma;
      }
      for (int e = tid; e < (int)off[3]; e += NTH) {
        const int a = (e >= o1) + (e >= o2);
        const int oa = a == 0 ? 0 : (a == 1 ? o1 : o2);
        const int ra_ = a == 0 ? r0 : (a == 1 ? r1 : r2);
        const int ma = a == 0 ? mn[0] : (a == 1 ? mn[1] : mn[2]);
        const int b0 = a == 0 ? p.band0[0] : (a == 1 ? p.band0[1] : p.band0[2]);
        const int within = e - oa;
        const int pr = b0 + within / ra_;
        tab[e] = rotary_factors(ma + within % ra_, p.pair_omega[pr]);
      }
    }
    // visible to every wave after the k-loop's barriers
  }

  // ---- k-loop ----------------------------------------------------------------
  // Software pipeline over k-tiles: step kt waits for tile kt+1, takes the
  // barrier (every wave has read tile kt, so its slot is free; tile kt+1 is
  // visible), then issues the products of tile kt from registers with the
  // loads of tile kt+4 into tile kt's slot and the fragment reads of tile
  // kt+1 placed between them, so the matrix pipe is fed across the barrier.
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int sw = (ql >> 2) & 3;   // rows 32 i + ql: (row >> 2) & 3 depends on ql only
  const int xo[2] = {(hg ^ sw) << 4, ((2 + hg) ^ sw) << 4};
  const int ra = (128 * wm + ql) * ROWB;
  const int rbo = A_BYTES + (64 * wn + ql) * ROWB;
  if (loader)
    k_loop<true>(ktiles, lds, wbase, xbase, aoff, boff, wave_lds, ra, rbo, xo, acc);
  else
    k_loop<false>(ktiles, lds, wbase, xbase, aoff, boff, wave_lds, ra, rbo, xo, acc);
  // the loads of the re-loaded tiles past the last one land in slots no one
  // reads; they complete before the staging area is written
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue ----------------------------------------------------------------
  __syncthreads();   // every wave is done with the ring: it becomes the stage
  const int hs = 2 * tl.ftile + wm;   // this wave's head among the computed ones
  if (hs >= n_heads) return;
  const int gh = gh0 + wm;
  const int sec = gh / p.heads, head = gh - sec * p.heads;
  char* stage = lds + wm * (RING / 2);
  const int ps = 1 << p.ps_log2;
  // K and V: the page of the wave's token 64 wn + lane, read before phase 1
  // so that its latency hides behind it; phase 2 takes a token's page from
  // its lane (one dependent table read per token instead of per store)
  int pg = 0;
  if (sec >= 1) {
    const int t = t0 + 64 * wn + lane;
    if (t < p.n_tok) pg = p.page_table[(p.dst_start + t) >> p.ps_log2];
  }
  // the bias of the lane's 64 features, as bf16 pairs
  uint2 bias2[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) bias2[k] = make_uint2(0u, 0u);
  if (p.bias) {
    const uint16_t* bp = p.bias + gh * D + 4 * hg;
    if ((reinterpret_cast<uintptr_t>(p.bias) & 7) == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        bias2[k] = *reinterpret_cast<const uint2*>(bp + 32 * (k >> 2) + 8 * (k & 3));
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint16_t* b = bp + 32 * (k >> 2) + 8 * (k & 3);
        bias2[k] = make_uint2((uint32_t)b[0] | ((uint32_t)b[1] << 16),
                              (uint32_t)b[2] | ((uint32_t)b[3] << 16));
      }
    }
  }
  int bad = 0;
  if (sec == 0)
    epilogue<0>(p, acc, bias2, lane, ql, hg, wn, t0, pg, use_tab, rbt, stage, post, tab, head,
                ps, bad);
  else if (sec == 1)
    epilogue<1>(p, acc, bias2, lane, ql, hg, wn, t0, pg, use_tab, rbt, stage, post, tab, head,
                ps, bad);
  else
    epilogue<2>(p, acc, bias2, lane, ql, hg, wn, t0, pg, use_tab, rbt, stage, post, tab, head,
                ps, bad);
  if (bad) atomicOr(p.status, WF_STATUS_BAD_PAGE);
}

}  // namespace

hipError_t launch_qkv_publish(const QkvParams& p, hipStream_t stream) {
  dim3 grid(p.feat_tiles * p.tok_tiles), block(NTH);
  hipLaunchKernelGGL(qkv_gemm_publish, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace wf

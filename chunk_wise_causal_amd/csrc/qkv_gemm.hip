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
// Block: 128 features (one head of one of Q, K, V) x 256 tokens, 8 waves of
// 64 features x 64 tokens (four 32x32 accumulators each; two waves per
// SIMD, so one wave's epilogue or wait overlaps the other's products).
// k-tiles of 64 go straight from global memory into a three-slot LDS ring
// (global_load_lds_dwordx4, two tiles ahead), 16-byte chunks XOR-swizzled by
// row so that the fragment reads of 8 consecutive rows hit distinct banks;
// one barrier per k-tile.  Blocks are dealt to the XCDs in contiguous runs,
// and a run walks 2 token tiles per feature tile, so the blocks resident on
// one XCD share weight and hidden-state tiles in its L2.
//
// Epilogue per element: + bias, round to bf16 (the unfused projection's
// output), then for Q and K the rotation of wf_kv_publish (double-precision
// angle and cos/sin rounded to float, float products and sums without fused
// multiply-add, round to bf16), then Q to q_out, K to its page row, V to its
// d-major page column.
#include "../../include/wf.h"
#include "wf_qkv.h"

namespace wf {
namespace {

constexpr int TM = 128;    // features per block (one head)
constexpr int TN = 256;    // tokens per block
constexpr int TK = 64;     // hidden elements per k-tile
constexpr int NTH = 512;   // threads per block (8 waves)
constexpr int NSL = 3;     // LDS ring slots
constexpr int GT = 2;      // token tiles per feature tile in the block order
constexpr int A_BYTES = TM * TK * 2;           // 16 KB
constexpr int B_BYTES = TN * TK * 2;           // 32 KB
constexpr int SLOT_BYTES = A_BYTES + B_BYTES;  // 48 KB
constexpr int A_DMA = A_BYTES / (NTH * 16);    // 16-byte loads per thread per k-tile: 2
constexpr int B_DMA = B_BYTES / (NTH * 16);    // 4
constexpr int DMAS = A_DMA + B_DMA;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// byte offset of logical 16-byte chunk c (0..7) of row r in an LDS tile of
// 128-byte rows
__device__ __forceinline__ int tile_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// y0 = x0*c - x1*s, y1 = x0*s + x1*c, every operation rounded on its own
__device__ __forceinline__ void rotate(float x0, float x1, float cs, float sn, float& y0,
                                       float& y1) {
#pragma clang fp contract(off)
  const float a = x0 * cs;
  const float b = x1 * sn;
  const float c = x0 * sn;
  const float d = x1 * cs;
  y0 = a - b;
  y1 = c + d;
}

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

// chunks I.. of one operand: chunk i goes 8 KB (one instruction of all 8
// waves, 64 rows) further than chunk i-1
template <uint32_t OFF, int I, int N>
__device__ __forceinline__ void dma_rows(const char* base, const uint32_t* off, uint32_t lds) {
  if constexpr (I < N) {
    dma16<OFF + I * 8192>(base, off[I], lds);
    dma_rows<OFF, I + 1, N>(base, off, lds);
  }
}

// the k-tile at hidden offset k0 into ring slot SLOT: A_DMA chunks of W rows,
// B_DMA of x rows per thread; each wave instruction fills 1 KB (8 rows)
template <int SLOT>
__device__ __forceinline__ void load_tile(const char* wbase, const char* xbase, int k0,
                                          const uint32_t* aoff, const uint32_t* boff,
                                          uint32_t wave_lds) {
  static_assert(NTH * 16 == 8192, "one instruction of every wave fills 8 KB");
  dma_rows<SLOT * SLOT_BYTES, 0, A_DMA>(wbase + 2 * k0, aoff, wave_lds);
  dma_rows<SLOT * SLOT_BYTES + A_BYTES, 0, B_DMA>(xbase + 2 * k0, boff, wave_lds);
}

__device__ __forceinline__ void load_slot(int slot, const char* wbase, const char* xbase, int k0,
                                          const uint32_t* aoff, const uint32_t* boff,
                                          uint32_t wave_lds) {
  if (slot == 0) load_tile<0>(wbase, xbase, k0, aoff, boff, wave_lds);
  else if (slot == 1) load_tile<1>(wbase, xbase, k0, aoff, boff, wave_lds);
  else load_tile<2>(wbase, xbase, k0, aoff, boff, wave_lds);
}

// fragments of k-step ks: A rows 64wm + 32i + ql, B rows 64wn + 32j + ql
__device__ __forceinline__ void frags(const char* slot_base, int ks, int wm, int wn, int ql,
                                      int hg, bf16x8* a, bf16x8* bv) {
  const int c = 2 * ks + hg;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(slot_base + tile_off(64 * wm + 32 * i + ql, c));
#pragma unroll
  for (int j = 0; j < 2; ++j)
    bv[j] = *reinterpret_cast<const bf16x8*>(slot_base + A_BYTES +
                                              tile_off(64 * wn + 32 * j + ql, c));
}

// The 4 accumulators of a wave += one k-tile of its slot.  The fragments of
// k-step ks+1 are read while the 4 products of k-step ks run.
__device__ __forceinline__ void mma_tile(const char* slot_base, int wm, int wn, int ql, int hg,
                                         f32x16 (&acc)[2][2]) {
  bf16x8 a[2][2], bv[2][2];
  frags(slot_base, 0, wm, wn, ql, hg, a[0], bv[0]);
#pragma unroll
  for (int ks = 0; ks < TK / 16; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < TK / 16) frags(slot_base, ks + 1, wm, wn, ql, hg, a[cur ^ 1], bv[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], bv[cur][j], acc[i][j],
                                                            0, 0, 0);
    if (ks + 1 < TK / 16) {
      // reads of the next k-step spread over this k-step's products
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(NTH, NTH)))
void qkv_gemm_publish(const QkvParams p) {
  __shared__ __attribute__((aligned(16))) char lds[NSL * SLOT_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int ql = lane & 31, hg = lane >> 5;

  // ---- block -> (feature tile, token tile) ----------------------------------
  const int nb = gridDim.x, b = blockIdx.x;
  const int per = nb >> 3;
  const int w = (b < (per << 3)) ? ((b & 7) * per + (b >> 3)) : b;
  // groups of GT token tiles; inside a group, feature tile major
  const int group_tiles = GT * p.feat_tiles;
  const int g = w / group_tiles, rem = w - g * group_tiles;
  const int tiles_in_g = min(GT, p.tok_tiles - g * GT);
  const int ftile = rem / tiles_in_g;
  const int ttile = g * GT + (rem - ftile * tiles_in_g);
  const int sec = p.sec0 + ftile / p.heads;            // 0 Q, 1 K, 2 V
  const int head = ftile % p.heads;
  const int f0 = (sec * p.heads + head) * TM;          // first W row
  const int t0 = ttile * TN;

  // ---- load addressing: thread q fills LDS byte 8192 i + 16 q of a tile,
  // i.e. row 64 i + q / 8, physical chunk q % 8 = logical chunk ^ (row & 7)
  const char* wbase = reinterpret_cast<const char*>(p.w + (int64_t)f0 * p.hidden);
  const char* xbase = reinterpret_cast<const char*>(p.x + (int64_t)t0 * p.x_stride);
  uint32_t aoff[A_DMA], boff[B_DMA];
  {
    const int r0 = tid >> 3, pc = tid & 7;
    const int lc = pc ^ (r0 & 7);
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      aoff[i] = (uint32_t)(((64 * i + r0) * p.hidden + lc * 8) * 2);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      // rows past the last token re-read the last token (their results are
      // never stored), so no load leaves x
      const int r = min(64 * i + r0, p.n_tok - 1 - t0);
      boff[i] = (uint32_t)((r * p.x_stride + lc * 8) * 2);
    }
  }
  const uint32_t wave_lds =
      (uint32_t)(uintptr_t)lds + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int ktiles = p.hidden / TK;
  load_slot(0, wbase, xbase, 0, aoff, boff, wave_lds);
  if (ktiles > 1) load_slot(1, wbase, xbase, TK, aoff, boff, wave_lds);
  for (int kt = 0; kt < ktiles; ++kt) {
    // this thread's loads of tile kt are done when at most the next tile's
    // are still in flight; the barrier then publishes every thread's
    if (kt + 1 < ktiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMAS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // slot (kt + 2) % 3 was last read in step kt - 1, which every wave has
    // left (barrier above)
    if (kt + 2 < ktiles) load_slot((kt + 2) % NSL, wbase, xbase, (kt + 2) * TK, aoff, boff, wave_lds);
    mma_tile(lds + (kt % NSL) * SLOT_BYTES, wm, wn, ql, hg, acc);
  }

  // ---- epilogue ------------------------------------------------------------
  const int ps = 1 << p.ps_log2;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 64 * wn + 32 * j + ql;
    if (t >= p.n_tok) continue;
    int page = -1, prow = 0;
    if (sec > 0) {
      const int L = p.dst_start + t;
      page = p.page_table[L >> p.ps_log2];
      if ((unsigned)page >= (unsigned)p.num_pages) {
        bad = 1;
        continue;
      }
      prow = L & (ps - 1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // features fl .. fl+3 of the head: registers 4q4 .. 4q4+3
        const int fl = 64 * wm + 32 * i + 8 * q4 + 4 * hg;
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[i][j][4 * q4 + e];
          if (p.bias) v += bf16_to_f32(p.bias[f0 + fl + e]);
          o[e] = f32_to_bf16_rne(v);
        }
        if (sec < 2 && p.rope) {
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const int pr = (fl + e) >> 1;
            const double phi = (double)p.pos[(int64_t)t * 3 + p.pair_axis[pr]] * p.pair_omega[pr];
            double sn, cn;
            sincos(phi, &sn, &cn);
            float y0, y1;
            rotate(bf16_to_f32(o[e]), bf16_to_f32(o[e + 1]), (float)cn, (float)sn, y0, y1);
            o[e] = f32_to_bf16_rne(y0);
            o[e + 1] = f32_to_bf16_rne(y1);
          }
        }
        const uint2 packed = make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                        (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        if (sec == 0) {
          *reinterpret_cast<uint2*>(p.q_out + (int64_t)t * p.q_stride + head * TM + fl) = packed;
        } else if (sec == 1) {
          *reinterpret_cast<uint2*>(
              p.k_pages + (((int64_t)page * p.heads + head) * ps + prow) * TM + fl) = packed;
        } else {
          uint16_t* vcol = p.v_pages + (((int64_t)page * p.heads + head) * TM + fl) * ps + prow;
#pragma unroll
          for (int e = 0; e < 4; ++e) vcol[(int64_t)e * ps] = o[e];
        }
      }
  }
  if (bad) atomicOr(p.status, WF_STATUS_BAD_PAGE);
}

}  // namespace

hipError_t launch_qkv_publish(const QkvParams& p, hipStream_t stream) {
  dim3 grid(p.feat_tiles * p.tok_tiles), block(NTH);
  hipLaunchKernelGGL(qkv_gemm_publish, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace wf

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
// Block: 128 features (one head of one of Q, K, V) x 128 tokens, 4 waves of
// 64 x 64; k-tiles of 64 staged through registers into a double-buffered,
// XOR-swizzled LDS tile, one barrier per k-tile.  Blocks are dealt to the
// XCDs in contiguous runs, and a run walks 8 token tiles per feature tile,
// so the blocks resident on one XCD share weight and hidden-state tiles in
// its L2.
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

constexpr int TM = 128;    // features per block
constexpr int TN = 128;    // tokens per block
constexpr int TK = 64;     // hidden elements per k-tile
constexpr int NTH = 256;   // threads per block
constexpr int GT = 8;      // token tiles per feature tile in the block order

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// element offset of 16-byte chunk c (0..7) of row r in a [128][64] LDS tile
__device__ __forceinline__ int tile_off(int r, int c) { return r * TK + ((c ^ (r & 7)) << 3); }

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

__global__ __attribute__((amdgpu_flat_work_group_size(NTH, NTH)))
void qkv_gemm_publish(const QkvParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][TM * TK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][TN * TK];
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

  // ---- global -> register assignment: chunk q + 256 i of each tile ---------
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
  bool xok[4];
  int loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + NTH * i;
    const int r = idx >> 3, c = idx & 7;
    wsrc[i] = p.w + (int64_t)(f0 + r) * p.hidden + c * 8;
    const int t = t0 + r;
    xok[i] = t < p.n_tok;
    xsrc[i] = p.x + (int64_t)(xok[i] ? t : 0) * p.x_stride + c * 8;
    loff[i] = tile_off(r, c);
  }
  uint4 ra[4], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(wsrc[i] + k0);
      rb[i] = xok[i] ? *reinterpret_cast<const uint4*>(xsrc[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&sa[buf][loff[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sb[buf][loff[i]]) = rb[i];
    }
  };

  // per-lane fragment rows: A rows 64wm + 32i + ql, B rows 64wn + 32j + ql
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int ktiles = p.hidden / TK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) fetch((kt + 1) * TK);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int c = 2 * ks + hg;
      bf16x8 a[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(&sa[buf][tile_off(64 * wm + 32 * i + ql, c)]);
        bv[i] = *reinterpret_cast<const bf16x8*>(&sb[buf][tile_off(64 * wn + 32 * i + ql, c)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ktiles) stash(buf ^ 1);
    __syncthreads();
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

// wf_kv_publish kernel: 3D RoPE on K (and optionally Q) and the paged scatter
// of K and V into the pool.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §4.2:
// K/V are published after the QKV projection and RoPE, straight into ordered
// paged attention slots, with no concatenation step.
//
// One block owns a 64-token tile of logical rows (aligned to 64 in logical
// space) and a group of heads.  It first evaluates the rotary factors of its
// tokens once (double-precision angle and cos/sin, rounded to float) into
// LDS, then for every head of its group:
//   K: 16-byte vector load -> rotate pairs in float (no fused multiply-add)
//      -> round to the storage type -> 16-byte store into the K page row;
//   V: rows staged in LDS, re-read by feature d, and stored as runs of 8
//      consecutive tokens into the d-major V page (16-byte stores for bf16).
// Memory-bound: every byte of K and V is read once and written once.
#include <type_traits>

#include "../../include/wf.h"
#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kTileTok = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// rotate one pair: y0 = x0*c - x1*s, y1 = x0*s + x1*c, every operation
// rounded on its own
__device__ __forceinline__ void rotate(float x0, float x1, float2 cs, float& y0, float& y1) {
#pragma clang fp contract(off)
  const float a = x0 * cs.x;
  const float b = x1 * cs.y;
  const float c = x0 * cs.y;
  const float d = x1 * cs.x;
  y0 = a - b;
  y1 = c + d;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void publish_kernel(const PublishParams p) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPV = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = D / EPV;               // vectors per head row
  constexpr int VPAD = BF16 ? 8 : 4;         // LDS row padding (elements)
  __shared__ float2 cs[kTileTok][D / 2];
  __shared__ __attribute__((aligned(16))) T vt[kTileTok][D + VPAD];
  __shared__ int page_of[kTileTok];

  const int tid = threadIdx.x;
  const int ps = 1 << p.ps_log2;
  const int L0 = (p.dst_start / kTileTok + (int)blockIdx.x) * kTileTok;
  const int lo = max(L0, p.dst_start);
  const int hi = min(L0 + kTileTok, p.dst_start + p.n_tok);
  const int h0 = (int)blockIdx.y * p.heads_per_block;
  const int h1 = min(p.heads, h0 + p.heads_per_block);

  if (tid < kTileTok) {
    const int L = L0 + tid;
    const int lp = L >> p.ps_log2;
    int page = -1;
    // host validation keeps lp < num_logical_pages for published rows
    if (L >= lo && L < hi) {
      page = p.page_table[lp];
      if (page < 0 || page >= p.num_pages) {
        atomicOr(p.status, WF_STATUS_BAD_PAGE);
        page = -1;
      }
    }
    page_of[tid] = page;
  }
  if (p.rope) {
    for (int idx = tid; idx < kTileTok * (D / 2); idx += kThreads) {
      const int ti = idx / (D / 2), pr = idx % (D / 2);
      const int L = L0 + ti;
      if (L < lo || L >= hi) continue;
      const int t = L - p.dst_start;
      const double phi = (double)p.pos[(int64_t)t * 3 + p.pair_axis[pr]] * p.pair_omega[pr];
      double s, c;
      sincos(phi, &s, &c);
      cs[ti][pr] = make_float2((float)c, (float)s);
    }
  }
  __syncthreads();

  const T* __restrict__ kin = static_cast<const T*>(p.k);
  const T* __restrict__ vin = static_cast<const T*>(p.v);
  T* qio = static_cast<T*>(p.q);
  T* __restrict__ kpg = static_cast<T*>(p.k_pages);
  T* __restrict__ vpg = static_cast<T*>(p.v_pages);

  for (int h = h0; h < h1; ++h) {
    // ---- K (and Q): rotate and store rows --------------------------------
    for (int idx = tid; idx < kTileTok * VPR; idx += kThreads) {
      const int ti = idx / VPR, c = idx % VPR;
      const int L = L0 + ti;
      if (L < lo || L >= hi) continue;
      const int64_t t = L - p.dst_start;
      uint4 kv = *reinterpret_cast<const uint4*>(kin + t * p.k_stride + h * D + c * EPV);
      if (p.rope) {
        T* e = reinterpret_cast<T*>(&kv);
        uint4 qv;
        T* qe = reinterpret_cast<T*>(&qv);
        T* qptr = qio ? qio + t * p.q_stride + h * D + c * EPV : nullptr;
        if (qptr) qv = *reinterpret_cast<const uint4*>(qptr);
#pragma unroll
        for (int j = 0; j < EPV / 2; ++j) {
          const float2 f = cs[ti][c * (EPV / 2) + j];
          float y0, y1;
          if constexpr (BF16) {
            rotate(bf16_to_f32(e[2 * j]), bf16_to_f32(e[2 * j + 1]), f, y0, y1);
            e[2 * j] = f32_to_bf16_rne(y0);
            e[2 * j + 1] = f32_to_bf16_rne(y1);
            if (qptr) {
              rotate(bf16_to_f32(qe[2 * j]), bf16_to_f32(qe[2 * j + 1]), f, y0, y1);
              qe[2 * j] = f32_to_bf16_rne(y0);
              qe[2 * j + 1] = f32_to_bf16_rne(y1);
            }
          } else {
            rotate(e[2 * j], e[2 * j + 1], f, y0, y1);
            e[2 * j] = y0;
            e[2 * j + 1] = y1;
            if (qptr) {
              rotate(qe[2 * j], qe[2 * j + 1], f, y0, y1);
              qe[2 * j] = y0;
              qe[2 * j + 1] = y1;
            }
          }
        }
        if (qptr) *reinterpret_cast<uint4*>(qptr) = qv;
      }
      const int page = page_of[ti];
      if (page >= 0) {
        T* dst = kpg + (((int64_t)page * p.heads + h) * ps + (L & (ps - 1))) * D + c * EPV;
        *reinterpret_cast<uint4*>(dst) = kv;
      }
    }
    // ---- V: stage rows, store d-major runs of 8 tokens ------------------
    for (int idx = tid; idx < kTileTok * VPR; idx += kThreads) {
      const int ti = idx / VPR, c = idx % VPR;
      const int L = L0 + ti;
      if (L < lo || L >= hi) continue;
      const int64_t t = L - p.dst_start;
      *reinterpret_cast<uint4*>(&vt[ti][c * EPV]) =
          *reinterpret_cast<const uint4*>(vin + t * p.v_stride + h * D + c * EPV);
    }
    __syncthreads();
    for (int idx = tid; idx < D * (kTileTok / 8); idx += kThreads) {
      const int d = idx / (kTileTok / 8), r8 = idx % (kTileTok / 8);
      const int ti0 = r8 * 8;
      const int L = L0 + ti0;
      if (L + 8 <= lo || L >= hi) continue;
      // 8-row runs never cross a page (page_size >= 16, runs 8-aligned)
      int page = -1;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (L + e >= lo && L + e < hi) page = page_of[ti0 + e];
      if (page < 0) continue;
      T* dst = vpg + (((int64_t)page * p.heads + h) * D + d) * ps + (L & (ps - 1));
      T run[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = vt[ti0 + e][d];
      if (L >= lo && L + 8 <= hi) {
#pragma unroll
        for (int v = 0; v < 8 / EPV; ++v)
          reinterpret_cast<uint4*>(dst)[v] = reinterpret_cast<const uint4*>(run)[v];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (L + e >= lo && L + e < hi) dst[e] = run[e];
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_publish(const PublishParams& p, int dtype, hipStream_t stream) {
  const int tiles = (p.dst_start + p.n_tok - 1) / kTileTok - p.dst_start / kTileTok + 1;
  dim3 grid(tiles, (p.heads + p.heads_per_block - 1) / p.heads_per_block);
  dim3 block(kThreads);
  const bool bf16 = dtype == WF_BF16;
  if (p.head_dim == 128) {
    if (bf16) hipLaunchKernelGGL((publish_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((publish_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (bf16) hipLaunchKernelGGL((publish_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((publish_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace wf

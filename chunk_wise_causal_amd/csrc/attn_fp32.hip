// wf_chunk_attn, float32: the same slot-masked attention as the bf16 kernel
// ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §3.1)
// for pools stored in float32.  It serves small shapes where bit width, not
// speed, matters: one lane per query row, keys streamed one at a time through
// the page table, online softmax in float32 with fused multiply-adds.
#include "../../include/wf.h"
#include "wf_internal.h"

namespace wf {
namespace {

constexpr int BM = 64;      // one wave, one query row per lane
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(BM) void attn_fwd_fp32(const AttnParams p) {
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int head = w / p.tiles_per_head;
  const int tw = w - head * p.tiles_per_head;
  int grp = 0;
  while (tw >= p.grp_tile_end[grp]) ++grp;
  const int qtile = tw - (grp ? p.grp_tile_end[grp - 1] : 0);
  const int qrow = p.grp_row0[grp] + qtile * BM + lane;
  const bool qvalid = qrow < p.grp_row1[grp];
  const int ps = 1 << p.ps_log2;
  const float* __restrict__ kpg = static_cast<const float*>(p.k_pages);
  const float* __restrict__ vpg = static_cast<const float*>(p.v_pages);

  float q[D], o[D];
  const float* qp = static_cast<const float*>(p.q) + (int64_t)qrow * p.q_stride + head * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qvalid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int ri = p.grp_rng0[grp]; ri < p.grp_rng1[grp]; ++ri) {
    const int lo = p.ranges[ri].x, hi = p.ranges[ri].y;
    for (int L = lo; L < hi; ++L) {
      const int page = p.page_table[L >> p.ps_log2];
      if (page < 0 || page >= p.num_pages) {
        if (lane == 0) atomicOr(p.status, WF_STATUS_BAD_PAGE);
        continue;
      }
      const int64_t base = (int64_t)page * p.heads + head;
      const float* kr = kpg + (base * ps + (L & (ps - 1))) * D;
      const float* vr = vpg + base * D * ps + (L & (ps - 1));
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
      s *= p.scale_log2;
      const float m_new = fmaxf(m, s);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      const float pe = __builtin_amdgcn_exp2f(s - m_new);
      l = l * alpha + pe;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, pe * vr[(int64_t)d * ps]);
      m = m_new;
    }
  }
  if (qvalid) {
    float* op = static_cast<float*>(p.out) + (int64_t)qrow * p.out_stride + head * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
    if (p.lse) p.lse[(int64_t)head * p.lse_stride + qrow] = (m + log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_fp32(const AttnParams& p, int head_dim, int block_m,
                            hipStream_t stream) {
  if (block_m != BM) return hipErrorInvalidValue;
  dim3 grid(p.tiles_per_head * p.heads), block(BM);
  if (head_dim == 128) hipLaunchKernelGGL(attn_fwd_fp32<128>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(attn_fwd_fp32<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace wf

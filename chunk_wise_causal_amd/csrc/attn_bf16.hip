// wf_chunk_attn, bfloat16: slot-masked flash-attention forward over the paged
// K/V pool on CDNA4 matrix cores ("Wave Forcing: Towards Speed-of-Light
// Streaming Video Generation", §3.1).  The walk, masks, softmax, P V and
// pipeline are the shared core (attn_core.h); this file supplies the
// bfloat16 score product:
//
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS (bf16 pages
//                 [H][ps][D], one 64-key tile per slot), B = Q^T held in
//                 registers for the whole kernel, D / 16 k-steps per 32x32
//                 block.
//
// LDS layout of a K slot: 16-byte chunks XOR-swizzled by row so that the
// A-operand reads of 8 (or 16) consecutive lanes hit distinct banks: chunk c
// of row r sits at column c ^ kswz(r).
#include "attn_core.h"

namespace wf {
namespace {

using namespace attn;

// K column swizzle (16-byte chunk units)
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return ((((r & 7) ^ ((r >> 1) & 4)) | (r & 8)) & (D / 8 - 1));
}

struct ScoreBf16 {
  struct Extra {};
  template <int D> static constexpr uint32_t KSLOT = BN * D * 2;   // bytes of one K slot
  template <int D> static constexpr uint32_t XSLOT = 0;            // no extra slots
  template <int D> static constexpr int PER_K = BN * (D / 8) / LT; // 16-byte chunks per thread
  template <int D> static constexpr int KDMAS = PER_K<D>;

  // A lane's query fragments (d = 16i+8hg..+8 of its query), the LDS element
  // offsets of its K A-operand reads, and the block-constant K load
  // addressing of a loading thread.  The K page [H][ps][D] and the V page
  // [H][D][ps] of one head have the same size.
  template <int D>
  struct Ctx {
    static constexpr int DK = D / 16;   // k-steps of S^T = K Q^T
    bf16x8 qf[DK];
    int kaddr[DK];
    const char* k_head;                 // K pages + head offset (bytes)
    int64_t page_bytes;
    uint32_t koff[PER_K<D>];            // per-lane byte offsets of the thread's chunks
  };

  template <int D>
  static __device__ __forceinline__ void setup(const AttnParams& p, const Extra&, int head,
                                               int qrow, bool qvalid, int wave, int ql, int hg,
                                               int lq, uint32_t wave_lds, uint16_t* lds,
                                               Ctx<D>& c) {
    constexpr int DK = Ctx<D>::DK;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (int64_t)qrow * p.q_stride +
                         head * D + 8 * hg;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * i) : make_uint4(0, 0, 0, 0);
      c.qf[i] = __builtin_bit_cast(bf16x8, v);
    }
    const int kr = sigma(ql);
    const int ku = hg ^ kswz<D>(kr);
#pragma unroll
    for (int i = 0; i < DK; ++i) c.kaddr[i] = kr * D + ((2 * i) ^ ku) * 8;
    const int ps = 1 << p.ps_log2;
    c.k_head = static_cast<const char*>(p.k_pages) + (int64_t)head * ps * D * 2;
    c.page_bytes = (int64_t)p.heads * ps * D * 2;
    // chunk i of a loading thread is row r0 + i*LT/CPR, which has the same
    // swizzle (a multiple of 16 rows further)
    constexpr int CPR = D / 8;
    static_assert((LT / CPR) % 16 == 0, "chunk rows keep their swizzle");
    const int r0 = lq / CPR, kcol = (lq % CPR) ^ kswz<D>(r0);
#pragma unroll
    for (int i = 0; i < PER_K<D>; ++i)
      c.koff[i] = (uint32_t)((r0 + i * (LT / CPR)) * D + kcol * 8) * 2u;
  }

  // ---- global -> LDS: the K tile [BN][D] of one head into the slot at byte
  // KOFF.  A full tile goes by direct loads (PER_K per thread, left in
  // flight); any other tile takes the register path and ends with every
  // older vector load complete.
  template <int D, bool BP, uint32_t KOFF, uint32_t XOFF>
  static __device__ __forceinline__ void load_k(const AttnParams& p, const Ctx<D>& c,
                                                uint32_t wave_lds, int head, const Tile& t,
                                                uint16_t* __restrict__ lds, int& bad) {
    constexpr int CPR = D / 8;   // chunks per K row
    constexpr int PER = PER_K<D>;
    const int ps = 1 << p.ps_log2;
    if (tile_full(t)) {
      const char* base = c.k_head + (int64_t)t.page * c.page_bytes +
                         (int64_t)(tile_kt(t) & (ps - 1)) * (D * 2);
      dma_chunks<KOFF, 0, PER>(base, c.koff, wave_lds);
      return;
    }
    if (t.ktc >= 0) {
      // rare (tile cut by a range boundary, spread over several pages, or on
      // a bad page): one chunk at a time, to keep register pressure off the
      // hot loop.  Rows outside the window hold bf16 quiet NaNs: their scores
      // are NaN, which the row max skips (IEEE maxNum), and the mask sets
      // them to -inf before any exponential, so the max of a cut tile is exact.
      const int tid = threadIdx.x;
      const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(p.k_pages);
      uint16_t* kbuf = lds + KOFF / 2;
      const uint4 nan8 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
      const uint4 zero = make_uint4(0, 0, 0, 0);
      int lo, hi;
      tile_window(p, t, lo, hi);
#pragma unroll 1
      for (int i = 0; i < PER; ++i) {
        const int q = i * LT + tid;
        const int r = q / CPR, col = (q % CPR) ^ kswz<D>(r);
        const int L = tile_kt(t) + r;
        uint4 val = nan8;
        if (L >= lo && L < hi) {
          const int page = BP ? t.page : lookup_page(p, L, bad);
          val = zero;
          if (page >= 0)
            val = *reinterpret_cast<const uint4*>(
                kpg + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * D + col * 8);
        }
        *reinterpret_cast<uint4*>(kbuf + q * 8) = val;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // S^T of one tile: s[sb] for keys 32sb.. of the K slot at byte KOFF
  template <int D, uint32_t KOFF, uint32_t XOFF>
  static __device__ __forceinline__ void qk(const uint16_t* __restrict__ lds, const Ctx<D>& c,
                                            f32x16* s) {
    const uint16_t* kbuf = lds + KOFF / 2;
#pragma unroll
    for (int sb = 0; sb < Frag<D>::SB; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int i = 0; i < Ctx<D>::DK; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf + c.kaddr[i] + 32 * sb * D);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, c.qf[i], s[sb], 0, 0, 0);
      }
    }
  }

  // Instruction-scheduling hint for the block that issues the S(j+1) MFMAs
  // and the softmax of tile j: K reads run a few ahead, and every MFMA is
  // followed by a share of the vector work (the tile's 32 exponentials and
  // about 64 other instructions over 16 MFMAs), so the matrix pipe and the
  // VALU run together.  The grouping counts the exponential as a
  // transcendental (mask 0x400), not as a plain vector instruction (0x002):
  // a group that names only the latter leaves the exponentials to bunch
  // behind the first MFMAs.  Three of each per MFMA (the exponentials done by
  // the eleventh MFMA, the rest of the vector work trailing) measured 3 %
  // faster than an even two and four.
  template <int D>
  static __device__ __forceinline__ void interleave_qk_softmax() {
    constexpr int NM = Frag<D>::SB * Ctx<D>::DK;   // MFMAs of S(j+1)
    constexpr int AHEAD = 3;
    constexpr int TPM = 3;                          // exponentials per MFMA
    constexpr int VPM = 3;                          // other VALU per MFMA
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, TPM, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      if (k + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
};

template <int D, bool BP>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[Loop<ScoreBf16, D, BP>::LDS_BYTES / 2];
  attn_body<ScoreBf16, D, BP>(p, ScoreBf16::Extra{}, lds);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int block_m,
                            hipStream_t stream) {
  if (block_m != BM) return hipErrorInvalidValue;
  dim3 grid(p.tiles_per_head * p.heads), block(NT);
  const bool bp = p.ps_log2 >= 6;   // pages of >= BN keys
  if (head_dim == 128) {
    if (bp) hipLaunchKernelGGL((attn_fwd_bf16<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_bf16<128, false>), grid, block, 0, stream, p);
  } else {
    if (bp) hipLaunchKernelGGL((attn_fwd_bf16<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_bf16<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace wf

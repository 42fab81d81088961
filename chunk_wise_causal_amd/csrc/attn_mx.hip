// wf_chunk_attn_mx: the chunk-wise causal attention forward with an 8-bit
// QK^T (MXFP8 queries and keys), P V in bfloat16, on CDNA4 matrix cores.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", §3.1
// (the slot mask and context order, as in the bfloat16 kernel) and §5.5
// (the pages also run attention with 8-bit QK^T, Sage + W8A8).
//
// The format is OCP microscaling FP8: E4M3 elements with one power-of-two
// (E8M0) scale per 32 consecutive features of a token's head vector.  Keys
// arrive quantized in their own pool (codes [pages][H][ps][D], scales
// [pages][H][ps][D/32]); each query row is quantized by the same rule when
// the block starts.  S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4,
// which applies both operands' block scales itself: per 32x32 block of S^T
// two products of 64 features each, with no per-score vector work.
//
// Operand layout of that product (established on the hardware): lane
// (row m, half h) holds in bytes 0-15 the features 16h..16h+15 of its
// 64-feature step and in bytes 16-31 the features 32+16h..32+16h+15; block
// b of the step (features 32b..32b+31) is bytes 16b..16b+15 of both halves,
// and its scale comes from lane m + 32b (the byte the operand selector
// picks).  Rows (keys) and columns (queries) share that layout.
//
// Everything after the scores (walk, masks, online softmax, P V, pipeline,
// LDS rings, XCD remap) is the shared core (attn_core.h), with the K slot
// half as large as in bfloat16 and a 256-byte scale slot per ring entry.
// Loads of a full tile: two 16-byte direct loads per loading thread for the
// K codes, one for the scales (four lanes of each loading wave), four for V^T.
#include "attn_core.h"
#include "wf_mx.h"
#include "wf_numerics.h"

namespace wf {
namespace {

using namespace attn;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// K code rows are 128 bytes (8 chunks); the 8 lanes read together cover
// rows {0-3, 8-11} or {4-7, 12-15} of a 16-row group (the sigma order)
__device__ __forceinline__ int kswz8(int r) { return (r & 3) | ((r >> 1) & 4); }

struct ScoreMx {
  typedef const uint8_t* Extra;   // the key scales [pages][H][ps][D/32]
  template <int D> static constexpr uint32_t KSLOT = BN * D;           // code bytes of one K slot
  template <int D> static constexpr uint32_t XSLOT = BN * (D / 32);    // scale bytes
  template <int D> static constexpr int PER_K = BN * (D / 16) / LT;    // code chunks per thread
  // per loading thread: the code chunks and one scale chunk (four lanes)
  template <int D> static constexpr int KDMAS = PER_K<D> + 1;

  // A lane's quantized query (one 32-byte fragment per 64-feature k-step)
  // and its scale bytes, the byte offsets of its key code chunks (k-step i:
  // kaddr[2i], kaddr[2i+1]), its key row kr (sigma order) and scale shift
  // 8h; and the block-constant K code / scale load addressing.
  template <int D>
  struct Ctx {
    static constexpr int DK = D / 64;   // k-steps (64 features) of S^T = K Q^T
    i32x8 qf[DK];
    int qsc;
    int kaddr[2 * DK];
    int kr, hsh;
    const uint8_t* k8s;
    const char* k_head;                 // key codes + head offset (bytes)
    const char* s_head;                 // key scales + head offset
    int64_t k_page_bytes, s_page_bytes;
    uint32_t koff[PER_K<D>];            // per-lane byte offsets of the thread's chunks
    uint32_t soff;                      // scale chunk of lanes 0..3 (16 bytes = 4 key rows)
    uint32_t sc_lds;                    // LDS byte address of this wave's 64 scale bytes
  };

  // The query row, quantized to MXFP8 here.  Lane (ql, hg) reads the
  // 16-feature units 2b+hg (b = 0..3) of its row; a 32-feature block is one
  // unit in each half, so the block maximum takes one cross-half exchange.
  // k-step i uses blocks 2i (bytes 0-15) and 2i+1 (bytes 16-31).
  template <int D>
  static __device__ __forceinline__ void setup(const AttnParams& p, const Extra& k8_scales,
                                               int head, int qrow, bool qvalid, int wave,
                                               int ql, int hg, int lq, uint32_t wave_lds,
                                               uint16_t* lds, Ctx<D>& c) {
    static_assert(D == 128, "8-bit scores: head_dim 128");
    constexpr int DK = Ctx<D>::DK;
    {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (int64_t)qrow * p.q_stride +
                           head * D + 16 * hg;
      uint32_t sc[4];
      uint32_t codes[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
        if (qvalid) {
          u0 = *reinterpret_cast<const uint4*>(qp + 32 * b);
          u1 = *reinterpret_cast<const uint4*>(qp + 32 * b + 8);
        }
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float x[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[2 * j] = __uint_as_float(w[j] << 16);
          x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(x[j]));
        amax = xhalf_max(amax);
        sc[b] = mx_scale_code(amax);
        const float mult = __uint_as_float((254u - sc[b]) << 23);   // 2^(127 - scale), exact
#pragma unroll
        for (int j = 0; j < 4; ++j)
          codes[b][j] = e4m3_code(x[4 * j] * mult) | (e4m3_code(x[4 * j + 1] * mult) << 8) |
                        (e4m3_code(x[4 * j + 2] * mult) << 16) |
                        (e4m3_code(x[4 * j + 3] * mult) << 24);
      }
#pragma unroll
      for (int i = 0; i < DK; ++i)
        c.qf[i] = i32x8{(int)codes[2 * i][0], (int)codes[2 * i][1], (int)codes[2 * i][2],
                        (int)codes[2 * i][3], (int)codes[2 * i + 1][0], (int)codes[2 * i + 1][1],
                        (int)codes[2 * i + 1][2], (int)codes[2 * i + 1][3]};
      // lane half hg supplies the scale of block 2i + hg for k-step i
      c.qsc = (int)(sc[hg] | (sc[2 + hg] << 8));
    }
    c.kr = sigma(ql);
    c.hsh = 8 * hg;
    const int ku = kswz8(c.kr);
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      c.kaddr[2 * i] = c.kr * D + ((4 * i + hg) ^ ku) * 16;
      c.kaddr[2 * i + 1] = c.kr * D + ((4 * i + 2 + hg) ^ ku) * 16;
    }
    const int ps = 1 << p.ps_log2;
    c.k8s = k8_scales;
    c.k_head = static_cast<const char*>(p.k_pages) + (int64_t)head * ps * D;
    c.s_head = reinterpret_cast<const char*>(k8_scales) + (int64_t)head * ps * (D / 32);
    c.k_page_bytes = (int64_t)p.heads * ps * D;
    c.s_page_bytes = (int64_t)p.heads * ps * (D / 32);
    // chunk i of a loading thread is row r0 + i*LT/CPR, which has the same
    // swizzle (a multiple of 16 rows further)
    constexpr int CPR = D / 16;
    static_assert((LT / CPR) % 16 == 0, "chunk rows keep their swizzle");
    const int r0 = lq / CPR, kcol = (lq % CPR) ^ kswz8(r0);
#pragma unroll
    for (int i = 0; i < PER_K<D>; ++i)
      c.koff[i] = (uint32_t)((r0 + i * (LT / CPR)) * D + kcol * 16);
    // scales: loading wave w brings key rows 16w..16w+15 (64 bytes) with
    // lanes 0..3, 16 bytes (4 rows) each
    const int lw = wave % (LT / 64);
    c.soff = (uint32_t)(lw * 64 + (lq & 3) * 16);
    const uint32_t wv = (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    c.sc_lds = (uint32_t)(uintptr_t)lds + (wv % (LT / 64)) * 64u;
  }

  // ---- global -> LDS: the K code tile [BN][D] into the slot at byte KOFF
  // and its scales [BN][D/32] into the slot at byte XOFF.  A full tile goes
  // by direct loads (PER_K per thread, plus one 16-byte scale chunk from
  // lanes 0..3 of each loading wave, left in flight); any other tile takes
  // the register path and ends with every older vector load complete.
  template <int D, bool BP, uint32_t KOFF, uint32_t XOFF>
  static __device__ __forceinline__ void load_k(const AttnParams& p, const Ctx<D>& c,
                                                uint32_t wave_lds, int head, const Tile& t,
                                                uint16_t* __restrict__ lds, int& bad) {
    constexpr int CPR = D / 16;   // chunks per code row
    constexpr int PER = PER_K<D>;
    const int ps = 1 << p.ps_log2;
    if (tile_full(t)) {
      const int64_t row = tile_kt(t) & (ps - 1);
      const char* base = c.k_head + (int64_t)t.page * c.k_page_bytes + row * D;
      dma_chunks<KOFF, 0, PER>(base, c.koff, wave_lds);
      const char* sbase = c.s_head + (int64_t)t.page * c.s_page_bytes + row * (D / 32);
      if ((threadIdx.x & 63) < 4) dma16<XOFF>(sbase, c.soff, c.sc_lds);
      return;
    }
    if (t.ktc >= 0) {
      // rare (tile cut by a range boundary, spread over several pages, or on
      // a bad page): one chunk at a time.  Rows outside the window hold E4M3
      // NaN codes: their scores are NaN, which the row max skips, and the
      // mask sets them to -inf before any exponential.  A bad page reads as
      // zeros.
      const int tid = threadIdx.x;
      const uint8_t* __restrict__ kpg = static_cast<const uint8_t*>(p.k_pages);
      uint8_t* kbuf = reinterpret_cast<uint8_t*>(lds) + KOFF;
      const uint4 nan16 = make_uint4(0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu);
      const uint4 zero = make_uint4(0, 0, 0, 0);
      int lo, hi;
      tile_window(p, t, lo, hi);
#pragma unroll 1
      for (int i = 0; i < PER; ++i) {
        const int q = i * LT + tid;
        const int r = q / CPR, col = (q % CPR) ^ kswz8(r);
        const int L = tile_kt(t) + r;
        uint4 val = nan16;
        if (L >= lo && L < hi) {
          const int page = BP ? t.page : lookup_page(p, L, bad);
          val = zero;
          if (page >= 0)
            val = *reinterpret_cast<const uint4*>(
                kpg + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * D + col * 16);
        }
        *reinterpret_cast<uint4*>(kbuf + q * 16) = val;
      }
      // scales: one 4-byte word per key row (unit scales outside the window)
      if (tid < BN) {
        const int L = tile_kt(t) + tid;
        uint32_t w = 0x7f7f7f7fu;
        if (L >= lo && L < hi) {
          const int page = BP ? t.page : lookup_page(p, L, bad);
          if (page >= 0)
            w = *reinterpret_cast<const uint32_t*>(
                c.k8s + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * (D / 32));
        }
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(lds) + XOFF + tid * 4) = w;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // one k-step's key codes of a lane: two 16-byte chunks
  static __device__ __forceinline__ i32x8 kfrag(const uint8_t* kb, int off0, int off1) {
    const uint4 lo = *reinterpret_cast<const uint4*>(kb + off0);
    const uint4 hi = *reinterpret_cast<const uint4*>(kb + off1);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  // S^T of one tile: s[sb] for keys 32sb.. of the K code slot at byte KOFF.
  // Per k-step i the lane's two 16-byte code chunks (kaddr, byte offsets)
  // and the scale bytes: the key row's scale word (scale slot at byte XOFF)
  // shifted by 8h puts block h in byte 0 and block 2+h in byte 2 (selected
  // by k-step); the query scale word holds the lane's blocks of steps 0 and
  // 1 in bytes 0 and 1.
  template <int D, uint32_t KOFF, uint32_t XOFF>
  static __device__ __forceinline__ void qk(const uint16_t* __restrict__ lds, const Ctx<D>& c,
                                            f32x16* s) {
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(lds) + KOFF;
    const uint32_t* sslot =
        reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lds) + XOFF);
#pragma unroll
    for (int sb = 0; sb < Frag<D>::SB; ++sb) {
      const int ksc = (int)(sslot[32 * sb + c.kr] >> c.hsh);
      // (the byte selectors are immediates: the two k-steps are written out)
      const i32x8 a0 = kfrag(kb + 32 * sb * D, c.kaddr[0], c.kaddr[1]);
      s[sb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, c.qf[0], f32x16{}, 0, 0, 0, ksc,
                                                              0, c.qsc);
      const i32x8 a1 = kfrag(kb + 32 * sb * D, c.kaddr[2], c.kaddr[3]);
      s[sb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, c.qf[1], s[sb], 0, 0, 2, ksc,
                                                              1, c.qsc);
    }
  }

  // Instruction-scheduling hint for the block that issues the S(j+1) MFMAs
  // and the softmax of tile j: K reads run a few ahead, and every MFMA is
  // followed by a share of the VALU work, so the matrix pipe and the VALU
  // run together.  (The block-scaled product is not in the hints' matrix
  // class, so the groups name only the vector work and the reads between
  // the products; the scheduler places the products among them.)
  template <int D>
  static __device__ __forceinline__ void interleave_qk_softmax() {
    constexpr int NM = Frag<D>::SB * Ctx<D>::DK;              // MFMAs of S(j+1), 64 cycles each
    constexpr int NDS = Frag<D>::SB * (2 * Ctx<D>::DK + 1);  // code chunks + scale words
    constexpr int AHEAD = 3;
    constexpr int VPM = 24;                                   // VALU per MFMA
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      if (AHEAD + 2 * k < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (AHEAD + 2 * k + 1 < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
};

template <int D, bool BP>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mx(const AttnParams p, const uint8_t* k8_scales) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[Loop<ScoreMx, D, BP>::LDS_BYTES / 2];
  attn_body<ScoreMx, D, BP>(p, k8_scales, lds);
}

}  // namespace

hipError_t launch_attn_mx(const AttnParams& p, const void* k8_scales, hipStream_t stream) {
  dim3 grid(p.tiles_per_head * p.heads), block(NT);
  const uint8_t* sc = static_cast<const uint8_t*>(k8_scales);
  if (p.ps_log2 >= 6) hipLaunchKernelGGL((attn_fwd_mx<128, true>), grid, block, 0, stream, p, sc);
  else hipLaunchKernelGGL((attn_fwd_mx<128, false>), grid, block, 0, stream, p, sc);
  return hipGetLastError();
}

}  // namespace wf

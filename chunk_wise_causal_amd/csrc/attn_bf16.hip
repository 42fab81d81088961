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
// Work unit: one block = (head, slot, 128-row query tile), 4 waves of 64
// lanes, each wave owning 32 query rows.  Per 64-key tile:
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
//                 stale max, and 2^8 keeps every term finite).
//   O^T += V^T P^T  A = V^T read from the d-major V pages via LDS, B = P^T
//                 straight from the S^T accumulators: the K rows of S^T are
//                 loaded in the order sigma(i) (bits 2 and 3 of the row index
//                 swapped) so that each lane's 8 probabilities of a k-step
//                 are 8 consecutive keys, matching a 16-byte V^T read.
// Tiles are double-buffered in LDS with register staging: the loads of the
// next tile are in flight while the current one is multiplied.
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

constexpr int BM = 128;     // query rows per block
constexpr int BN = 64;      // keys per tile
constexpr int NT = 256;     // threads per block
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

template <int D>
struct Stage {
  static constexpr int KCH = BN * D / 8 / NT;   // 16-byte K chunks per thread
  static constexpr int VCH = D * BN / 8 / NT;   // 16-byte V chunks per thread
  uint4 k[KCH];
  uint4 v[VCH];
};

__device__ __forceinline__ int lookup_page(const AttnParams& p, int L) {
  const int page = p.page_table[L >> p.ps_log2];
  if (page < 0 || page >= p.num_pages) {
    atomicOr(p.status, WF_STATUS_BAD_PAGE);
    return -1;
  }
  return page;
}

// global -> registers: keys [kt, kt+BN) of one head, only rows in [lo, hi)
template <int D>
__device__ __forceinline__ void load_tile(const AttnParams& p, int head, int kt, int lo, int hi,
                                          Stage<D>& st) {
  const int tid = threadIdx.x;
  const int ps = 1 << p.ps_log2;
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(p.k_pages);
  const uint16_t* __restrict__ vpg = static_cast<const uint16_t*>(p.v_pages);
  const bool one_page = p.ps_log2 >= 6;           // tile inside one page
  const int tile_page = one_page ? lookup_page(p, max(kt, lo)) : -1;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  if (one_page && tile_page >= 0 && lo == kt && hi == kt + BN) {
    // the common case: a whole tile of one page, no masking, no branches
    const int64_t base = (int64_t)tile_page * p.heads + head;
    const uint16_t* kb = kpg + (base * ps + (kt & (ps - 1))) * D;
    const uint16_t* vb = vpg + base * D * ps + (kt & (ps - 1));
#pragma unroll
    for (int i = 0; i < Stage<D>::KCH; ++i) {
      const int c = tid + NT * i;
      st.k[i] = *reinterpret_cast<const uint4*>(kb + (c / (D / 8)) * D + (c % (D / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < Stage<D>::VCH; ++i) {
      const int c = tid + NT * i;
      st.v[i] = *reinterpret_cast<const uint4*>(vb + (int64_t)(c / (BN / 8)) * ps +
                                                (c % (BN / 8)) * 8);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int row = c / (D / 8), col = c % (D / 8);
    const int L = kt + row;
    uint4 val = zero;
    if (L >= lo && L < hi) {
      const int page = one_page ? tile_page : lookup_page(p, L);
      if (page >= 0)
        val = *reinterpret_cast<const uint4*>(
            kpg + (((int64_t)page * p.heads + head) * ps + (L & (ps - 1))) * D + col * 8);
    }
    st.k[i] = val;
  }
#pragma unroll
  for (int i = 0; i < Stage<D>::VCH; ++i) {
    const int c = tid + NT * i;
    const int d = c / (BN / 8), kc = c % (BN / 8);
    const int L = kt + kc * 8;
    uint4 val = zero;
    if (L + 8 > lo && L < hi) {
      const int page = one_page ? tile_page : lookup_page(p, max(L, lo));
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
    st.v[i] = val;
  }
}

template <int D>
__device__ __forceinline__ void store_tile(uint16_t* kl, uint16_t* vl, const Stage<D>& st) {
  constexpr int KS = D + 8, VS = BN + 8;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int row = c / (D / 8), col = c % (D / 8);
    *reinterpret_cast<uint4*>(kl + row * KS + col * 8) = st.k[i];
  }
#pragma unroll
  for (int i = 0; i < Stage<D>::VCH; ++i) {
    const int c = tid + NT * i;
    const int d = c / (BN / 8), kc = c % (BN / 8);
    *reinterpret_cast<uint4*>(vl + d * VS + kc * 8) = st.v[i];
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const AttnParams p) {
  constexpr int KS = D + 8;           // K row stride in LDS (elements)
  constexpr int VS = BN + 8;          // V^T row stride in LDS (elements)
  constexpr int KT = BN * KS;         // elements of one K tile buffer
  constexpr int VT = D * VS;          // elements of one V^T tile buffer
  constexpr int DK = D / 16;          // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;          // 32-wide d blocks of O^T
  constexpr int SB = BN / 32;         // 32-key blocks of S^T
  constexpr int PK = BN / 16;         // k-steps of O^T += V^T P^T
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (KT + VT)];

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

  // ---- Q^T operand in registers: lane (query ql, half hg) holds d = 16i+8hg..+8
  bf16x8 qf[DK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (int64_t)qrow * p.q_stride +
                         head * D + 8 * hg;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * i) : make_uint4(0, 0, 0, 0);
      qf[i] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*<q,k>
  float l_part[PK];          // this half-lane's partial denominators
#pragma unroll
  for (int t = 0; t < PK; ++t) l_part[t] = 0.f;
  const float sl2 = p.scale_log2;

  // ---- tile cursor over the merged visible ranges -------------------------
  int ri = rng0;
  int r_lo = p.ranges[ri].x, r_hi = p.ranges[ri].y;
  int kt = r_lo & ~(BN - 1);
  Stage<D> st;
  load_tile<D>(p, head, kt, max(kt, r_lo), min(kt + BN, r_hi), st);
  store_tile<D>(lds, lds + KT, st);
  __syncthreads();
  int buf = 0;

  while (true) {
    // next tile
    int nri = ri, n_lo = r_lo, n_hi = r_hi, nkt = kt + BN;
    if (nkt >= r_hi) {
      nri = ri + 1;
      if (nri < rng1) {
        n_lo = p.ranges[nri].x;
        n_hi = p.ranges[nri].y;
        nkt = n_lo & ~(BN - 1);
      }
    }
    const bool more = nri < rng1;
    if (more) load_tile<D>(p, head, nkt, max(nkt, n_lo), min(nkt + BN, n_hi), st);

    // ---- compute on buffer `buf` ------------------------------------------
    const uint16_t* kl = lds + buf * (KT + VT);
    const uint16_t* vl = kl + KT;
    const int w_lo = max(kt, r_lo), w_hi = min(kt + BN, r_hi);

    f32x16 s[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      s[sb] = f32x16{};
      const uint16_t* kr = kl + (32 * sb + sigma(ql)) * KS + 8 * hg;
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * i);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i], s[sb], 0, 0, 0);
      }
    }
    // register r of block sb holds key kt + 32sb + 16(r/8) + 8hg + r%8
    if (w_lo > kt || w_hi < kt + BN) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * sb + 16 * (r >> 3) + 8 * hg + (r & 7);
          if (key < w_lo || key >= w_hi) s[sb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    const float mt = xhalf_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int t = 0; t < PK; ++t) l_part[t] *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    // probabilities, rounded to bf16 for the PV product; the denominator sums
    // the same rounded values exactly in float, so the weights applied to V
    // are normalized exactly even when one key dominates a row
    bf16x8 pb[PK];
#pragma unroll
    for (int t = 0; t < PK; ++t) {
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x2 x = {__builtin_amdgcn_exp2f(s[t >> 1][8 * (t & 1) + 2 * j] * sl2 - m_run),
                         __builtin_amdgcn_exp2f(s[t >> 1][8 * (t & 1) + 2 * j + 1] * sl2 - m_run)};
        const bf16x2 b = __builtin_convertvector(x, bf16x2);
        pk[j] = __builtin_bit_cast(uint32_t, b);
        l_part[t] += __uint_as_float(pk[j] << 16) + __uint_as_float(pk[j] & 0xffff0000u);
      }
      pb[t] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
#pragma unroll
    for (int t = 0; t < PK; ++t) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(vl + (32 * db + ql) * VS + 16 * t + 8 * hg);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
      }
    }

    if (!more) break;
    store_tile<D>(lds + (buf ^ 1) * (KT + VT), lds + (buf ^ 1) * (KT + VT) + KT, st);
    __syncthreads();
    buf ^= 1;
    ri = nri;
    r_lo = n_lo;
    r_hi = n_hi;
    kt = nkt;
  }

  // ---- epilogue: O = O^T / l, LSE ------------------------------------------
  float l_run = 0.f;
#pragma unroll
  for (int t = 0; t < PK; ++t) l_run += l_part[t];
  const float l = xhalf_sum(l_run);
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
  if (head_dim == 128) hipLaunchKernelGGL(attn_fwd_bf16<128>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(attn_fwd_bf16<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace wf

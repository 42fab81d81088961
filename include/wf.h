/*
 * wf.h — C ABI of libwf: the per-layer attention hot path of chunk-wise
 * causal streaming video diffusion on AMD Instinct MI355X (gfx950).
 *
 * Source of the method (cited below as [WF]):
 *   "Wave Forcing: Towards Speed-of-Light Streaming Video Generation"
 *     §3.1  chunk-wise causal attention: full attention inside a chunk; a query
 *           in denoising slot s sees the K/V of slot j iff j >= s; per-layer
 *           context order anchor, bounded clean history, live store, then the
 *           denoising slots in increasing j with self first.
 *     §4.2  K/V are published after the QKV projection and RoPE, written
 *           directly into ordered, paged attention slots (no concatenation),
 *           and must be ready before attention reads them.
 *
 * Two calls form the path, in this order on one stream:
 *   wf_kv_publish()  3D RoPE on K (optionally Q) + scatter of K and V into a
 *                    paged pool through a page table            ([WF] §4.2)
 *   wf_chunk_attn()  slot-masked softmax attention forward of the query chunks
 *                    over that pool                             ([WF] §3.1)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensors are caller-owned.  Pointers marked "device" are HIP device
 *    pointers (e.g. torch tensor data_ptr()); pointers marked "host" are read
 *    synchronously during the call and may be freed when it returns.
 *  - The library never allocates device memory and never synchronizes: every
 *    call validates its arguments on the host, enqueues its kernels on
 *    `stream` (0 = the null stream) and returns.  Readiness of published K/V
 *    ([WF] §4.2) is stream order: publish, then attention on the same stream,
 *    is safe; across streams the caller must order them with an event.
 *  - Element types: WF_BF16 (bfloat16) or WF_FP32.  Q, K, V, the pool and the
 *    output of one call share one type.
 *  - Row strides are in ELEMENTS between consecutive tokens.  Inside a token
 *    row the layout is [num_heads][head_dim], contiguous.  Row strides must be
 *    multiples of 8 elements (16 bytes for bf16) and >= num_heads*head_dim, and
 *    base pointers 16-byte aligned, so that kernels move 16-byte vectors.
 *  - Return value: WF_OK, or a negative WF_ERR_* code.  Nothing is thrown and
 *    nothing aborts.  Argument checks run entirely on the host before any HIP
 *    call, so a rejected call has no side effect.  wf_last_error() returns a
 *    message naming the failed check (thread-local, valid until the next call
 *    from the same thread).
 *  - Device-side data the host cannot check (page-table entries, positions)
 *    never causes an out-of-bounds access: a page-table entry outside
 *    [0, num_pages) makes publish skip the row and makes attention read zeros
 *    for that page.  Either case raises a bit in the per-device status word
 *    read by wf_device_status(); results of such a call are undefined.
 */
#ifndef WF_H
#define WF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----- status codes ------------------------------------------------------ */
enum {
  WF_OK = 0,
  WF_ERR_INVALID = -1,     /* an argument violates the documented contract  */
  WF_ERR_UNSUPPORTED = -2, /* valid, but outside what is built (head_dim,
                              table sizes)                                   */
  WF_ERR_HIP = -3          /* a HIP runtime call failed (launch, device)    */
};

/* device status bits (wf_device_status) */
enum {
  WF_STATUS_BAD_PAGE = 1   /* a page-table entry was outside [0, num_pages)  */
};

typedef enum { WF_BF16 = 0, WF_FP32 = 1 } wf_dtype;

/* ----- the paged K/V pool ([WF] §4.2: paged, ordered attention slots) -----
 *
 * The pool holds the per-layer context of [WF] §3.1 in LOGICAL token order
 * (anchor | clean history | live store | slot 0 | ... | slot W-1 in the usual
 * layout).  Logical token L lives in logical page L / page_size at row
 * L % page_size; page_table maps logical page -> physical page.
 *
 *   k_pages   device, [num_pages][num_heads][page_size][head_dim]   (row-major
 *             rows: one token's head vector is contiguous)
 *   v_pages   device, [num_pages][num_heads][head_dim][page_size]   (d-major:
 *             inside a page, one head's V block is stored transposed, so a
 *             run of tokens is contiguous for every feature d)
 *   page_table device int32 [num_logical_pages], entries in [0, num_pages).
 *             Physical pages not named by the table are never read.
 *
 * Constraints: head_dim in {64, 128}; page_size a power of two in [16, 1024];
 * num_heads >= 1; num_pages, num_logical_pages >= 1; both page arrays 16-byte
 * aligned.  The caller owns all memory; the struct itself is read during the
 * call only.
 */
typedef struct {
  void*          k_pages;
  void*          v_pages;
  const int32_t* page_table;
  int32_t        num_pages;
  int32_t        num_logical_pages;
  int32_t        page_size;
  int32_t        num_heads;
  int32_t        head_dim;
  int32_t        dtype;        /* wf_dtype */
} wf_kv_pool;

/* ----- 3D rotary position embedding --------------------------------------
 * The head dimension is split into three contiguous sub-bands of widths
 * d_t, d_h, d_w (time, latent row, latent column; each even, summing to
 * head_dim).  Within the sub-band of axis a, element pairs (2i, 2i+1) are
 * rotated by the angle pos_a * theta^(-2i/d_a): a one-dimensional rotary
 * embedding per axis.  Precision (so that every implementation agrees bit
 * for bit): the frequency and angle are evaluated in double precision,
 * cos and sin are evaluated in double precision and rounded to float; the
 * rotation y0 = x0*c - x1*s, y1 = x0*s + x1*c is evaluated in float with each
 * product and the sum rounded separately (no fused multiply-add); the result
 * is rounded to the storage type with round-to-nearest-even.
 */
typedef struct {
  int32_t d_t, d_h, d_w;
  double  theta;               /* > 0, e.g. 10000 */
} wf_rope;

/* ----- context segments ([WF] §3.1) --------------------------------------
 * A segment is a run of logical tokens [kv_start, kv_start + kv_len) and the
 * slot it belongs to.  slot < 0 marks context every query sees (anchor, clean
 * history, live store); slot j >= 0 marks the K/V of denoising slot j.  A
 * query of slot s sees every segment with slot < 0 or slot >= s.  Segments
 * must not overlap; their order and any gaps between them are free.
 */
typedef struct {
  int32_t kv_start;
  int32_t kv_len;
  int32_t slot;
} wf_segment;

/* ------------------------------------------------------------------------
 * wf_kv_publish — RoPE + paged scatter ([WF] §4.2: K/V are published after
 * the QKV projection and RoPE, straight into paged attention slots).
 *
 * For t in [0, n_tok) and every head h, with L = dst_logical_start + t,
 * page = page_table[L / page_size], r = L % page_size:
 *   k_pages[page][h][r][:]   = RoPE(k[t][h][:], pos_thw[t])   (rope != NULL)
 *                            = k[t][h][:]                    (rope == NULL)
 *   v_pages[page][h][:][r]   = v[t][h][:]                    (bit copy)
 *   q_inout[t][h][:]        <- RoPE(q_inout[t][h][:], pos_thw[t])  (if given)
 * No other pool byte is written.
 *
 *   pool             host struct describing the pool (see above)
 *   rope             host, nullable: NULL publishes K unrotated
 *   k, v             device, [n_tok] rows of [num_heads][head_dim]
 *   k_row_stride,
 *   v_row_stride     elements between token rows (fused-QKV outputs can be
 *                    read in place)
 *   pos_thw          device int32 [n_tok][3] = (t, h, w) positions; may be
 *                    NULL only if rope == NULL
 *   n_tok            >= 0 (0 is a no-op)
 *   dst_logical_start  >= 0, dst_logical_start + n_tok <=
 *                    num_logical_pages * page_size
 *   q_inout          device, nullable, rotated in place with the same
 *                    positions; requires rope != NULL
 *   q_row_stride     elements between Q rows (ignored if q_inout == NULL)
 * Aliasing: k, v and q_inout must not overlap the pool or each other.
 * Returns WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED or WF_ERR_HIP.
 */
int wf_kv_publish(const wf_kv_pool* pool, const wf_rope* rope,
                  const void* k, int64_t k_row_stride,
                  const void* v, int64_t v_row_stride,
                  const int32_t* pos_thw, int32_t n_tok,
                  int32_t dst_logical_start,
                  void* q_inout, int64_t q_row_stride,
                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * wf_chunk_attn — chunk-wise causal attention forward over the pool
 * ([WF] §3.1).
 *
 * Query groups: group g = 0..n_slots-1 is denoising slot s = first_slot + g
 * and owns query rows [q_slot_start[g], q_slot_start[g+1]).  For every head
 * h and query row i of slot s, with vis(s) the union of the segments whose
 * slot is < 0 or >= s:
 *   z_L   = scale * <q[i][h], K_L[h]>                    for L in vis(s)
 *   out[i][h] = sum_L softmax(z)_L * V_L[h]
 *   lse[h][i] = log(sum_L exp(z_L))          (natural log; if lse != NULL)
 * where K_L, V_L are token L's vectors read through the page table.  Within
 * a chunk the attention is therefore full (bidirectional); across slots it
 * is the j >= s mask.  Keys outside vis(s) are never read, so unmapped or
 * stale pool memory cannot reach the output.
 *
 *   pool           host struct; pages as written by wf_kv_publish
 *   segs, n_segs   host array, 1 <= n_segs <= 64; non-overlapping, inside
 *                  [0, num_logical_pages * page_size), kv_len >= 1
 *   q              device, rows [0, q_slot_start[n_slots]) of
 *                  [num_heads][head_dim]; RoPE already applied
 *   q_row_stride   elements between query rows
 *   q_slot_start   host int32 [n_slots + 1], non-decreasing, first >= 0
 *   n_slots        1..32
 *   first_slot     slot id of group 0 (>= 0); lets one call compute a single
 *                  slot's share, e.g. first_slot = s, n_slots = 1
 *   scale          softmax scale, finite and > 0 (usually 1/sqrt(head_dim))
 *   out            device, same row layout as q, written for every row in
 *                  [q_slot_start[0], q_slot_start[n_slots])
 *   out_row_stride elements between output rows
 *   lse            device float [num_heads][q_slot_start[n_slots]], nullable
 * Every query slot s in [first_slot, first_slot + n_slots) must own at least
 * one segment (slot == s), so no query has an empty key set.  After merging
 * adjacent visible segments the visible ranges of all groups together must
 * number at most 256 (else WF_ERR_UNSUPPORTED).
 * Aliasing: out must not overlap q, lse or the pool.
 * Returns WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED or WF_ERR_HIP.
 */
int wf_chunk_attn(const wf_kv_pool* pool,
                  const wf_segment* segs, int32_t n_segs,
                  const void* q, int64_t q_row_stride,
                  const int32_t* q_slot_start, int32_t n_slots,
                  int32_t first_slot, float scale,
                  void* out, int64_t out_row_stride,
                  float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * wf_group_attn — attention forward for arbitrary query groups over the pool.
 *
 * The same computation as wf_chunk_attn with the visibility given per group
 * instead of derived from slots.  It covers the store stage ("Wave Forcing:
 * Towards Speed-of-Light Streaming Video Generation", overview and §B.1:
 * the store stage runs on its own replica; §3.1: its chunk sits after the
 * anchor and the clean history in the per-layer context), whose queries are
 * the store chunk over anchor | history | store, and any layout where a
 * group's keys are not a slot rule (rotated history, gaps).
 *
 * For every head h, group g and query row i in [q_row_start, q_row_end) of
 * g, with vis(g) the union of the runs runs[run_begin .. run_end):
 *   z_L   = scale * <q[i][h], K_L[h]>                    for L in vis(g)
 *   out[i][h] = sum_L softmax(z)_L * V_L[h]
 *   lse[h * lse_stride + i] = log(sum_L exp(z_L))   (natural log, if lse)
 * Attention inside vis(g) is full; keys outside it are never read.
 *
 *   pool           host struct; pages as written by wf_kv_publish
 *   runs, n_runs   host array, 1 <= n_runs <= 256; each run inside
 *                  [0, num_logical_pages * page_size), kv_len >= 1
 *   groups         host array, 1 <= n_groups <= 32; 0 <= q_row_start <=
 *                  q_row_end; 0 <= run_begin < run_end <= n_runs; the runs
 *                  of one group must not overlap (different groups may share
 *                  keys); the row ranges of different groups must not overlap
 *   q              device, query rows of [num_heads][head_dim], RoPE applied
 *   q_row_stride   elements between query rows
 *   scale          softmax scale, finite and > 0
 *   out            device, same row layout as q; written for every row of
 *                  every group, nothing else
 *   out_row_stride elements between output rows
 *   lse            device float [num_heads][lse_stride], nullable
 *   lse_stride     >= the largest q_row_end (ignored if lse == NULL)
 * After merging adjacent runs, the visible ranges of all groups together
 * must number at most 256 (else WF_ERR_UNSUPPORTED).
 * Aliasing: out must not overlap q, lse or the pool.
 * Returns WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED or WF_ERR_HIP.
 */
typedef struct {
  int32_t kv_start;  /* first logical token of the run */
  int32_t kv_len;    /* tokens in the run, >= 1 */
} wf_kv_run;

typedef struct {
  int32_t q_row_start;  /* query rows [q_row_start, q_row_end) */
  int32_t q_row_end;
  int32_t run_begin;    /* visible keys: runs[run_begin .. run_end) */
  int32_t run_end;
} wf_query_group;

int wf_group_attn(const wf_kv_pool* pool,
                  const wf_kv_run* runs, int32_t n_runs,
                  const wf_query_group* groups, int32_t n_groups,
                  const void* q, int64_t q_row_stride, float scale,
                  void* out, int64_t out_row_stride,
                  float* lse, int64_t lse_stride, hipStream_t stream);

/* ------------------------------------------------------------------------
 * wf_qkv_publish — the QKV projection with the publish fused into its
 * epilogue ([WF] §4.2: K/V are published right after the QKV projection and
 * RoPE).  Projected K and V go straight from the accumulators into the pool;
 * they are never stored as a dense tensor and read back.
 *
 * For t in [0, n_tok), output feature f in [0, 3*H*D):
 *   qkv[t][f] = bf16( sum_k x[t][k] * w_qkv[f][k]  (+ bias[f]) )
 * computed with float32 accumulation and rounded once to bfloat16 (the
 * output of an unfused bfloat16 projection); features [0, H*D) are Q,
 * [H*D, 2*H*D) K and [2*H*D, 3*H*D) V, each [H][D].  Then, exactly as
 * wf_kv_publish with these K and V at dst_logical_start (and q_inout = Q):
 * K and Q are rotated by the 3D RoPE (if rope), K and V are scattered into
 * the pool, and the rotated Q is written to q_out.
 *
 *   pool            bfloat16 pool with head_dim 128 (else WF_ERR_UNSUPPORTED)
 *   rope, pos_thw   as in wf_kv_publish
 *   x               device bf16 [n_tok] rows of [hidden]; 16-byte aligned,
 *                   x_row_stride >= hidden and a multiple of 8 (elements)
 *   hidden          a multiple of 64 in [64, 65536], x_row_stride at most
 *                   2^22 (else WF_ERR_UNSUPPORTED)
 *   w_qkv           device bf16 [3*H*D][hidden], rows contiguous (the layout
 *                   of a fused linear layer's weight); 16-byte aligned
 *   bias            device bf16 [3*H*D], nullable
 *   n_tok, dst_logical_start   as in wf_kv_publish
 *   q_out           device bf16 [n_tok] rows of [H][D], nullable (Q is then
 *                   not computed); q_row_stride as for q in wf_kv_publish
 * The float32 accumulation order is the kernel's own, so a value within
 * float32 rounding of a bfloat16 rounding boundary may round to the other
 * neighbour than a different summation order would.
 * Aliasing: no output may overlap x, w_qkv, bias or each other.
 * Returns WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED or WF_ERR_HIP.
 */
int wf_qkv_publish(const wf_kv_pool* pool, const wf_rope* rope,
                   const void* x, int64_t x_row_stride, int32_t hidden,
                   const void* w_qkv, const void* bias,
                   const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                   void* q_out, int64_t q_row_stride, hipStream_t stream);

/* ----- 8-bit keys and scores ([WF] §5.5: the pages also run attention with
 * 8-bit QK^T, Sage + W8A8) ------------------------------------------------
 *
 * MXFP8 (OCP microscaling FP8): every token's head vector of K is stored as
 * FP8 E4M3 codes with one power-of-two scale per 32 consecutive features:
 *   k8_pages   device uint8 [num_pages][num_heads][page_size][head_dim]
 *              E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
 *              bits; no infinities; 0x7F/0xFF are NaN; largest finite 448)
 *   k8_scales  device uint8 [num_pages][num_heads][page_size][head_dim / 32]
 *              biased exponents e (E8M0): the block's scale is 2^(e - 127)
 * They share the pool's page table and page geometry; both 16-byte aligned.
 * Quantization of a block v[0..31]: e = floor(log2 max|v|) - 8 + 127,
 * clamped to [0, 254] (0 for an all-zero block); code_i = the E4M3 value
 * nearest to v_i / 2^(e - 127), ties to even, saturating at +-448.
 * Built for bfloat16 pools with head_dim 128 (else WF_ERR_UNSUPPORTED).
 */
typedef struct {
  void* k8_pages;
  void* k8_scales;
} wf_mx_keys;

/* wf_kv_publish_mx — wf_kv_publish for the 8-bit variant: K is rotated and
 * rounded to bfloat16 exactly as wf_kv_publish stores it, then quantized to
 * MXFP8 into `keys` (codes and scales of every published row and head); V
 * goes to pool->v_pages as in wf_kv_publish, and q_inout is rotated the same
 * way.  pool->k_pages is neither read nor written and may be NULL.  Other
 * arguments, aliasing and errors as wf_kv_publish; `keys` must not overlap
 * the inputs. */
int wf_kv_publish_mx(const wf_kv_pool* pool, const wf_mx_keys* keys, const wf_rope* rope,
                     const void* k, int64_t k_row_stride,
                     const void* v, int64_t v_row_stride,
                     const int32_t* pos_thw, int32_t n_tok, int32_t dst_logical_start,
                     void* q_inout, int64_t q_row_stride, hipStream_t stream);

/* wf_chunk_attn_mx — wf_chunk_attn with the 8-bit QK^T: for every visible
 * key L, z_L = scale * <mx(q[i][h]), mx(K_L[h])>, where mx(K) are the
 * pool's MXFP8 keys (written by wf_kv_publish_mx) and mx(q) is the bfloat16
 * query quantized by the same rule, per row, head and 32-feature block,
 * inside the call.  Softmax, P V (bfloat16 probabilities, float32
 * accumulation), out and lse as in wf_chunk_attn.  pool->k_pages is not read
 * and may be NULL.  Other arguments, aliasing and errors as wf_chunk_attn. */
int wf_chunk_attn_mx(const wf_kv_pool* pool, const wf_mx_keys* keys,
                     const wf_segment* segs, int32_t n_segs,
                     const void* q, int64_t q_row_stride,
                     const int32_t* q_slot_start, int32_t n_slots, int32_t first_slot,
                     float scale, void* out, int64_t out_row_stride, float* lse,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * wf_history_rotate — end-of-round history rotation by page-table edits
 * ([WF] §3.1: the context holds a bounded clean history, oldest first,
 * followed by the live store; when a round completes a chunk, the store joins
 * the history as its newest chunk and the oldest history chunk leaves).
 *
 * The window of logical tokens [window_start, window_start + n_chunks *
 * chunk_stride) holds n_chunks chunks of chunk_stride tokens each: the
 * history chunks, oldest first, then the live store.  The call rotates the
 * window's page-table entries left by one chunk, in place:
 *   new[w0 + i] = old[w0 + (i + cp) mod n]     for i in [0, n)
 * with w0 = window_start / page_size, cp = chunk_stride / page_size and
 * n = n_chunks * cp.  Afterwards the history reads, oldest first, the old
 * history without its oldest chunk and then the old store; the store position
 * maps to the evicted chunk's physical pages, which the next round's
 * wf_kv_publish of the store overwrites.  No K/V byte moves and no other
 * entry changes.  Copy-free rotation needs chunks that start on page
 * boundaries: window_start and chunk_stride must be multiples of page_size
 * (a chunk of C tokens then occupies ceil(C / page_size) pages; the tail of
 * its last page is a gap that no segment names).
 *
 *   page_table       device int32 [num_logical_pages] (the pool's table),
 *                    updated in place; its entries are moved, never read
 *                    as page numbers
 *   num_logical_pages, page_size   as in the pool
 *   window_start     >= 0, multiple of page_size
 *   chunk_stride     >= page_size, multiple of page_size
 *   n_chunks         >= 1 (1 is a no-op); the window must end at or before
 *                    num_logical_pages * page_size and span at most 16384
 *                    pages (else WF_ERR_UNSUPPORTED)
 * Stream-ordered like every call: attention or publish work enqueued earlier
 * on the stream sees the old table, later work the new one.
 * Returns WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED or WF_ERR_HIP.
 */
int wf_history_rotate(int32_t* page_table, int32_t num_logical_pages, int32_t page_size,
                      int32_t window_start, int32_t chunk_stride, int32_t n_chunks,
                      hipStream_t stream);

/* Message describing the last failure of a wf_* call on this thread ("" if
 * the last call succeeded).  The string is owned by the library. */
const char* wf_last_error(void);

/* Reads (and, if clear != 0, resets) the status word of the current device:
 * an OR of WF_STATUS_* bits raised by kernels since the last reset.  This
 * call synchronizes the device.  Returns WF_OK or WF_ERR_HIP. */
int wf_device_status(int32_t* status, int32_t clear);

/* Library version, e.g. "libwf 0.1.0 gfx950". */
const char* wf_version(void);

#ifdef __cplusplus
}
#endif
#endif /* WF_H */

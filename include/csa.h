/*
 * csa.h -- C ABI of the CSA / HCA long-context attention hot path (gfx950).
 *
 * The operations follow the description of DeepSeek-V4's hybrid attention in
 * the b-lab.team summary of the DeepSeek-V4 report ("Core Methodological
 * Innovations", item 1, Hybrid Attention Architecture, CSA and HCA bullets;
 * item 4, Quantization-Aware Training bullet for the FP4 indexer path).  Where
 * that text leaves a step open, the reading taken is stated at the function.
 *
 * Conventions (all functions):
 *   - Every pointer argument except `stream` and the csa_tensor / status
 *     structures themselves is DEVICE memory owned by the caller.  The library
 *     never allocates or frees device memory; scratch comes in through `ws`.
 *   - Every call only enqueues work on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and returns; results are ready when
 *     the stream has reached that point.
 *   - Scalars, null pointers, dtype/shape support and workspace sizes are
 *     checked on the host BEFORE anything is launched; on any error nothing
 *     has been enqueued and the return value says why (details in
 *     csa_last_error(), a thread-local string).  Device-resident metadata
 *     (q_pos, raw_base, block_first, block_count, idx) is a documented
 *     precondition and is not validated.  NaN/Inf inputs give unspecified
 *     results.
 *   - Results are deterministic: the same inputs give bitwise the same
 *     outputs, independent of `batch` (each sequence's work is split only by
 *     its own sizes; no floating-point atomics).
 *   - Positions are absolute token positions (0-based).  Compressed block j of
 *     block size m covers raw positions [j*m, j*m+m-1] and is visible to a
 *     query at position t once it is complete: j*m + m - 1 <= t.  The sliding
 *     window of a query at t is raw positions max(0, t-W+1) .. t.
 *   - Rows of every stored tensor hold `dim` contiguous elements.
 *
 * Calls that overlap on one stream are ordered; calls on different streams
 * that share a workspace race.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL                              */
  CSA_ERR_SHAPE = 2,       /* a size/stride argument is out of range                  */
  CSA_ERR_DTYPE = 3,       /* a dtype code is unknown or the combination is invalid   */
  CSA_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. heads not multiple of 16) */
  CSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returns   */
  CSA_ERR_HIP = 6          /* a HIP launch failed; see csa_last_error()               */
} csa_status;

/* Element formats of stored tensors.
 *   CSA_F32       float32.
 *   CSA_BF16      bfloat16 (round-to-nearest-even from fp32 when written here).
 *   CSA_FP8_E4M3  OCP e4m3 ("fn", max 448) codes with one float32 scale per row:
 *                 value = e4m3(code) * scale[row]; a NULL scale means 1.0.  When
 *                 written here: scale = amax/448 in fp32 (1 for an all-zero row),
 *                 code = RNE(x/scale) with the quotient in fp32, saturated.
 *   CSA_MXFP4     OCP MX FP4: e2m1 codes packed two per byte (element 2i in the
 *                 low nibble of byte i) plus one e8m0 scale byte per 32 elements:
 *                 value = e2m1(code) * 2^(scale-127).  When written here: scale
 *                 exponent e = floor(log2(amax)) - 2 clamped to [-127,127]
 *                 (code 0 and all-zero elements for an all-zero block), element =
 *                 RNE(x / 2^e) on {0,.5,1,1.5,2,3,4,6}, saturated, sign copied. */
typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_MXFP4 = 3 } csa_dtype;

/* A strided [batch, rows, dim] tensor in device memory.
 *   data        element storage (MXFP4: packed codes).
 *   scale       FP8: float per row; MXFP4: uint8 per 32 elements; else ignored.
 *   stride_b    distance between batch items, in elements (MXFP4: bytes).
 *   stride_row  distance between rows, in elements (MXFP4: bytes).
 *   scale_stride_b / scale_stride_row: the same for `scale`, in scale entries
 *               (FP8: floats, MXFP4: bytes).  Within a row the dim/32 MXFP4
 *               scales are contiguous. */
typedef struct csa_tensor {
  void* data;
  void* scale;
  int32_t dtype;
  int32_t reserved;
  int64_t stride_b;
  int64_t stride_row;
  int64_t scale_stride_b;
  int64_t scale_stride_row;
} csa_tensor;

int32_t csa_abi_version(void);
const char* csa_status_string(csa_status s);
const char* csa_last_error(void);

/* ---------------------------------------------------------------------------
 * (a) KV compression.  CSA shrinks the KV cache m-fold by merging each run of
 * m neighbouring entries into one; HCA does the same with a much larger m'
 * (b-lab.team summary, Core Methodological Innovations 1, CSA and HCA bullets).  Reading of the
 * merge: c_j = sum_{r<m} softmax(logits)_r * x[j*m + r], one logit per offset,
 * shared by every channel and block, softmax computed in fp32 (max-subtracted),
 * terms accumulated in fp32 in ascending r.
 *
 *   raw          [batch, R, dim], dtype F32, BF16 or FP8_E4M3; row r of sequence
 *                b holds absolute position raw_base[b] + r.
 *   raw_base     [batch] int32.
 *   logits       [m] float.
 *   m            block size, 1..1024.
 *   dim          row length (MXFP4 output: a multiple of 32; <= 4096).
 *   block_first, block_count  [batch] int32: produce blocks
 *                j = block_first[b] .. block_first[b] + block_count[b] - 1.
 *                Precondition: their raw rows lie inside [0, R) and j indexes a
 *                row of `out`; 0 <= block_count[b] <= max_blocks.
 *   max_blocks   host-side upper bound of block_count (sizes the launch).
 *   out          [batch, N_cap, dim] destination cache, dtype F32, BF16,
 *                FP8_E4M3 (row scale written) or MXFP4 (scales written); only
 *                rows j listed above are written.
 * ------------------------------------------------------------------------- */
csa_status csa_compress(const csa_tensor* raw, const int32_t* raw_base, const float* logits, int32_t m,
                        int32_t dim, const int32_t* block_first, const int32_t* block_count, int32_t max_blocks,
                        int32_t batch, const csa_tensor* out, void* stream);

/* Several independent compressions in one launch (e.g. the KV stream and the
 * indexer-key stream of a decode step, whose short chains of dependent loads
 * then overlap).  Each job has exactly the arguments, preconditions and result
 * of one csa_compress call; jobs must not write the same output rows.  The job
 * array is HOST memory, read before the call returns; n_jobs <= 4.  Any
 * invalid job fails the whole call (nothing is enqueued); the error message
 * names the job. */
#define CSA_MAX_COMPRESS_JOBS 4
typedef struct csa_compress_job {
  csa_tensor raw;
  const int32_t* raw_base;
  const float* logits;
  int32_t m;
  int32_t dim;
  const int32_t* block_first;
  const int32_t* block_count;
  int32_t max_blocks;
  int32_t batch;
  csa_tensor out;
} csa_compress_job;
csa_status csa_compress_jobs(const csa_compress_job* jobs, int32_t n_jobs, void* stream);

/* ---------------------------------------------------------------------------
 * Indexer query from the query hidden state (the step before (b)): for every
 * query row, c = W_dq h (rank r), q_idx = reshape(W_uq c, [n_idx_heads,
 * idx_dim]) and w = W_w h -- the indexer scores with low-rank projections of
 * the query hidden state h_t (b-lab.team summary of DeepSeek-V4, Core
 * Methodological Innovations 1, CSA bullet).  No norm or activation between.
 *   h      [batch, tq, d_model] BF16 (stride_b, stride_row in elements).
 *   w_dq   [rank, d_model], w_uq [n_idx_heads * idx_dim, rank] and w_w
 *          [n_idx_heads, d_model]: BF16, row pitch stride_row (stride_b unused).
 *   q_idx  [batch, tq, n_idx_heads, idx_dim] F32 or BF16 (stride_b, stride_row in
 *          elements; a row's n_idx_heads * idx_dim values contiguous).
 *   w      [batch, tq, n_idx_heads] float, contiguous.
 *   ws     at least csa_index_query_workspace_size(...) bytes; contents on entry
 *          do not matter.
 * Arithmetic: bf16 products summed in fp32, in chunks of 128 along d_model (rank)
 * added in a fixed order, so results do not depend on batch or tq; c is rounded
 * to bf16 before the second projection.  d_model and rank must be multiples of
 * 32 (at most 65536), n_idx_heads * idx_dim at most 65536, every row pitch a
 * multiple of 8 elements and every pointer 16-byte aligned (CSA_ERR_SHAPE
 * otherwise).
 * ------------------------------------------------------------------------- */
csa_status csa_index_query(const csa_tensor* h, const csa_tensor* w_dq, const csa_tensor* w_uq,
                           const csa_tensor* w_w, int32_t batch, int32_t tq, int32_t d_model, int32_t rank,
                           int32_t n_idx_heads, int32_t idx_dim, const csa_tensor* q_idx, float* w, void* ws,
                           size_t ws_bytes, void* stream);
size_t csa_index_query_workspace_size(int32_t batch, int32_t tq, int32_t d_model, int32_t rank,
                                      int32_t n_idx_heads, int32_t idx_dim);

/* ---------------------------------------------------------------------------
 * MLA projections on either side of attention over the shared latent rows
 * (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
 * bullet: attention reads the compressed latent entries; head h's key is
 * W_uk[h] c and its value W_uv[h] c for a latent row c, so the key projection
 * moves onto the query and the value projection onto the output):
 *   csa_latent_query:  q_lat[r, h, :] = W_uk[h]^T q[r, h, :]
 *   csa_latent_output: out[r, h, :]  = W_uv[h] o_lat[r, h, :]
 * rows = batch * tq query rows; every array contiguous.
 *   q       [rows, heads, head_dim] BF16.
 *   w_uk_t  [heads, dim, head_dim] BF16: each head's key up-projection stored
 *           transposed (row j holds column j of W_uk[h]).
 *   q_lat   [rows, heads, dim] BF16 (the BF16 query csa_sparse_attn takes).
 *   o_lat   [rows, heads, dim] F32 (the attention output as csa_sparse_attn /
 *           hca_attn write it).
 *   w_uv    [heads, head_dim, dim] BF16: each head's value up-projection.
 *   out     [rows, heads, head_dim] of out_dtype, F32 or BF16.
 *   ws      at least the matching *_workspace_size(...) bytes; contents on entry
 *           do not matter.
 * Arithmetic: bf16 products summed in fp32 in chunks of 128 along the summed
 * dimension, added in a fixed order (results do not depend on rows); o_lat
 * enters as bf16 hi + lo (about 16 significant bits).  Limits: rows <= 1048576,
 * heads in [1, 65535], head_dim and dim multiples of 32 in [32, 65536], inputs
 * and weights 16-byte aligned (CSA_ERR_SHAPE otherwise).  The workspace-size
 * functions return 0 for unsupported shapes.
 * ------------------------------------------------------------------------- */
csa_status csa_latent_query(const void* q, const void* w_uk_t, int32_t rows, int32_t heads, int32_t head_dim,
                            int32_t dim, void* q_lat, void* ws, size_t ws_bytes, void* stream);
size_t csa_latent_query_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t dim);
csa_status csa_latent_output(const float* o_lat, const void* w_uv, int32_t rows, int32_t heads, int32_t head_dim,
                             int32_t dim, void* out, csa_dtype out_dtype, void* ws, size_t ws_bytes, void* stream);
size_t csa_latent_output_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t dim);

/* ---------------------------------------------------------------------------
 * (b) Lightning-indexer scores.  The indexer scores every compressed block
 * from low-rank projections of the query's hidden state, and its scores pick
 * the k blocks to attend to (b-lab.team summary, Core Methodological
 * Innovations 1, CSA bullet); the indexer QK path is FP4 (same page, item 4, Quantization-
 * Aware Training).  Reading of the formula (the pages give none): the
 * DeepSeek-V3.2 lightning-indexer form
 *     I[b,t,j] = sum_h w[b,t,h] * max(0, <q_idx[b,t,h], k_idx[b,j]>)
 * for visible j (j*m+m-1 <= q_pos[b,t]), -inf for j >= visible count.
 *
 *   q_idx   [batch, tq, n_idx_heads, idx_dim]: stride_b / stride_row step batch
 *           and query; heads*idx_dim contiguous.  dtype F32 (keys F32, BF16 or
 *           MXFP4; with MXFP4 keys q is quantised to MXFP4 inside by the rule
 *           above) or BF16 (keys BF16).
 *   w       [batch, tq, n_idx_heads] float, contiguous.
 *   k_idx   [batch, n_cap, idx_dim] compressed indexer keys: F32, BF16 or MXFP4.
 *   q_pos   [batch, tq] int32 query positions; precondition visible <= n_cap.
 *   n_idx_heads, idx_dim  >= 1.  F32 / BF16 keys: n_idx_heads * idx_dim <= 8192
 *           (8 heads of 64 with a BF16 query use bf16 MFMA, other shapes the
 *           fp32 VALU kernel).  MXFP4 keys: idx_dim == 64 and n_idx_heads <= 32.
 *           Anything else is CSA_ERR_UNSUPPORTED.
 *   scores  [batch, tq, n_cap] float, contiguous (every entry written).
 * ------------------------------------------------------------------------- */
csa_status csa_index_scores(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                            const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads,
                            int32_t idx_dim, int32_t m, int32_t n_cap, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * (c) Top-k block selection: the k highest-scoring compressed blocks of each
 * query (b-lab.team summary, Core Methodological Innovations 1, CSA bullet).
 * Reading of the order: score descending, then block index ascending; -0.0
 * equals +0.0.  Only the visible blocks j < (q_pos+1)/m of each row take part.
 *
 *   scores  [batch, tq, n_cap] float.
 *   idx     [batch, tq, k] int32 output: the selected block indices in
 *           ascending order, then -1 for the slots beyond the visible count.
 *   ws      workspace of at least csa_topk_workspace_size() bytes; its
 *           contents on entry do not matter.
 * ------------------------------------------------------------------------- */
csa_status csa_topk(const float* scores, const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_cap,
                    int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);
size_t csa_topk_workspace_size(int32_t batch, int32_t tq, int32_t n_cap, int32_t k);

/* ---------------------------------------------------------------------------
 * (b)+(c) fused: indexer scores and top-k selection in one call.  idx equals
 * what csa_topk returns for the scores csa_index_scores computes, bit for bit.
 *   scores  [batch, tq, n_cap] float, or NULL.  When given, every score is
 *           written there (exactly csa_index_scores' result).  When NULL, the
 *           scores are not returned and, where the fused path applies, mostly
 *           never stored at all.
 *   ws      at least csa_index_topk_workspace_size(batch, tq, n_cap, k,
 *           scores != NULL) bytes; its contents on entry do not matter.
 * With MXFP4 keys on rows longer than the single-workgroup top-k (n_cap >
 * 20480, at most 262,144), each indexer workgroup also lists its 1024-block
 * slice's candidates as it scores them (every block at or above a cut of the
 * slice's scores), and one merge pass selects the row's top-k from the lists,
 * certified exact.  Rows with few full slices are selected from their scores,
 * kept in the workspace.  The rare rows whose certificate fails are selected
 * again: over the lists plus every score of the failing slices when at most 8
 * fail, else over the whole row.  Those scores are the caller's when kept,
 * otherwise recomputed with the indexer's arithmetic.
 * Other shapes run the two stages one after the other.
 * ------------------------------------------------------------------------- */
csa_status csa_index_topk(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx, const int32_t* q_pos,
                          int32_t batch, int32_t tq, int32_t n_idx_heads, int32_t idx_dim, int32_t m,
                          int32_t n_cap, int32_t k, float* scores, int32_t* idx, void* ws, size_t ws_bytes,
                          void* stream);
size_t csa_index_topk_workspace_size(int32_t batch, int32_t tq, int32_t n_cap, int32_t k, int32_t scores_kept);
/* csa_index_topk in two launches, for callers that schedule (or time) the scoring
 * and the selection separately: part 1 scores (and, where the fused path applies,
 * leaves the slices' candidates in ws), part 2 selects; part 3 is both, exactly
 * csa_index_topk.  A part-2 call must follow a part-1 call with the same
 * arguments on the same stream, with scores and ws untouched in between; its
 * result then equals csa_index_topk's bit for bit.  idx may be NULL for part 1;
 * scores may be NULL as for csa_index_topk. */
csa_status csa_index_topk_part(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                               const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads,
                               int32_t idx_dim, int32_t m, int32_t n_cap, int32_t k, float* scores, int32_t* idx,
                               void* ws, size_t ws_bytes, int32_t part, void* stream);

/* (a)+(b)+(c) of one decode step in as few launches as the shapes allow: exactly
 * csa_compress_jobs over kv_job and key_job (either may be NULL) followed by
 * csa_index_topk_part(..., part), bit for bit, with the same arguments and
 * requirements.  The compressions only run for part 1 or 3.  When the indexer
 * scores MXFP4 keys with slice candidates (see csa_index_topk), tq == 1, the key
 * job writes the very key tensor being scored (k_idx: same pointers and strides,
 * dim 64, m <= 4, max_blocks <= 4, batch equal) and the KV job has m <= 16 and
 * dim <= 512, both
 * jobs run inside the indexer launch: KV blocks on extra workgroups, and each new
 * key by the wave that scores it, before that wave reads its keys.  Otherwise the
 * jobs run in a launch of their own first.  Errors: as csa_compress_jobs (the
 * message names the job) and csa_index_topk_part. */
csa_status csa_compress_index_topk(const csa_compress_job* kv_job, const csa_compress_job* key_job,
                                   const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                                   const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads,
                                   int32_t idx_dim, int32_t m, int32_t n_cap, int32_t k, float* scores, int32_t* idx,
                                   void* ws, size_t ws_bytes, int32_t part, void* stream);

/* ---------------------------------------------------------------------------
 * (d) CSA sparse attention: attention over the selected compressed entries
 * plus a sliding window of raw local entries, which both CSA and HCA add to
 * keep fine-grained local context (b-lab.team summary, Core Methodological
 * Innovations 1, HCA bullet).  Readings: key = value = the stored row (shared
 * MQA latent); the entry list is the selected compressed rows followed by the
 * window's raw rows, not de-duplicated, in ONE softmax:
 *     l_e = scale * <q[b,t,h], e>,  out = sum_e softmax(l)_e * e,
 *     lse = log sum_e exp(l_e)  (natural log).
 *
 *   q       [batch, tq, heads, dim]: stride_b / stride_row step batch and query,
 *           heads*dim contiguous.  dtype F32 with F32 caches, BF16 otherwise.
 *   kv_cmp  [batch, N_cap, dim] compressed cache: F32, BF16 or FP8_E4M3.
 *   idx     [batch, tq, k] int32 from csa_topk (-1 slots are skipped).
 *           Precondition: every index >= 0 is a visible block.
 *   kv_raw  [batch, R, dim] raw rows (same dtype as kv_cmp); row r holds
 *           position raw_base[b] + r.  Precondition: the window of every
 *           query lies inside it.
 *   out     [batch, tq, heads, dim] float; lse [batch, tq, heads] float or NULL.
 *   ws      at least csa_attn_workspace_size(batch, tq, heads, dim, k + window).
 * Supported: F32 path heads <= 64, dim <= 512, dim % 4 == 0, k + window <=
 * 8192; BF16 / FP8 path heads a multiple of 16 up to 64, dim == 512 and
 * k + window <= 131072 (64 splits of at most 2048 entries).  Anything else is
 * CSA_ERR_UNSUPPORTED, reported before any launch.
 * ------------------------------------------------------------------------- */
csa_status csa_sparse_attn(const csa_tensor* q, const csa_tensor* kv_cmp, const int32_t* idx, int32_t k,
                           const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window,
                           const int32_t* q_pos, int32_t batch, int32_t tq, int32_t heads, int32_t dim,
                           float scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * (e) HCA attention: dense attention over every complete heavily-compressed
 * block plus the same sliding window: HCA compresses m'-fold and then attends
 * densely to everything that remains (b-lab.team summary, Core Methodological
 * Innovations 1, HCA bullet).  Same readings and formats
 * as csa_sparse_attn; the compressed entries of a query at t are blocks
 * 0 .. (t+1)/m_hc - 1 of kv_hc (precondition: <= n_cap_hc).
 *   ws  at least csa_attn_workspace_size(batch, tq, heads, dim, n_cap_hc + window).
 * ------------------------------------------------------------------------- */
csa_status hca_attn(const csa_tensor* q, const csa_tensor* kv_hc, int32_t m_hc, int32_t n_cap_hc,
                    const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window, const int32_t* q_pos,
                    int32_t batch, int32_t tq, int32_t heads, int32_t dim, float scale, float* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

size_t csa_attn_workspace_size(int32_t batch, int32_t tq, int32_t heads, int32_t dim, int32_t n_entries_max);

/* ---------------------------------------------------------------------------
 * Allocation-free csa_sparse_attn, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as csa_sparse_attn
 * minus the workspace: the split partials live in a static device array of
 * CSA_NOALLOC_SCRATCH_BYTES (64 MiB), one per device, held
 * until the process ends.  Calls whose csa_attn_workspace_size exceeds it get
 * CSA_ERR_WORKSPACE before any launch.  The call itself allocates nothing; its
 * first call on a device looks up the array's address there.  Every call on a
 * device shares that device's array (nothing in it needs clearing: each call
 * writes every partial it reads), so calls that overlap in time on one device
 * (different streams) race; calls on one stream are ordered.
 * ------------------------------------------------------------------------- */
csa_status csa_sparse_attn_noalloc(const csa_tensor* q, const csa_tensor* kv_cmp, const int32_t* idx, int32_t k,
                                   const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window,
                                   const int32_t* q_pos, int32_t batch, int32_t tq, int32_t heads, int32_t dim,
                                   float scale, float* out, float* lse, void* stream);
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ---------------------------------------------------------------------------
 * Quantisers (the FP4 indexer path: b-lab.team summary, Core Methodological
 * Innovations 4, Quantization-Aware Training; fp8 KV is a storage variant).
 *   csa_quantize_mxfp4: x [rows, cols] float (cols % 32 == 0) -> codes
 *     [rows, cols/2] uint8 and scales [rows, cols/32] uint8 (rule at CSA_MXFP4).
 *   csa_quantize_fp8:   x [rows, cols] float -> codes [rows, cols] uint8 and
 *     row_scale [rows] float (rule at CSA_FP8_E4M3).  cols <= 8192.
 * ------------------------------------------------------------------------- */
csa_status csa_quantize_mxfp4(const float* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream);
csa_status csa_quantize_fp8(const float* x, int64_t rows, int32_t cols, uint8_t* codes, float* row_scale,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Measurement: the device's HBM streaming-read ceiling, the practical bound the
 * bandwidth-bound stages are compared with beside the nominal peak.  Not part of
 * the attention path.
 *   csa_stream_read reads every byte of data[0, bytes) once (bytes % 16 == 0,
 *   data 16-byte aligned) and writes one word per workgroup to sink, which must
 *   hold csa_stream_read_sink_size() bytes.  Time it with events around the call.
 * ------------------------------------------------------------------------- */
csa_status csa_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream);
size_t csa_stream_read_sink_size(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */

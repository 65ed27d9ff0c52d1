// Internal launch interface between the C ABI layer (abi.cpp) and the kernel
// translation units.  Arguments arrive validated; launchers only enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

struct TensorView {
  const void* data;
  const void* scale;
  int dtype;
  int64_t sb, sr;    // batch / row strides (elements; MXFP4: bytes)
  int64_t ssb, ssr;  // scale strides
};

inline TensorView view_of(const csa_tensor* t) {
  TensorView v;
  v.data = t->data;
  v.scale = t->scale;
  v.dtype = t->dtype;
  v.sb = t->stride_b;
  v.sr = t->stride_row;
  v.ssb = t->scale_stride_b;
  v.ssr = t->scale_stride_row;
  return v;
}

// ---------------------------------------------------------------- compression
struct CompressArgs {
  TensorView raw;
  const int32_t* raw_base;
  const float* logits;
  int m, dim;
  const int32_t* block_first;
  const int32_t* block_count;
  int max_blocks, batch;
  void* out;
  void* out_scale;
  int out_dtype;
  int64_t out_sb, out_sr, out_ssb, out_ssr;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
constexpr int kMaxCompressJobs = 4;
hipError_t launch_compress_jobs(const CompressArgs* jobs, int n, hipStream_t s);  // n <= kMaxCompressJobs
hipError_t launch_quantize_mxfp4(const float* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
hipError_t launch_quantize_fp8(const float* x, int64_t rows, int cols, uint8_t* codes, float* row_scale,
                               hipStream_t s);

// ---------------------------------------------------------------- indexer
struct IndexArgs {
  TensorView q;  // [B, Tq, H_I, d_I]
  const float* w;
  TensorView k;  // [B, N, d_I]
  const int32_t* q_pos;
  int batch, tq, heads, dim, m, n_cap;
  float* scores;
};
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s);

// ---------------------------------------------------------------- top-k
// Rows longer than this are selected by the multi-workgroup path.
constexpr int kTopkLdsMax = 20480;
constexpr int kTopkSlice = 4096;  // keys per candidate workgroup on long rows
size_t topk_workspace_bytes(int64_t rows, int n_cap, int k);
hipError_t launch_topk(const float* scores, const int32_t* q_pos, int batch, int tq, int n_cap, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s);

// A slice's candidate list, as written by a candidate pass: up to C (order-preserving
// score key, block index) pairs in ascending index order, empty slots (0, 0) after
// them, and:
struct SliceMeta {
  uint32_t count;     // candidates written
  uint32_t trunc;     // 1 when some visible key of the slice was left out
  uint32_t last_key;  // every key left out ranks strictly after (last_key, last_idx)
  uint32_t last_idx;  //   in (key desc, index asc) order (when trunc)
};
struct CandOut {
  int C, slice, nslices;  // candidates per slice, keys per slice, slices per row
  uint2* cand;            // [rows][nslices][C]
  SliceMeta* meta;        // [rows][nslices]
  int k;                  // rows with at most k visible keys need no candidates
  float* row_scores;      // [rows][n_cap] where short rows' scores go when the caller keeps none
};

// Fused (b)+(c) for MXFP4 keys on long rows: the indexer's workgroups also emit
// their 1024-key slice's candidate list, and one merge pass selects the top-k.
constexpr int kFusedSlice = 1024;  // keys per indexer workgroup
constexpr int kFusedC = 32;        // list slots per slice (the slice's exact top-32)
bool index_topk_fused_ok(const IndexArgs& a, int k);
// Rows whose full slices alone cannot hold more than k candidates (each full slice
// lists kFusedC keys) are selected from their scores: the indexer writes them.
__host__ __device__ inline bool index_topk_short_row(int visible, int k) { return kFusedC * (visible / kFusedSlice) <= k; }
size_t index_topk_workspace_bytes(int64_t rows, int n_cap, int k, bool scores_in_ws);
// Where the score rows start in that workspace (when the caller keeps none).
size_t index_topk_score_offset(int64_t rows, int n_cap, int k);
// A decode step's compressions, run by the indexer launch (index.hip): the KV
// compression on extra workgroups, and the indexer-key compression by the waves
// whose keys include a block just completed (they compress it, store it and score
// it), so no launch of its own precedes the scoring.  batch == 0: no such job.
// Preconditions (checked by the caller): tq == 1; key.out is the indexer's key
// tensor (MXFP4, dim 64), key.m <= kFusedCompressMaxM and key.max_blocks <=
// kFusedCompressMaxNew; kv.m <= 16, kv.dim <= 512.
constexpr int kFusedCompressMaxM = 4;    // the indexer-key job's block size m (CSA)
constexpr int kFusedCompressMaxNew = 4;  // and its blocks per sequence (max_blocks)
struct FusedCompress {
  CompressArgs key, kv;
  int key_in, kv_in;  // raw row format of each job: 0 F32, 1 BF16, 2 FP8
  int nslices, rows;  // scoring workgroups per row, query rows (set by the launcher)
};
hipError_t launch_index_scores_cand(const IndexArgs& a, const CandOut& c, hipStream_t s,
                                    const FusedCompress* fc = nullptr);  // index.hip
// the two kernels of launch_index_topk, one launch each
hipError_t launch_index_topk_cand(const IndexArgs& a, int k, void* ws, hipStream_t s,
                                  const FusedCompress* fc = nullptr);
hipError_t launch_index_topk_merge(const IndexArgs& a, int k, int32_t* idx, void* ws, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  TensorView q;        // [B, Tq, H, D]
  TensorView kv;       // compressed cache
  const int32_t* idx;  // CSA: [B, Tq, k]; HCA: nullptr
  int k;               // CSA: slots per query
  int m_hc;            // HCA block size (0 for CSA)
  int n_cap;           // HCA cache capacity
  TensorView raw;
  const int32_t* raw_base;
  int window;
  const int32_t* q_pos;
  int batch, tq, heads, dim;
  float scale;
  float* out;
  float* lse;
  void* ws;
};
// A query row's entry list is cut into at most kAttnMaxSplits splits of at most
// kAttnMaxSplitEntries entries each.
constexpr int kAttnMaxSplits = 64;
constexpr int kAttnMaxSplitEntries = 2048;
int attn_split_size(int tq, int n_entries_max, bool dense);  // dense: HCA (every visible block)
size_t attn_workspace_bytes(int64_t rows, int heads, int dim, int n_entries_max, int tq);
hipError_t launch_attention(const AttnArgs& a, int n_entries_max, hipStream_t s);

// ---------------------------------------------------------------- indexer query
// [c | w] = h . [W_dq ; W_w]^T, then q_I = bf16(c) . W_uq^T (project.hip).
struct IndexQueryArgs {
  const void* h;  // bf16 [batch, tq, d_model] (element strides h_sb, h_sr)
  int64_t h_sb, h_sr;
  const void* w_dq;  // bf16 [rank, d_model], row pitch ld_dq
  const void* w_uq;  // bf16 [H_I * d_I, rank], row pitch ld_uq
  const void* w_w;   // bf16 [H_I, d_model], row pitch ld_w
  int64_t ld_dq, ld_uq, ld_w;
  int batch, tq, d_model, rank, n_idx_heads, idx_dim;
  void* q_out;  // f32 or bf16 [batch, tq, H_I * d_I] (element strides q_sb, q_sr)
  int64_t q_sb, q_sr;
  int q_bf16;
  float* w_out;  // [batch, tq, H_I]
  void* ws;
};
size_t index_query_workspace_bytes(int64_t rows, int d_model, int rank, int n_idx_heads, int idx_dim);
hipError_t launch_index_query(const IndexQueryArgs& a, hipStream_t s);

// Per-head products Y_z = X_z . W_z^T (MLA absorbed query, output up-projection):
// X [rows, heads, K] (bf16, or fp32 taken as bf16 hi + lo), W [heads, N, K] bf16,
// Y [rows, heads, N] fp32 or bf16; ws holds latent_proj_workspace_bytes.
struct LatentProjArgs {
  const void* x;
  int x_f32;
  const void* w;
  int64_t rows;
  int heads, K, N;
  void* y;
  int y_bf16;
  void* ws;
};
size_t latent_proj_workspace_bytes(int64_t rows, int heads, int K, int N);
hipError_t launch_latent_proj(const LatentProjArgs& a, hipStream_t s);

// ---------------------------------------------------------------- measurement
constexpr int kStreamReadBlocks = 2048;  // workgroups of the streaming-read probe (one sink word each)
hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace csa

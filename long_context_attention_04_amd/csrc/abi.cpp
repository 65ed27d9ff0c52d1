// C ABI of the CSA / HCA hot path: host-side validation and dispatch.
//
// Every check runs before anything is enqueued, so a call either enqueues its
// whole work or nothing.  Device-resident metadata (positions, bases, block
// lists, indices) is a documented precondition and is not read on the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/csa.h"
#include "kernels.h"

#include <algorithm>

namespace csa {
bool attn_plain_fits(int n_entries_max);
}

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa_status ok() {
  g_last_error.clear();
  return CSA_OK;
}

csa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool known_dtype(int d) { return d >= CSA_F32 && d <= CSA_MXFP4; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

csa_status check_tensor(const csa_tensor* t, const char* name) {
  REQUIRE(t != nullptr, CSA_ERR_NULL, "%s is NULL", name);
  REQUIRE(t->data != nullptr, CSA_ERR_NULL, "%s->data is NULL", name);
  REQUIRE(known_dtype(t->dtype), CSA_ERR_DTYPE, "%s has unknown dtype %d", name, t->dtype);
  REQUIRE(t->stride_b >= 0 && t->stride_row >= 0, CSA_ERR_SHAPE, "%s has a negative stride", name);
  if (t->dtype == CSA_MXFP4) REQUIRE(t->scale != nullptr, CSA_ERR_NULL, "%s is MXFP4 but has no scale", name);
  return CSA_OK;
}

}  // namespace

extern "C" {

int32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "null pointer";
    case CSA_ERR_SHAPE: return "invalid shape or size";
    case CSA_ERR_DTYPE: return "invalid dtype";
    case CSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

// Validates one compression's arguments and fills its launch description.
static csa_status compress_args(const csa_tensor* raw, const int32_t* raw_base, const float* logits, int32_t m,
                                int32_t dim, const int32_t* block_first, const int32_t* block_count,
                                int32_t max_blocks, int32_t batch, const csa_tensor* out, csa::CompressArgs* a) {
  csa_status st;
  if ((st = check_tensor(raw, "raw")) != CSA_OK) return st;
  if ((st = check_tensor(out, "out")) != CSA_OK) return st;
  REQUIRE(raw_base && logits && block_first && block_count, CSA_ERR_NULL, "raw_base/logits/block_first/block_count is NULL");
  REQUIRE(raw->dtype != CSA_MXFP4, CSA_ERR_DTYPE, "raw rows must be F32, BF16 or FP8_E4M3");
  REQUIRE(m >= 1 && m <= 1024, CSA_ERR_SHAPE, "m=%d outside [1, 1024]", m);
  REQUIRE(dim >= 1 && dim <= 4096, CSA_ERR_SHAPE, "dim=%d outside [1, 4096]", dim);
  REQUIRE(batch >= 0 && max_blocks >= 0, CSA_ERR_SHAPE, "negative batch or max_blocks");
  if (out->dtype == CSA_MXFP4) REQUIRE(dim % 32 == 0, CSA_ERR_SHAPE, "MXFP4 output needs dim %% 32 == 0 (dim=%d)", dim);
  if (out->dtype == CSA_FP8_E4M3) REQUIRE(out->scale != nullptr, CSA_ERR_NULL, "FP8 output needs a row-scale pointer");
  a->raw = csa::view_of(raw);
  a->raw_base = raw_base;
  a->logits = logits;
  a->m = m;
  a->dim = dim;
  a->block_first = block_first;
  a->block_count = block_count;
  a->max_blocks = max_blocks;
  a->batch = batch;
  a->out = out->data;
  a->out_scale = out->scale;
  a->out_dtype = out->dtype;
  a->out_sb = out->stride_b;
  a->out_sr = out->stride_row;
  a->out_ssb = out->scale_stride_b;
  a->out_ssr = out->scale_stride_row;
  return CSA_OK;
}

csa_status csa_compress(const csa_tensor* raw, const int32_t* raw_base, const float* logits, int32_t m, int32_t dim,
                        const int32_t* block_first, const int32_t* block_count, int32_t max_blocks, int32_t batch,
                        const csa_tensor* out, void* stream) {
  csa::CompressArgs a;
  const csa_status st = compress_args(raw, raw_base, logits, m, dim, block_first, block_count, max_blocks, batch,
                                      out, &a);
  if (st != CSA_OK) return st;
  return from_hip(csa::launch_compress(a, (hipStream_t)stream), "csa_compress launch");
}

csa_status csa_compress_jobs(const csa_compress_job* jobs, int32_t n_jobs, void* stream) {
  REQUIRE(n_jobs >= 0 && n_jobs <= CSA_MAX_COMPRESS_JOBS, CSA_ERR_SHAPE, "n_jobs=%d outside [0, %d]", n_jobs,
          CSA_MAX_COMPRESS_JOBS);
  REQUIRE(jobs || n_jobs == 0, CSA_ERR_NULL, "jobs is NULL");
  static_assert(CSA_MAX_COMPRESS_JOBS == csa::kMaxCompressJobs, "one job limit");
  csa::CompressArgs a[CSA_MAX_COMPRESS_JOBS];
  for (int j = 0; j < n_jobs; ++j) {
    const csa_compress_job& J = jobs[j];
    const csa_status st = compress_args(&J.raw, J.raw_base, J.logits, J.m, J.dim, J.block_first, J.block_count,
                                        J.max_blocks, J.batch, &J.out, &a[j]);
    if (st != CSA_OK) {
      g_last_error = "job " + std::to_string(j) + ": " + g_last_error;
      return st;
    }
  }
  return from_hip(csa::launch_compress_jobs(a, n_jobs, (hipStream_t)stream), "csa_compress_jobs launch");
}

// Validates the indexer arguments and fills the launch description.
static csa_status index_args(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx, const int32_t* q_pos,
                             int32_t batch, int32_t tq, int32_t n_idx_heads, int32_t idx_dim, int32_t m,
                             int32_t n_cap, float* scores, csa::IndexArgs* out, bool scores_required = true) {
  csa_status st;
  if ((st = check_tensor(q_idx, "q_idx")) != CSA_OK) return st;
  if ((st = check_tensor(k_idx, "k_idx")) != CSA_OK) return st;
  REQUIRE(w && q_pos, CSA_ERR_NULL, "w/q_pos is NULL");
  REQUIRE(scores || !scores_required, CSA_ERR_NULL, "scores is NULL");
  REQUIRE(batch >= 0 && tq >= 0 && n_cap >= 0, CSA_ERR_SHAPE, "negative batch, tq or n_cap");
  REQUIRE(n_idx_heads >= 1 && idx_dim >= 1 && m >= 1, CSA_ERR_SHAPE, "n_idx_heads, idx_dim and m must be >= 1");
  const int kd = k_idx->dtype, qd = q_idx->dtype;
  if (kd == CSA_MXFP4) {
    REQUIRE(qd == CSA_F32, CSA_ERR_DTYPE, "MXFP4 keys take an F32 query (quantised inside)");
    REQUIRE(idx_dim == 64 && n_idx_heads <= 32, CSA_ERR_UNSUPPORTED,
            "MXFP4 indexer supports idx_dim == 64 and n_idx_heads <= 32 (got %d, %d)", idx_dim, n_idx_heads);
  } else if (kd == CSA_BF16) {
    REQUIRE(qd == CSA_F32 || qd == CSA_BF16, CSA_ERR_DTYPE, "BF16 keys take an F32 or BF16 query");
  } else if (kd == CSA_F32) {
    REQUIRE(qd == CSA_F32, CSA_ERR_DTYPE, "F32 keys take an F32 query");
  } else {
    return fail(CSA_ERR_UNSUPPORTED, "FP8 indexer keys are not supported");
  }
  if (kd != CSA_MXFP4 && !(kd == CSA_BF16 && qd == CSA_BF16 && n_idx_heads == 8 && idx_dim == 64))
    REQUIRE((int64_t)n_idx_heads * idx_dim <= 8192, CSA_ERR_UNSUPPORTED, "n_idx_heads * idx_dim > 8192");
  csa::IndexArgs& a = *out;
  a.q = csa::view_of(q_idx);
  a.w = w;
  a.k = csa::view_of(k_idx);
  a.q_pos = q_pos;
  a.batch = batch;
  a.tq = tq;
  a.heads = n_idx_heads;
  a.dim = idx_dim;
  a.m = m;
  a.n_cap = n_cap;
  a.scores = scores;
  return CSA_OK;
}

csa_status csa_index_scores(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx, const int32_t* q_pos,
                            int32_t batch, int32_t tq, int32_t n_idx_heads, int32_t idx_dim, int32_t m, int32_t n_cap,
                            float* scores, void* stream) {
  csa::IndexArgs a;
  const csa_status st = index_args(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, scores, &a);
  if (st != CSA_OK) return st;
  return from_hip(csa::launch_index_scores(a, (hipStream_t)stream), "csa_index_scores launch");
}

size_t csa_topk_workspace_size(int32_t batch, int32_t tq, int32_t n_cap, int32_t k) {
  if (batch < 0 || tq < 0 || n_cap < 0 || k < 1) return 0;
  return csa::topk_workspace_bytes((int64_t)batch * tq, n_cap, k);
}

csa_status csa_topk(const float* scores, const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_cap, int32_t m,
                    int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(scores && q_pos && idx, CSA_ERR_NULL, "scores/q_pos/idx is NULL");
  REQUIRE(batch >= 0 && tq >= 0 && n_cap >= 0, CSA_ERR_SHAPE, "negative batch, tq or n_cap");
  REQUIRE(k >= 1 && m >= 1, CSA_ERR_SHAPE, "k and m must be >= 1");
  const size_t need = csa::topk_workspace_bytes((int64_t)batch * tq, n_cap, k);
  if (need > 0) REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "top-k needs %zu workspace bytes, got %zu", need, ws_bytes);
  return from_hip(csa::launch_topk(scores, q_pos, batch, tq, n_cap, m, k, idx, ws, (hipStream_t)stream),
                  "csa_topk launch");
}

size_t csa_index_topk_workspace_size(int32_t batch, int32_t tq, int32_t n_cap, int32_t k, int32_t scores_kept) {
  if (batch < 0 || tq < 0 || n_cap < 0 || k < 1) return 0;
  return csa::index_topk_workspace_bytes((int64_t)batch * tq, n_cap, k, scores_kept == 0);
}

// Checks the index+top-k arguments shared by the part-wise and combined calls.
static csa_status index_topk_args(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                                  const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads,
                                  int32_t idx_dim, int32_t m, int32_t n_cap, int32_t k, float* scores, int32_t* idx,
                                  void* ws, size_t ws_bytes, int32_t part, csa::IndexArgs* a) {
  const csa_status st = index_args(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, scores, a, false);
  if (st != CSA_OK) return st;
  REQUIRE(part >= 1 && part <= 3, CSA_ERR_SHAPE, "part=%d must be 1 (scores), 2 (selection) or 3 (both)", part);
  REQUIRE(idx != nullptr || !(part & 2), CSA_ERR_NULL, "idx is NULL");
  REQUIRE(k >= 1, CSA_ERR_SHAPE, "k=%d must be >= 1", k);
  const size_t need = csa_index_topk_workspace_size(batch, tq, n_cap, k, scores != nullptr);
  if (need > 0)
    REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "index+top-k needs %zu workspace bytes, got %zu",
            need, ws_bytes);
  // Without a caller buffer the two-stage path keeps its scores in the workspace; the
  // fused path writes none (short rows excepted, which it keeps there itself).
  if (scores == nullptr && !csa::index_topk_fused_ok(*a, k))
    a->scores = (float*)((char*)ws + csa::index_topk_score_offset((int64_t)batch * tq, n_cap, k));
  return CSA_OK;
}

csa_status csa_index_topk_part(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                               const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads, int32_t idx_dim,
                               int32_t m, int32_t n_cap, int32_t k, float* scores, int32_t* idx, void* ws,
                               size_t ws_bytes, int32_t part, void* stream) {
  csa::IndexArgs a;
  csa_status st = index_topk_args(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx,
                                  ws, ws_bytes, part, &a);
  if (st != CSA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const bool fused = csa::index_topk_fused_ok(a, k);
  if (part & 1) {
    st = fused ? from_hip(csa::launch_index_topk_cand(a, k, ws, s), "csa_index_topk scores launch")
               : from_hip(csa::launch_index_scores(a, s), "csa_index_topk scores launch");
    if (st != CSA_OK) return st;
  }
  if (part & 2)
    return fused ? from_hip(csa::launch_index_topk_merge(a, k, idx, ws, s), "csa_index_topk selection launch")
                 : from_hip(csa::launch_topk(a.scores, q_pos, batch, tq, n_cap, m, k, idx, ws, s),
                            "csa_index_topk selection launch");
  return ok();
}

// A job the indexer launch can run: its raw-row format code (0 F32, 1 BF16, 2 FP8).
static int raw_format(const csa::CompressArgs& c) {
  return c.raw.dtype == CSA_F32 ? 0 : c.raw.dtype == CSA_BF16 ? 1 : 2;
}

csa_status csa_compress_index_topk(const csa_compress_job* kv_job, const csa_compress_job* key_job,
                                   const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx,
                                   const int32_t* q_pos, int32_t batch, int32_t tq, int32_t n_idx_heads,
                                   int32_t idx_dim, int32_t m, int32_t n_cap, int32_t k, float* scores, int32_t* idx,
                                   void* ws, size_t ws_bytes, int32_t part, void* stream) {
  // every argument is validated before anything is launched
  csa::CompressArgs jobs[2];
  int n_jobs = 0;
  for (const csa_compress_job* J : {kv_job, key_job}) {
    if (!J) continue;
    const csa_status st = compress_args(&J->raw, J->raw_base, J->logits, J->m, J->dim, J->block_first,
                                        J->block_count, J->max_blocks, J->batch, &J->out, &jobs[n_jobs]);
    if (st != CSA_OK) {
      g_last_error = std::string(J == kv_job ? "kv_job: " : "key_job: ") + g_last_error;
      return st;
    }
    ++n_jobs;
  }
  csa::IndexArgs a;
  csa_status st = index_topk_args(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx,
                                  ws, ws_bytes, part, &a);
  if (st != CSA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  // The compressions run inside the indexer launch when it scores MXFP4 keys with slice
  // candidates for single-query rows, the key job writes exactly the keys being scored
  // and its blocks are small; otherwise they run first, on their own.
  const csa::CompressArgs* kvc = kv_job ? &jobs[0] : nullptr;
  const csa::CompressArgs* kyc = key_job ? &jobs[kv_job ? 1 : 0] : nullptr;
  bool in_launch = (part & 1) && csa::index_topk_fused_ok(a, k) && tq == 1;
  if (in_launch && kyc)
    in_launch = kyc->out_dtype == CSA_MXFP4 && kyc->out == a.k.data && kyc->out_scale == a.k.scale &&
                kyc->out_sb == a.k.sb && kyc->out_sr == a.k.sr && kyc->out_ssb == a.k.ssb &&
                kyc->out_ssr == a.k.ssr && kyc->dim == idx_dim && idx_dim == 64 &&
                kyc->m <= csa::kFusedCompressMaxM && kyc->max_blocks <= csa::kFusedCompressMaxNew &&
                kyc->batch == batch;
  if (in_launch && kvc) in_launch = kvc->m <= 16 && kvc->dim <= 512 && kvc->batch <= batch;
  if (!in_launch) {
    if ((part & 1) && n_jobs > 0) {
      st = from_hip(csa::launch_compress_jobs(jobs, n_jobs, s), "csa_compress_index_topk compression launch");
      if (st != CSA_OK) return st;
    }
    return csa_index_topk_part(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx, ws,
                               ws_bytes, part, stream);
  }
  csa::FusedCompress fc{};
  if (kyc) {
    fc.key = *kyc;
    fc.key_in = raw_format(*kyc);
  }
  if (kvc && kvc->max_blocks > 0) {
    fc.kv = *kvc;
    fc.kv_in = raw_format(*kvc);
  }
  st = from_hip(csa::launch_index_topk_cand(a, k, ws, s, &fc), "csa_compress_index_topk scores launch");
  if (st != CSA_OK) return st;
  if (part & 2)
    return from_hip(csa::launch_index_topk_merge(a, k, idx, ws, s), "csa_compress_index_topk selection launch");
  return ok();
}

csa_status csa_index_topk(const csa_tensor* q_idx, const float* w, const csa_tensor* k_idx, const int32_t* q_pos,
                          int32_t batch, int32_t tq, int32_t n_idx_heads, int32_t idx_dim, int32_t m, int32_t n_cap,
                          int32_t k, float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return csa_index_topk_part(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx, ws,
                             ws_bytes, 3, stream);
}

static bool proj_shape_ok(int32_t batch, int32_t tq, int32_t d_model, int32_t rank, int32_t n_idx_heads,
                          int32_t idx_dim) {
  return batch >= 0 && tq >= 0 && d_model >= 32 && d_model <= 65536 && d_model % 32 == 0 && rank >= 32 &&
         rank <= 65536 && rank % 32 == 0 && n_idx_heads >= 1 && idx_dim >= 1 &&
         (int64_t)n_idx_heads * idx_dim <= 65536;
}

size_t csa_index_query_workspace_size(int32_t batch, int32_t tq, int32_t d_model, int32_t rank,
                                      int32_t n_idx_heads, int32_t idx_dim) {
  if (!proj_shape_ok(batch, tq, d_model, rank, n_idx_heads, idx_dim)) return 0;
  return csa::index_query_workspace_bytes((int64_t)batch * tq, d_model, rank, n_idx_heads, idx_dim);
}

csa_status csa_index_query(const csa_tensor* h, const csa_tensor* w_dq, const csa_tensor* w_uq,
                           const csa_tensor* w_w, int32_t batch, int32_t tq, int32_t d_model, int32_t rank,
                           int32_t n_idx_heads, int32_t idx_dim, const csa_tensor* q_idx, float* w, void* ws,
                           size_t ws_bytes, void* stream) {
  csa_status st;
  if ((st = check_tensor(h, "h")) != CSA_OK) return st;
  if ((st = check_tensor(w_dq, "w_dq")) != CSA_OK) return st;
  if ((st = check_tensor(w_uq, "w_uq")) != CSA_OK) return st;
  if ((st = check_tensor(w_w, "w_w")) != CSA_OK) return st;
  if ((st = check_tensor(q_idx, "q_idx")) != CSA_OK) return st;
  REQUIRE(w != nullptr, CSA_ERR_NULL, "w is NULL");
  REQUIRE(h->dtype == CSA_BF16 && w_dq->dtype == CSA_BF16 && w_uq->dtype == CSA_BF16 && w_w->dtype == CSA_BF16,
          CSA_ERR_DTYPE, "h and the projection weights must be BF16");
  REQUIRE(q_idx->dtype == CSA_F32 || q_idx->dtype == CSA_BF16, CSA_ERR_DTYPE, "q_idx must be F32 or BF16");
  REQUIRE(proj_shape_ok(batch, tq, d_model, rank, n_idx_heads, idx_dim), CSA_ERR_SHAPE,
          "need batch, tq >= 0, d_model and rank multiples of 32 in [32, 65536], n_idx_heads * idx_dim in "
          "[1, 65536] (got d_model=%d rank=%d heads=%d dim=%d)", d_model, rank, n_idx_heads, idx_dim);
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  REQUIRE(aligned(h->data) && aligned(w_dq->data) && aligned(w_uq->data) && aligned(w_w->data), CSA_ERR_SHAPE,
          "h and the weights must be 16-byte aligned");
  REQUIRE(h->stride_b % 8 == 0 && h->stride_row % 8 == 0 && w_dq->stride_row % 8 == 0 &&
              w_uq->stride_row % 8 == 0 && w_w->stride_row % 8 == 0,
          CSA_ERR_SHAPE, "row pitches of h and the weights must be multiples of 8 elements");
  REQUIRE(w_dq->stride_row >= d_model && w_w->stride_row >= d_model && w_uq->stride_row >= rank, CSA_ERR_SHAPE,
          "a weight's row pitch is shorter than its row");
  REQUIRE(tq <= 1 || h->stride_row >= d_model, CSA_ERR_SHAPE, "h's row pitch is shorter than d_model");
  const size_t need = csa::index_query_workspace_bytes((int64_t)batch * tq, d_model, rank, n_idx_heads, idx_dim);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "csa_index_query needs %zu workspace bytes, got %zu",
          need, ws_bytes);
  csa::IndexQueryArgs a{};
  a.h = h->data;
  a.h_sb = h->stride_b;
  a.h_sr = h->stride_row;
  a.w_dq = w_dq->data;
  a.w_uq = w_uq->data;
  a.w_w = w_w->data;
  a.ld_dq = w_dq->stride_row;
  a.ld_uq = w_uq->stride_row;
  a.ld_w = w_w->stride_row;
  a.batch = batch;
  a.tq = tq;
  a.d_model = d_model;
  a.rank = rank;
  a.n_idx_heads = n_idx_heads;
  a.idx_dim = idx_dim;
  a.q_out = q_idx->data;
  a.q_sb = q_idx->stride_b;
  a.q_sr = q_idx->stride_row;
  a.q_bf16 = q_idx->dtype == CSA_BF16;
  a.w_out = w;
  a.ws = ws;
  return from_hip(csa::launch_index_query(a, (hipStream_t)stream), "csa_index_query launch");
}

static bool latent_shape_ok(int32_t rows, int32_t heads, int32_t head_dim, int32_t dim) {
  const auto dim_ok = [](int32_t x) { return x >= 32 && x <= 65536 && x % 32 == 0; };
  return rows >= 0 && rows <= (1 << 20) && heads >= 1 && heads <= 65535 && dim_ok(head_dim) && dim_ok(dim);
}

size_t csa_latent_query_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t dim) {
  if (!latent_shape_ok(rows, heads, head_dim, dim)) return 0;
  return csa::latent_proj_workspace_bytes(rows, heads, head_dim, dim);
}

size_t csa_latent_output_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t dim) {
  if (!latent_shape_ok(rows, heads, head_dim, dim)) return 0;
  return csa::latent_proj_workspace_bytes(rows, heads, dim, head_dim);
}

static csa_status latent_common(const char* name, const void* x, const void* w, int32_t rows, int32_t heads,
                                int32_t head_dim, int32_t dim, const void* y, void* ws, size_t ws_bytes, size_t need) {
  REQUIRE(x && w && y, CSA_ERR_NULL, "%s: an input, weight or output pointer is NULL", name);
  REQUIRE(latent_shape_ok(rows, heads, head_dim, dim), CSA_ERR_SHAPE,
          "%s: need 0 <= rows <= 1048576, heads in [1, 65535], head_dim and dim multiples of 32 in [32, 65536] "
          "(got rows=%d heads=%d head_dim=%d dim=%d)", name, rows, heads, head_dim, dim);
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  REQUIRE(aligned(x) && aligned(w), CSA_ERR_SHAPE, "%s: input and weights must be 16-byte aligned", name);
  REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need,
          ws_bytes);
  return CSA_OK;
}

csa_status csa_latent_query(const void* q, const void* w_uk_t, int32_t rows, int32_t heads, int32_t head_dim,
                            int32_t dim, void* q_lat, void* ws, size_t ws_bytes, void* stream) {
  const size_t need = latent_shape_ok(rows, heads, head_dim, dim)
                          ? csa::latent_proj_workspace_bytes(rows, heads, head_dim, dim) : 0;
  csa_status st = latent_common("csa_latent_query", q, w_uk_t, rows, heads, head_dim, dim, q_lat, ws, ws_bytes, need);
  if (st != CSA_OK) return st;
  const csa::LatentProjArgs a{q, 0, w_uk_t, rows, heads, head_dim, dim, q_lat, 1, ws};
  return from_hip(csa::launch_latent_proj(a, (hipStream_t)stream), "csa_latent_query launch");
}

csa_status csa_latent_output(const float* o_lat, const void* w_uv, int32_t rows, int32_t heads, int32_t head_dim,
                             int32_t dim, void* out, csa_dtype out_dtype, void* ws, size_t ws_bytes, void* stream) {
  const size_t need = latent_shape_ok(rows, heads, head_dim, dim)
                          ? csa::latent_proj_workspace_bytes(rows, heads, dim, head_dim) : 0;
  csa_status st = latent_common("csa_latent_output", o_lat, w_uv, rows, heads, head_dim, dim, out, ws, ws_bytes, need);
  if (st != CSA_OK) return st;
  REQUIRE(out_dtype == CSA_F32 || out_dtype == CSA_BF16, CSA_ERR_DTYPE, "csa_latent_output: out must be F32 or BF16");
  const csa::LatentProjArgs a{o_lat, 1, w_uv, rows, heads, dim, head_dim, out, out_dtype == CSA_BF16, ws};
  return from_hip(csa::launch_latent_proj(a, (hipStream_t)stream), "csa_latent_output launch");
}

size_t csa_attn_workspace_size(int32_t batch, int32_t tq, int32_t heads, int32_t dim, int32_t n_entries_max) {
  if (batch < 0 || tq < 0 || heads < 1 || dim < 1 || n_entries_max < 0) return 0;
  return csa::attn_workspace_bytes((int64_t)batch * tq, heads, dim, n_entries_max, tq);
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free attention
// The split partials of csa_sparse_attn_noalloc live in this file-scope device array
// (one copy per device, held until the process ends).  Host code never passes the
// array's name to a kernel: its device address is looked up once per device with
// that device current and kept in g_scratch_ptr.
namespace {
constexpr size_t kNoAllocScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];

csa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  REQUIRE(dev >= 0 && dev < kNoAllocMaxDevices, CSA_ERR_UNSUPPORTED,
          "device %d: the allocation-free entry point serves devices 0..%d", dev, kNoAllocMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    REQUIRE(p != nullptr, CSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}
}  // namespace

extern "C" {

static csa_status attn_common(const csa_tensor* q, const csa_tensor* kv, const int32_t* idx, int32_t k, int32_t m_hc,
                              int32_t n_cap_hc, const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window,
                              const int32_t* q_pos, int32_t batch, int32_t tq, int32_t heads, int32_t dim, float scale,
                              float* out, float* lse, void* ws, size_t ws_bytes, void* stream, int n_entries_max,
                              bool use_scratch = false) {
  csa_status st;
  if ((st = check_tensor(q, "q")) != CSA_OK) return st;
  if ((st = check_tensor(kv, "kv")) != CSA_OK) return st;
  if ((st = check_tensor(kv_raw, "kv_raw")) != CSA_OK) return st;
  REQUIRE(raw_base && q_pos && out, CSA_ERR_NULL, "raw_base/q_pos/out is NULL");
  REQUIRE(batch >= 0 && tq >= 0 && window >= 0, CSA_ERR_SHAPE, "negative batch, tq or window");
  REQUIRE(heads >= 1 && dim >= 1, CSA_ERR_SHAPE, "heads and dim must be >= 1");
  REQUIRE(kv->dtype == kv_raw->dtype || (kv->dtype == CSA_MXFP4 && kv_raw->dtype == CSA_BF16), CSA_ERR_DTYPE,
          "compressed and raw rows must share a dtype (MXFP4 compressed rows take BF16 raw rows)");
  REQUIRE(kv_raw->dtype != CSA_MXFP4, CSA_ERR_DTYPE, "raw rows are F32, BF16 or FP8_E4M3 (MXFP4 compressed rows "
          "take BF16 raw rows)");
  if (kv->dtype == CSA_F32) {
    REQUIRE(q->dtype == CSA_F32, CSA_ERR_DTYPE, "F32 caches take an F32 query");
    REQUIRE(dim <= 512 && dim % 4 == 0 && heads <= 64, CSA_ERR_UNSUPPORTED,
            "F32 attention supports dim <= 512 (multiple of 4) and heads <= 64");
    REQUIRE(csa::attn_plain_fits(n_entries_max), CSA_ERR_UNSUPPORTED, "F32 attention supports at most 8192 entries per query");
  } else if (kv->dtype == CSA_BF16 || kv->dtype == CSA_FP8_E4M3 || kv->dtype == CSA_MXFP4) {
    REQUIRE(q->dtype == CSA_BF16, CSA_ERR_DTYPE, "BF16/FP8/MXFP4 caches take a BF16 query");
    REQUIRE(dim == 512 && heads % 16 == 0 && heads <= 64, CSA_ERR_UNSUPPORTED,
            "BF16/FP8/MXFP4 attention supports dim == 512 and heads a multiple of 16 up to 64 (got %d, %d)", dim,
            heads);
    // rows are read 16 (BF16), 8 (FP8) or 4 (MXFP4) bytes per lane; the query 16 bytes per lane
    const int64_t align = kv->dtype == CSA_BF16 ? 16 : kv->dtype == CSA_FP8_E4M3 ? 8 : 4;
    const int64_t esz = kv->dtype == CSA_BF16 ? 2 : 1;  // stride units in bytes (MXFP4 strides are bytes)
    const auto rows_aligned = [](const csa_tensor* t, int64_t al, int64_t es) {
      return (uintptr_t)t->data % al == 0 && (t->stride_b * es) % al == 0 && (t->stride_row * es) % al == 0;
    };
    const bool raw_bf16 = kv_raw->dtype == CSA_BF16;
    REQUIRE(rows_aligned(kv, align, esz) && rows_aligned(kv_raw, raw_bf16 ? 16 : align, raw_bf16 ? 2 : esz),
            CSA_ERR_SHAPE, "cache rows must start on %lld-byte boundaries (data and strides; BF16 rows 16)",
            (long long)align);
    REQUIRE((uintptr_t)q->data % 16 == 0 && q->stride_b % 8 == 0 && q->stride_row % 8 == 0, CSA_ERR_SHAPE,
            "q must be 16-byte aligned with strides a multiple of 8 elements");
    const int split = csa::attn_split_size(tq, n_entries_max, false);  // CSA cuts at least as many as HCA
    const int64_t nsplit = ((int64_t)std::max(n_entries_max, 1) + split - 1) / split;
    REQUIRE(nsplit <= csa::kAttnMaxSplits, CSA_ERR_UNSUPPORTED,
            "BF16/FP8/MXFP4 attention supports at most %d entries per query (got %d)",
            csa::kAttnMaxSplits * csa::kAttnMaxSplitEntries, n_entries_max);
  } else {
    return fail(CSA_ERR_DTYPE, "attention caches must be F32, BF16, FP8_E4M3 or MXFP4");
  }
  const size_t need = csa::attn_workspace_bytes((int64_t)batch * tq, heads, dim, n_entries_max, tq);
  if (need > 0 && !use_scratch)
    REQUIRE(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (use_scratch) {  // the allocation-free entry point, after every other check
    REQUIRE(need <= kNoAllocScratchBytes, CSA_ERR_WORKSPACE,
            "attention needs %zu scratch bytes; csa_sparse_attn_noalloc holds at most %zu (use csa_sparse_attn with a "
            "workspace)", need, kNoAllocScratchBytes);
    ws = nullptr;
    if (need > 0) {
      const csa_status sst = scratch_address(&ws);
      if (sst != CSA_OK) return sst;
    }
  }
  csa::AttnArgs a;
  a.q = csa::view_of(q);
  a.kv = csa::view_of(kv);
  a.idx = idx;
  a.k = k;
  a.m_hc = m_hc;
  a.n_cap = n_cap_hc;
  a.raw = csa::view_of(kv_raw);
  a.raw_base = raw_base;
  a.window = window;
  a.q_pos = q_pos;
  a.batch = batch;
  a.tq = tq;
  a.heads = heads;
  a.dim = dim;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  return from_hip(csa::launch_attention(a, n_entries_max, (hipStream_t)stream), "attention launch");
}

csa_status csa_sparse_attn(const csa_tensor* q, const csa_tensor* kv_cmp, const int32_t* idx, int32_t k,
                           const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window, const int32_t* q_pos,
                           int32_t batch, int32_t tq, int32_t heads, int32_t dim, float scale, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(idx != nullptr, CSA_ERR_NULL, "idx is NULL");
  REQUIRE(k >= 0, CSA_ERR_SHAPE, "k=%d must be >= 0", k);
  REQUIRE((int64_t)k + window <= (1 << 30), CSA_ERR_SHAPE, "k + window too large");
  return attn_common(q, kv_cmp, idx, k, 0, 0, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim, scale, out, lse,
                     ws, ws_bytes, stream, k + window);
}

csa_status csa_sparse_attn_noalloc(const csa_tensor* q, const csa_tensor* kv_cmp, const int32_t* idx, int32_t k,
                                   const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window,
                                   const int32_t* q_pos, int32_t batch, int32_t tq, int32_t heads, int32_t dim,
                                   float scale, float* out, float* lse, void* stream) {
  REQUIRE(idx != nullptr, CSA_ERR_NULL, "idx is NULL");
  REQUIRE(k >= 0, CSA_ERR_SHAPE, "k=%d must be >= 0", k);
  REQUIRE((int64_t)k + window <= (1 << 30), CSA_ERR_SHAPE, "k + window too large");
  return attn_common(q, kv_cmp, idx, k, 0, 0, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim, scale, out, lse,
                     nullptr, 0, stream, k + window, /*use_scratch=*/true);
}

csa_status hca_attn(const csa_tensor* q, const csa_tensor* kv_hc, int32_t m_hc, int32_t n_cap_hc,
                    const csa_tensor* kv_raw, const int32_t* raw_base, int32_t window, const int32_t* q_pos,
                    int32_t batch, int32_t tq, int32_t heads, int32_t dim, float scale, float* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(m_hc >= 1 && n_cap_hc >= 0, CSA_ERR_SHAPE, "m_hc must be >= 1 and n_cap_hc >= 0");
  REQUIRE((int64_t)n_cap_hc + window <= (1 << 30), CSA_ERR_SHAPE, "n_cap_hc + window too large");
  return attn_common(q, kv_hc, nullptr, 0, m_hc, n_cap_hc, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim,
                     scale, out, lse, ws, ws_bytes, stream, n_cap_hc + window);
}

csa_status csa_quantize_mxfp4(const float* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream) {
  REQUIRE(x && codes && scales, CSA_ERR_NULL, "x/codes/scales is NULL");
  REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, CSA_ERR_SHAPE, "cols must be a non-negative multiple of 32");
  return from_hip(csa::launch_quantize_mxfp4(x, rows, cols, codes, scales, (hipStream_t)stream), "csa_quantize_mxfp4");
}

csa_status csa_quantize_fp8(const float* x, int64_t rows, int32_t cols, uint8_t* codes, float* row_scale,
                            void* stream) {
  REQUIRE(x && codes && row_scale, CSA_ERR_NULL, "x/codes/row_scale is NULL");
  REQUIRE(rows >= 0 && cols >= 1 && cols <= 8192, CSA_ERR_SHAPE, "cols must be in [1, 8192]");
  return from_hip(csa::launch_quantize_fp8(x, rows, cols, codes, row_scale, (hipStream_t)stream), "csa_quantize_fp8");
}

size_t csa_stream_read_sink_size(void) { return (size_t)csa::kStreamReadBlocks * sizeof(uint32_t); }

csa_status csa_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  REQUIRE(data && sink, CSA_ERR_NULL, "data/sink is NULL");
  REQUIRE(bytes % 16 == 0, CSA_ERR_SHAPE, "bytes must be a multiple of 16");
  return from_hip(csa::launch_stream_read(data, bytes, sink, (hipStream_t)stream), "csa_stream_read launch");
}

}  // extern "C"

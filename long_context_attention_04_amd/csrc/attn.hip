// (d) CSA sparse attention and (e) HCA dense attention.
//
// Both attend over compressed entries plus a sliding window of raw local
// entries (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations
// 1: CSA bullet for the top-k compressed blocks, HCA bullet for dense
// attention over the heavily compressed entries and the window).  Readings:
// key = value = the stored (shared, MQA) row; one softmax over the compressed
// entries followed by the window rows, not de-duplicated.
//
// MFMA path (bf16 / fp8 caches, 16..64 heads, dim 512).  Decode attention of
// 64 query heads against a shared 512-wide latent is a [64 x 512] x [512 x n]
// contraction, so QK and PV both run on bf16 MFMA 16x16x32.  A workgroup
// (4 waves) handles one query row and one contiguous split of its entry list.
// Wave w owns latent columns [128w, 128w+128): it loads exactly that slice of
// every entry row from HBM (16 B per lane, the MFMA B-operand layout), uses it
// for its partial QK and stages it in LDS for PV, so every entry byte is read
// from HBM once.  The four partial logit tiles are summed in a fixed order in
// LDS and all 256 threads run the online softmax.  The probabilities go to
// PV as two bf16 terms (hi + lo), so PV carries ~16 significant bits of P
// instead of bf16's 8; PV reads the staged slice transposed with
// ds_read_b64_tr_b16.  Splits are merged by a second
// kernel with a fixed-order log-sum-exp combine; the split size depends only
// on the call shape, never on the batch, so results are batch-invariant.
// fp8 rows keep their per-row scale out of the MFMA: it multiplies the logit
// and the probability used for PV.
//
// Plain path (fp32 caches): a straightforward fp32 VALU kernel, one workgroup
// per (query, head).
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kThreads = 256;
constexpr int kTileE = 32;
constexpr int kSplitDecode = 128;
constexpr int kEsStride = 136;  // bf16 elements per staged row (128 + 8 pad)
constexpr int kPsStride = 40;   // bf16 elements per P row (32 + 8 pad)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowInfo {
  int b, t, pos, w0, n_cmp, n_tot;
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int row) {
  RowInfo r;
  r.b = row / a.tq;
  r.t = row % a.tq;
  r.pos = a.q_pos[row];
  r.w0 = max(0, r.pos - a.window + 1);
  const int n_win = a.window > 0 ? r.pos - r.w0 + 1 : 0;
  r.n_cmp = a.idx ? a.k : visible_blocks(r.pos, a.m_hc);
  r.n_tot = r.n_cmp + n_win;
  return r;
}

__device__ __forceinline__ int elem_bytes(int dtype) { return dtype == CSA_F32 ? 4 : dtype == CSA_BF16 ? 2 : 1; }

// Byte pointer to entry e of a row's list (nullptr when the slot is empty) and its row scale.
// `jl` (optional) holds the compressed indices of entries [jl_base, jl_base + kMaxSplit).
__device__ __forceinline__ const uint8_t* entry_ptr(const AttnArgs& a, const RowInfo& r, int row, int e, float* sc,
                                                    const int* jl = nullptr, int jl_base = 0) {
  *sc = 1.f;
  if (e >= r.n_tot) return nullptr;
  if (e < r.n_cmp) {
    const int j = a.idx ? (jl ? jl[e - jl_base] : a.idx[(int64_t)row * a.k + e]) : e;
    if (j < 0) return nullptr;
    if (a.kv.dtype == CSA_FP8_E4M3 && a.kv.scale) *sc = ((const float*)a.kv.scale)[(int64_t)r.b * a.kv.ssb + (int64_t)j * a.kv.ssr];
    return (const uint8_t*)a.kv.data + ((int64_t)r.b * a.kv.sb + (int64_t)j * a.kv.sr) * elem_bytes(a.kv.dtype);
  }
  const int64_t rr = (int64_t)(r.w0 + (e - r.n_cmp)) - a.raw_base[r.b];
  if (a.raw.dtype == CSA_FP8_E4M3 && a.raw.scale) *sc = ((const float*)a.raw.scale)[(int64_t)r.b * a.raw.ssb + rr * a.raw.ssr];
  return (const uint8_t*)a.raw.data + ((int64_t)r.b * a.raw.sb + rr * a.raw.sr) * elem_bytes(a.raw.dtype);
}

template <bool FP8>
__device__ __forceinline__ v8bf load8(const uint8_t* p, int col) {
  v8bf v;
  if (!p) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.f;
    return v;
  }
  if constexpr (!FP8) {
    return *(const v8bf*)(p + 2 * col);
  } else {
    const uint2 c = *(const uint2*)(p + col);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = ((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xffu;
      v[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(e4m3_to_f32(byte)) >> 16));  // exact
    }
    return v;
  }
}

// Workgroup -> (row, split, head group).  Consecutive workgroup ids go to
// different XCDs (round robin over 8), so the nhg head groups of one
// (row, split) get ids 8 apart: same XCD, same L2, run side by side, and the
// entry rows the first one fetches from HBM are L2 hits for the others.
__device__ __forceinline__ void decode_block(int id, int nhg, int nsplit_max, int* row, int* split, int* hg) {
  *hg = (id / 8) % nhg;
  const int c = (id / (8 * nhg)) * 8 + id % 8;  // (row, split) pair
  *row = c / nsplit_max;
  *split = c % nsplit_max;
}

template <int NHT, bool FP8>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(AttnArgs a, int split, int nsplit_max, int nhg,
                                                             int partial, int64_t rows) {
  constexpr int HW = 16 * NHT;       // heads in this workgroup
  constexpr int TPH = 16 / NHT;      // softmax threads per head
  constexpr int EPT = kTileE / TPH;  // entries per softmax thread
  int row, s, hg;
  decode_block(blockIdx.x, nhg, nsplit_max, &row, &s, &hg);
  if (row >= rows) return;
  const RowInfo ri = row_info(a, row);
  const int nsplit = max(1, (ri.n_tot + split - 1) / split);
  if (s >= nsplit) return;
  const int e_begin = s * split, e_end = min(ri.n_tot, e_begin + split);
  const int h0 = hg * HW;  // first head of this workgroup

  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = lane / 16, n = lane % 16;

  __shared__ float red[4][HW][kTileE];
  __shared__ __attribute__((aligned(16))) uint16_t Es[4][kTileE][kEsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[2][HW][kPsStride];  // P = hi + lo, both bf16
  __shared__ float al[HW];
  __shared__ float ev_scale[2][kTileE];  // per tile parity; 0 marks an empty slot
  __shared__ float fin_m[HW], fin_l[HW];
  __shared__ int jl[kSplitDecode];  // this split's compressed indices (decode splits)
  const bool use_jl = a.idx != nullptr && split <= kSplitDecode;
  if (use_jl) {
    const int e = e_begin + (int)threadIdx.x;
    if (threadIdx.x < kSplitDecode && e < min(e_end, ri.n_cmp)) jl[threadIdx.x] = a.idx[(int64_t)row * a.k + e];
  }
  __syncthreads();

  // q operands: head h0 + 16*ht + n, latent columns 128w + 32kk + 8g .. +7
  v8bf qa[NHT][4];
  const uint16_t* qp = (const uint16_t*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qa[ht][kk] = *(const v8bf*)(qp + (h0 + 16 * ht + n) * 512 + 128 * w + 32 * kk + 8 * g);

  const float sl2 = a.scale * kLog2e;
  // softmax role: thread -> head sh = tid / TPH, entries EPT*(tid % TPH) .. +EPT-1 of each tile
  const int sh = threadIdx.x / TPH, seb = EPT * (threadIdx.x % TPH);
  float m_run = kNegInf, l_run = 0.f;
  v4f O[NHT][8];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) O[ht][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  // software pipeline: the next tile's rows are in flight while this one is processed
  v8bf bq[2][4];
  auto load_tile = [&](int e0, int par) {
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      const int e = e0 + 16 * et + n;
      float sc;
      const uint8_t* p = e < e_end ? entry_ptr(a, ri, row, e, &sc, use_jl ? jl : nullptr, e_begin) : nullptr;
      if (w == 0 && g == 0) ev_scale[par][16 * et + n] = p ? (FP8 ? sc : 1.f) : 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bq[et][kk] = load8<FP8>(p, 128 * w + 32 * kk + 8 * g);
    }
  };
  load_tile(e_begin, 0);
  int par = 0;
  for (int e0 = e_begin; e0 < e_end; e0 += kTileE, par ^= 1) {
    // partial logits over this wave's 128 columns; stage the slice for PV
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int et = 0; et < 2; ++et) {
        v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][kk], bq[et][kk], c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) red[w][16 * ht + 4 * g + r][16 * et + n] = c[r];
      }
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) *(v8bf*)&Es[w][16 * et + n][32 * kk + 8 * g] = bq[et][kk];
    if (e0 + kTileE < e_end) load_tile(e0 + kTileE, par ^ 1);
    __syncthreads();

    {  // online softmax: every thread owns EPT entries of one head
      float sv[EPT], esc[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        esc[i] = ev_scale[par][seb + i];
        const float x = ((red[0][sh][seb + i] + red[1][sh][seb + i]) + red[2][sh][seb + i]) + red[3][sh][seb + i];
        sv[i] = esc[i] != 0.f ? x * esc[i] * sl2 : kNegInf;
      }
      float tmax = sv[0];
#pragma unroll
      for (int i = 1; i < EPT; ++i) tmax = fmaxf(tmax, sv[i]);
#pragma unroll
      for (int o = 1; o < TPH; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == kNegInf ? 1.f : exp2f(m_run - m_new);
      float psum = 0.f;
      uint16_t ph[EPT], plo[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float p = m_new == kNegInf ? 0.f : exp2f(sv[i] - m_new);
        psum += p;
        const float pv = FP8 ? p * esc[i] : p;
        ph[i] = f32_to_bf16_bits(pv);
        plo[i] = f32_to_bf16_bits(pv - bf16_bits_to_f32(ph[i]));  // exact remainder, rounded once more
      }
#pragma unroll
      for (int o = 1; o < TPH; o <<= 1) psum += __shfl_xor(psum, o);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        Ps[0][sh][seb + i] = ph[i];
        Ps[1][sh][seb + i] = plo[i];
      }
      if (threadIdx.x % TPH == 0) al[sh] = alpha;
    }
    __syncthreads();

    // O[heads, this wave's columns] = O * alpha + P[heads, 32] . E[32, columns]
    v8bf pa[NHT], pal[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      pa[ht] = *(const v8bf*)&Ps[0][16 * ht + n][8 * g];
      pal[ht] = *(const v8bf*)&Ps[1][16 * ht + n][8 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float alr = al[16 * ht + 4 * g + r];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) O[ht][ct][r] *= alr;
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      // transposed read: lane (n, g) gets column 16ct+n of staged rows 8g..8g+3 (t0) and
      // 8g+4..8g+7 (t1); the 16 lanes of a group address 4 rows x 4 column quads.
      // (The bf16 form plus a shuffle is used on purpose: extracting elements of the
      // i16 form one by one was miscompiled into reads of the first dword only.)
      typedef __attribute__((address_space(3))) v4bf lds_v4bf;
      const v4bf t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)&Es[w][8 * g + n / 4][16 * ct + 4 * (n % 4)]);
      const v4bf t1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)&Es[w][8 * g + 4 + n / 4][16 * ct + 4 * (n % 4)]);
      const v8bf vb = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        O[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ht], vb, O[ht][ct], 0, 0, 0);
        O[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal[ht], vb, O[ht][ct], 0, 0, 0);
      }
    }
  }

  if (threadIdx.x % TPH == 0) {
    fin_m[sh] = m_run;
    fin_l[sh] = l_run;
  }
  __syncthreads();
  const int H = a.heads;
  if (partial) {
    float* po = (float*)a.ws + (((int64_t)row * nsplit_max + s) * H + h0) * 512;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[(16 * ht + 4 * g + r) * 512 + 128 * w + 16 * ct + n] = O[ht][ct][r];
    float* pml = (float*)a.ws + rows * nsplit_max * H * 512 + (((int64_t)row * nsplit_max + s) * H + h0) * 2;
    if (threadIdx.x < HW) {
      pml[2 * threadIdx.x] = fin_m[threadIdx.x];
      pml[2 * threadIdx.x + 1] = fin_l[threadIdx.x];
    }
  } else {
    float* po = a.out + ((int64_t)row * H + h0) * 512;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * ht + 4 * g + r;
        const float L = fin_l[h];
        const float f = L > 0.f ? __fdiv_rn(1.0f, L) : 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) po[h * 512 + 128 * w + 16 * ct + n] = O[ht][ct][r] * f;
      }
    if (a.lse && threadIdx.x < HW) {
      const float L = fin_l[threadIdx.x];
      a.lse[(int64_t)row * H + h0 + threadIdx.x] = L > 0.f ? (fin_m[threadIdx.x] + log2f(L)) * kLn2 : kNegInf;
    }
  }
}

// Fixed-order log-sum-exp merge of the splits of one (row, head); one pass over
// the partials with every split's row in flight at once.
constexpr int kMergeMaxSplits = 64;

__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int split, int nsplit_max, int64_t rows) {
  const int row = blockIdx.x, h = blockIdx.y;
  const RowInfo ri = row_info(a, row);
  const int nsplit = min(kMergeMaxSplits, max(1, (ri.n_tot + split - 1) / split));
  const int H = a.heads;
  const float* pml = (const float*)a.ws + rows * nsplit_max * H * 512;
  __shared__ float wts[kMergeMaxSplits];
  __shared__ float sh_L, sh_M;
  if (threadIdx.x < kWave) {  // one wave forms the split weights
    const int s = threadIdx.x;
    const int64_t o = (((int64_t)row * nsplit_max + s) * H + h) * 2;
    const float ms = s < nsplit ? pml[o] : kNegInf;
    const float ls = s < nsplit ? pml[o + 1] : 0.f;
    const float M = wave_max(ms);
    const float e = (M == kNegInf || s >= nsplit) ? 0.f : exp2f(ms - M);
    // L = sum over splits in ascending order (fixed, independent of scheduling)
    float L = 0.f;
    for (int i = 0; i < nsplit; ++i) L += __shfl(ls * e, i);
    if (s < kMergeMaxSplits) wts[s] = e;
    if (s == 0) {
      sh_L = L;
      sh_M = M;
    }
  }
  __syncthreads();
  const float L = sh_L;
  const float inv = L > 0.f ? __fdiv_rn(1.0f, L) : 0.f;
  const float4* src = (const float4*)((const float*)a.ws + ((int64_t)row * nsplit_max * H + h) * 512) + threadIdx.x;
  const int64_t sstride = (int64_t)H * 512 / 4;  // float4s between consecutive splits
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = wts[s] * inv;
    const float4 v = src[s * sstride];
    acc.x = fmaf(v.x, wgt, acc.x);
    acc.y = fmaf(v.y, wgt, acc.y);
    acc.z = fmaf(v.z, wgt, acc.z);
    acc.w = fmaf(v.w, wgt, acc.w);
  }
  ((float4*)(a.out + ((int64_t)row * H + h) * 512))[threadIdx.x] = acc;
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)row * H + h] = L > 0.f ? (sh_M + log2f(L)) * kLn2 : kNegInf;
}

// ------------------------------------------------------------------ fp32 VALU path
constexpr int kPlainThreads = 128;
constexpr int kPlainMaxEntries = 8192;

__global__ __launch_bounds__(kPlainThreads) void attn_plain_kernel(AttnArgs a) {
  const int row = blockIdx.x, h = blockIdx.y;
  const RowInfo ri = row_info(a, row);
  __shared__ float logit[kPlainMaxEntries];
  __shared__ float qs[512];
  __shared__ float red[kPlainThreads / kWave];
  const int D = a.dim;
  const float* qp = (const float*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr + (int64_t)h * D;
  for (int d = threadIdx.x; d < D; d += kPlainThreads) qs[d] = qp[d];
  __syncthreads();
  float mx = kNegInf;
  for (int e = threadIdx.x; e < ri.n_tot; e += kPlainThreads) {
    float sc;
    const float* p = (const float*)entry_ptr(a, ri, row, e, &sc);
    float l = kNegInf;
    if (p) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], p[d], dot);
      l = dot * a.scale;
    }
    logit[e] = l;
    mx = fmaxf(mx, l);
  }
  mx = wave_max(mx);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float sum = 0.f;
  for (int e = threadIdx.x; e < ri.n_tot; e += kPlainThreads) {
    const float p = mx == kNegInf ? 0.f : expf(logit[e] - mx);
    logit[e] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  const float inv = sum > 0.f ? __fdiv_rn(1.0f, sum) : 0.f;
  for (int d = threadIdx.x; d < D; d += kPlainThreads) {
    float acc = 0.f;
    for (int e = 0; e < ri.n_tot; ++e) {
      float sc;
      const float* p = (const float*)entry_ptr(a, ri, row, e, &sc);
      if (p) acc = fmaf(logit[e], p[d], acc);
    }
    a.out[((int64_t)row * a.heads + h) * D + d] = acc * inv;
  }
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)row * a.heads + h] = sum > 0.f ? mx + logf(sum) : kNegInf;
}

template <int NHT>
hipError_t launch_mfma(const AttnArgs& a, int64_t rows, int split, int nsplit_max, hipStream_t s) {
  const int partial = nsplit_max > 1;
  const int nhg = a.heads / (16 * NHT);
  const int64_t pairs = rows * nsplit_max;
  const int64_t blocks = (pairs + 7) / 8 * 8 * nhg;
  if (a.kv.dtype == CSA_FP8_E4M3)
    hipLaunchKernelGGL((attn_mfma_kernel<NHT, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a, split,
                       nsplit_max, nhg, partial, rows);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<NHT, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a, split,
                       nsplit_max, nhg, partial, rows);
  if (partial)
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)rows, a.heads), dim3(128), 0, s, a, split, nsplit_max, rows);
  return hipGetLastError();
}

}  // namespace

// Splits depend only on the call shape (decode or not) and the entry capacity,
// never on the batch, so each sequence's arithmetic is batch-invariant.
int attn_split_size(int tq, int n_entries_max) {
  const int n = max(n_entries_max, 1);
  return tq == 1 ? min(kSplitDecode, (n + kTileE - 1) / kTileE * kTileE) : n;
}

size_t attn_workspace_bytes(int64_t rows, int heads, int dim, int n_entries_max, int tq) {
  const int split = attn_split_size(tq, n_entries_max);
  const int64_t nsplit = (n_entries_max + split - 1) / split;
  if (nsplit <= 1) return 0;
  return (size_t)rows * nsplit * heads * (dim + 2) * sizeof(float);
}

bool attn_plain_fits(int n_entries_max) { return n_entries_max <= kPlainMaxEntries; }

hipError_t launch_attention(const AttnArgs& a, int n_entries_max, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.tq;
  if (rows == 0) return hipSuccess;
  if (a.kv.dtype == CSA_F32) {
    hipLaunchKernelGGL(attn_plain_kernel, dim3((unsigned)rows, a.heads), dim3(kPlainThreads), 0, s, a);
    return hipGetLastError();
  }
  const int split = attn_split_size(a.tq, n_entries_max);
  const int nsplit_max = max(1, (n_entries_max + split - 1) / split);
  if (nsplit_max > kMergeMaxSplits) return hipErrorInvalidValue;
  // decode: 16 heads per workgroup (4x the workgroups, head groups share L2);
  // many queries per call: every head in one workgroup (entry rows read once)
  if (a.tq == 1) return launch_mfma<1>(a, rows, split, nsplit_max, s);
  switch (a.heads / 16) {
    case 1: return launch_mfma<1>(a, rows, split, nsplit_max, s);
    case 2: return launch_mfma<2>(a, rows, split, nsplit_max, s);
    case 3: return launch_mfma<3>(a, rows, split, nsplit_max, s);
    default: return launch_mfma<4>(a, rows, split, nsplit_max, s);
  }
}

}  // namespace csa

// (b) Lightning-indexer scores.
//
// The indexer scores compressed blocks from low-rank projections of the
// query (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1,
// CSA bullet), with the QK path in FP4 (same page, item 4, Quantization-Aware
// Training).  Reading of the score: I = sum_h w_h * relu(<q_h, kappa_j>).
//
// Three kernels, one per key format:
//  * MXFP4 keys: the key stream is the dominant HBM traffic of long-context
//    decode (34 B per key).  Each wave streams 32 keys per step straight into
//    the B operand of one scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
//    lane l carries key l%32's 32-element block l/32 (16 B of codes) and that
//    block's e8m0 scale, so the block scales are applied by the matrix core and
//    no dequantisation happens on the VALU.  Query heads are the MFMA rows
//    (quantised to MXFP4 in-kernel once per workgroup).  ReLU, head weights and
//    the cross-head sum are a short epilogue (one cross-lane add).
//  * BF16 keys: bf16 MFMA 16x16x32 with (query, head) pairs as rows, keys as
//    columns; used by decode and by prefill chunks (where it is a dense
//    contraction of many queries against the same keys).
//  * F32 keys: plain fp32 VALU kernel (small shapes).
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ fp32 VALU
constexpr int kPlainThreads = 256;

__global__ __launch_bounds__(kPlainThreads) void index_plain_kernel(IndexArgs a) {
  extern __shared__ float qs[];  // [heads * dim]
  const int row = blockIdx.y;
  const int b = row / a.tq, t = row % a.tq;
  const int HD = a.heads * a.dim;
  const int64_t qoff = (int64_t)b * a.q.sb + (int64_t)t * a.q.sr;
  for (int i = threadIdx.x; i < HD; i += kPlainThreads) qs[i] = load_elem(a.q.data, a.q.dtype, qoff + i);
  __syncthreads();
  const int j = blockIdx.x * kPlainThreads + threadIdx.x;
  if (j >= a.n_cap) return;
  const int V = visible_blocks(a.q_pos[row], a.m);
  float score = kNegInf;
  if (j < V) {
    const int64_t koff = (int64_t)b * a.k.sb + (int64_t)j * a.k.sr;
    score = 0.f;
    for (int h = 0; h < a.heads; ++h) {
      float dot = 0.f;
      for (int d = 0; d < a.dim; ++d) dot = fmaf(qs[h * a.dim + d], load_elem(a.k.data, a.k.dtype, koff + d), dot);
      score = fmaf(a.w[(int64_t)row * a.heads + h], fmaxf(dot, 0.f), score);
    }
  }
  a.scores[(int64_t)row * a.n_cap + j] = score;
}

// ------------------------------------------------------------------ bf16 MFMA
// heads == 8, dim == 64.  Workgroup tile: 16 queries x 128 keys; each of the 4
// waves takes 32 keys (2 column tiles of 16) for all 16 queries (8 row tiles
// of 2 queries x 8 heads).
constexpr int kBfQT = 16;
constexpr int kBfKT = 128;

__global__ __launch_bounds__(256) void index_bf16_kernel(IndexArgs a) {
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * kBfQT;
  const int kbase = blockIdx.x * kBfKT;
  const int wave = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int g = l / 16, n = l % 16;

  int Vmax = 0;
  for (int i = 0; i < kBfQT && q0 + i < a.tq; ++i) Vmax = max(Vmax, visible_blocks(a.q_pos[b * a.tq + q0 + i], a.m));

  // B operands: key = kbase + 32*wave + 16*nt + n ; k-step ks covers dims 32*ks + 8*g .. +7
  v8bf B[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = kbase + 32 * wave + 16 * nt + n;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (key < Vmax) {
        const uint16_t* p = (const uint16_t*)a.k.data + (int64_t)b * a.k.sb + (int64_t)key * a.k.sr + 32 * ks + 8 * g;
        B[nt][ks] = *(const v8bf*)p;
      } else {
        for (int e = 0; e < 8; ++e) B[nt][ks][e] = (__bf16)0.f;
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < kBfQT / 2; ++mt) {
    const int qa = q0 + 2 * mt;  // row tile = queries qa, qa+1; row m -> query qa + m/8, head m%8
    if (qa >= a.tq) break;
    // A operand: row m = n (lane%16), dims 32*ks + 8*g .. +7
    const int qq = qa + n / 8, hh = n % 8;
    v8bf A[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (qq < a.tq) {
        const int64_t off = (int64_t)b * a.q.sb + (int64_t)qq * a.q.sr + hh * 64 + 32 * ks + 8 * g;
        A[ks] = *(const v8bf*)((const uint16_t*)a.q.data + off);
      } else {
        for (int e = 0; e < 8; ++e) A[ks][e] = (__bf16)0.f;
      }
    }
    // this lane's output rows: m = 4g + r -> query qa + (g >= 2), heads 4*(g&1) + r
    const int myq = qa + (g >> 1);
    float wv[4];
    const int Vq = myq < a.tq ? visible_blocks(a.q_pos[b * a.tq + myq], a.m) : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r] = myq < a.tq ? a.w[((int64_t)b * a.tq + myq) * 8 + 4 * (g & 1) + r] : 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], B[nt][1], c, 0, 0, 0);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(wv[r], fmaxf(c[r], 0.f), part);
      const float other = __shfl_xor(part, 16);
      const float tot = (g & 1) ? other + part : part + other;  // heads 0-3 first, then 4-7
      const int key = kbase + 32 * wave + 16 * nt + n;
      if ((g & 1) == 0 && myq < a.tq && key < a.n_cap)
        a.scores[((int64_t)b * a.tq + myq) * a.n_cap + key] = key < Vq ? tot : kNegInf;
    }
  }
}

// ------------------------------------------------------------------ MXFP4 MFMA
// heads <= 32, dim == 64.  Each wave streams groups of 32 keys; a workgroup of
// 4 waves covers kFp4KeysPerWG keys of one query row.
constexpr int kFp4KeysPerWave = 1024;
constexpr int kFp4KeysPerWG = 4 * kFp4KeysPerWave;
constexpr int kFp4Unroll = 8;

__global__ __launch_bounds__(256) void index_mxfp4_kernel(IndexArgs a) {
  const int row = blockIdx.y;
  const int b = row / a.tq, t = row % a.tq;
  const int wave = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int V = visible_blocks(a.q_pos[row], a.m);
  const int wbase = blockIdx.x * kFp4KeysPerWG + wave * kFp4KeysPerWave;
  if (wbase >= a.n_cap) return;

  // A operand: row (head) m = l%32, K block kb = l/32, quantised to MXFP4 here.
  const int m = l % 32, kb = l / 32;
  v8i A = {0, 0, 0, 0, 0, 0, 0, 0};
  int sa = 127;
  if (m < a.heads) {
    const float* qp = (const float*)a.q.data + (int64_t)b * a.q.sb + (int64_t)t * a.q.sr + m * 64 + 32 * kb;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) { v[i] = qp[i]; amax = fmaxf(amax, fabsf(v[i])); }
    const int e = mx_scale_exp(amax);
    sa = e + 127;
    if (amax > 0.f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) A[i / 8] |= (int)(f32_to_e2m1(v[i], e) << (4 * (i % 8)));
    }
  }
  // head weights for this lane's accumulator rows m = 8*(r/4) + 4*(l/32) + r%4
  float wv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = 8 * (r / 4) + 4 * (l / 32) + (r % 4);
    wv[r] = h < a.heads ? a.w[(int64_t)row * a.heads + h] : 0.f;
  }
  const uint8_t* kc = (const uint8_t*)a.k.data + (int64_t)b * a.k.sb + 16 * kb;
  const uint8_t* ks = (const uint8_t*)a.k.scale + (int64_t)b * a.k.ssb + kb;
  float* srow = a.scores + (int64_t)row * a.n_cap;
  const int wend = min(wbase + kFp4KeysPerWave, a.n_cap);

  for (int g0 = wbase; g0 < wend; g0 += 32 * kFp4Unroll) {
    v4i codes[kFp4Unroll];
    int sb[kFp4Unroll];
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int key = g0 + 32 * u + (l % 32);
      if (key < V) {
        codes[u] = *(const v4i*)(kc + (int64_t)key * a.k.sr);
        sb[u] = ks[(int64_t)key * a.k.ssr];
      } else {
        codes[u] = (v4i){0, 0, 0, 0};
        sb[u] = 127;
      }
    }
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      v8i Bop = {codes[u][0], codes[u][1], codes[u][2], codes[u][3], 0, 0, 0, 0};
      v16f c;
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = 0.f;
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bop, c, 4, 4, 0, sa, 0, sb[u]);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part = fmaf(wv[r], fmaxf(c[r], 0.f), part);
      const float other = __shfl_xor(part, 32);
      const int key = g0 + 32 * u + l;
      if (l < 32 && key < wend) srow[key] = key < V ? part + other : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s) {
  const int rows = a.batch * a.tq;
  if (rows == 0 || a.n_cap == 0) return hipSuccess;
  if (a.k.dtype == CSA_MXFP4) {
    dim3 grid((a.n_cap + kFp4KeysPerWG - 1) / kFp4KeysPerWG, rows);
    hipLaunchKernelGGL(index_mxfp4_kernel, grid, dim3(256), 0, s, a);
  } else if (a.k.dtype == CSA_BF16 && a.q.dtype == CSA_BF16 && a.heads == 8 && a.dim == 64) {
    dim3 grid((a.n_cap + kBfKT - 1) / kBfKT, (a.tq + kBfQT - 1) / kBfQT, a.batch);
    hipLaunchKernelGGL(index_bf16_kernel, grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((a.n_cap + kPlainThreads - 1) / kPlainThreads, rows);
    const size_t lds = (size_t)a.heads * a.dim * sizeof(float);
    hipLaunchKernelGGL(index_plain_kernel, grid, dim3(kPlainThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace csa

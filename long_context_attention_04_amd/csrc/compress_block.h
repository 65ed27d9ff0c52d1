// The compression of one block (a workgroup's work) and the arithmetic it is made
// of, shared by the compression kernels and the indexer launch that runs a
// decode step's compressions alongside its scoring: one code path, so every
// caller produces bitwise the same stored entries.
//
// Compression merges each block of m adjacent raw rows into one entry
// (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
// and HCA bullets), read as a softmax-weighted sum over the m offsets with one
// logit per offset; the stored format's quantisation is fused into the store.
#pragma once
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kCompressThreads = 256;
constexpr int kRowBatch = 4;
constexpr float kNegInfC = -__builtin_inff();

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x / kWave); ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Writes one finished fp32 row (thread t holds columns t + 256*i, i < nv) in the output format.
template <int NV>
__device__ __forceinline__ void store_row(const float (&vals)[NV], int nv, int out_dtype, void* out, int64_t off,
                                          void* out_scale, int64_t soff, float* red) {
  const int t = threadIdx.x;
  if (out_dtype == CSA_F32) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i < nv) ((float*)out)[off + t + i * kCompressThreads] = vals[i];
  } else if (out_dtype == CSA_BF16) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i < nv) ((uint16_t*)out)[off + t + i * kCompressThreads] = f32_to_bf16_bits(vals[i]);
  } else if (out_dtype == CSA_FP8_E4M3) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i < nv) amax = fmaxf(amax, fabsf(vals[i]));
    amax = block_max(amax, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i < nv) ((uint8_t*)out)[off + t + i * kCompressThreads] = (uint8_t)f32_to_e4m3(__fdiv_rn(vals[i], s));
    if (t == 0) ((float*)out_scale)[soff] = s;
  } else {  // MXFP4: 32 consecutive columns live in 32 consecutive lanes
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i >= nv) continue;
      const int col = t + i * kCompressThreads;
      float a = fabsf(vals[i]);
      for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
      const int e = mx_scale_exp(a);
      uint32_t nib = a > 0.f ? f32_to_e2m1(vals[i], e) : 0u;
      const uint32_t hi = __shfl_down(nib, 1, 32);
      if ((col & 1) == 0) ((uint8_t*)out)[off + col / 2] = (uint8_t)(nib | (hi << 4));
      if ((col & 31) == 0) ((uint8_t*)out_scale)[soff + col / 32] = (uint8_t)(e + 127);
    }
  }
}

constexpr int kLocalSoftmaxMax = 16;  // up to this many offsets every thread forms the weights itself

// One element of a stored raw row; the input format is a compile-time choice so the
// loads of a row group are issued back to back.
template <int IN>
__device__ __forceinline__ float load_raw(const void* p, int64_t i) {
  if constexpr (IN == CSA_F32) return ((const float*)p)[i];
  else if constexpr (IN == CSA_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  else return e4m3_to_f32(((const uint8_t*)p)[i]);
}

// The softmax weights of m <= kLocalSoftmaxMax offset logits (loaded into zl), in
// fp32: max-subtracted, exponentials summed in ascending offset order, each divided
// by the sum.  Every thread does the same arithmetic.
// N: capacity of zl (m <= N); the operations, and their order, do not depend on it.
template <int N>
__device__ __forceinline__ void local_softmax(int m, float (&zl)[N]) {
  float mx = zl[0];
#pragma unroll
  for (int r = 1; r < N; ++r)
    if (r < m) mx = fmaxf(mx, zl[r]);
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < N; ++r)
    if (r < m) {
      zl[r] = expf(zl[r] - mx);
      sum += zl[r];
    }
#pragma unroll
  for (int r = 0; r < N; ++r)
    if (r < m) zl[r] = __fdiv_rn(zl[r], sum);
}

// One stored element's merged value: column col of block j (raw rows row0 .. row0+m-1
// of sequence b) with the local weights w, terms added in ascending offset order --
// exactly the per-column arithmetic of compress_block.
// The raw values it reads (x[r] = row row0 + r, column col, fp8 rows times their
// scale), r < a.m <= N; and their combination, in that order.
template <int IN, int N>
__device__ __forceinline__ void compress_element_load(const CompressArgs& a, int b, int64_t row0, int col,
                                                      float (&x)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) {
    if (r >= a.m) break;
    float xv = load_raw<IN>(a.raw.data, (int64_t)b * a.raw.sb + (row0 + r) * a.raw.sr + col);
    if (IN == CSA_FP8_E4M3 && a.raw.scale)
      xv *= ((const float*)a.raw.scale)[(int64_t)b * a.raw.ssb + (row0 + r) * a.raw.ssr];
    x[r] = xv;
  }
}
template <int N>
__device__ __forceinline__ float compress_element_combine(int m, const float (&x)[N], const float (&w)[N]) {
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    if (r >= m) break;
    acc = fmaf(w[r], x[r], acc);
  }
  return acc;
}

// Block i of sequence b of one compression (a workgroup's whole work).
// LOCAL_ONLY: m <= kLocalSoftmaxMax is known (omega_s is then never touched).
template <int NV, int IN, bool LOCAL_ONLY = false>  // columns per thread: dim <= 256 * NV; IN: raw row format
__device__ __forceinline__ void compress_block(const CompressArgs& a, int b, int i, float* omega_s, float* red) {
  // independent scalars first, all in flight together (one memory round trip)
  const int cnt = a.block_count[b];
  const int jfirst = a.block_first[b];
  const int rbase = a.raw_base[b];
  const int m = a.m;
  float zl[kLocalSoftmaxMax];  // logits, held by every thread when m is small
  const bool local = LOCAL_ONLY || m <= kLocalSoftmaxMax;
  if (local) {
#pragma unroll
    for (int r = 0; r < kLocalSoftmaxMax; ++r)
      if (r < m) zl[r] = a.logits[r];
  }
  if (i >= cnt) return;
  const int j = jfirst + i;
  const int64_t row0 = (int64_t)j * m - rbase;
  float acc[NV];
  const int nv = (a.dim - threadIdx.x + kCompressThreads - 1) / kCompressThreads;
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.f;

  // omega = softmax(logits) in fp32: max-subtracted, exponentials summed in ascending
  // offset order, each weight divided by the sum.  The same arithmetic on every thread.
  if (local) {
    local_softmax(m, zl);
  } else if constexpr (!LOCAL_ONLY) {
    for (int r = threadIdx.x; r < m; r += kCompressThreads) omega_s[r] = a.logits[r];
    __syncthreads();
    float lm = kNegInfC;
    for (int r = threadIdx.x; r < m; r += kCompressThreads) lm = fmaxf(lm, omega_s[r]);
    const float mx = block_max(lm, red);
    for (int r = threadIdx.x; r < m; r += kCompressThreads) omega_s[r] = expf(omega_s[r] - mx);
    __syncthreads();
    float sum = 0.f;
    for (int r = 0; r < m; ++r) sum += omega_s[r];  // ascending order, same on every thread
    __syncthreads();
    for (int r = threadIdx.x; r < m; r += kCompressThreads) omega_s[r] = __fdiv_rn(omega_s[r], sum);
    __syncthreads();
  }

  // rows in groups of kRowBatch: all loads of a group are issued before its FMAs
  // (terms are still added in ascending offset order)
  // Loads are unconditional (row and column clamped to valid ones), so a group's loads
  // are all in flight together; out-of-range terms are dropped afterwards.
  auto row_group = [&](int r0, auto wfun) {
    float x[kRowBatch][NV];
    float rs[kRowBatch];
#pragma unroll
    for (int jj = 0; jj < kRowBatch; ++jj) {
      const int r = min(r0 + jj, m - 1);
      const int64_t base = (int64_t)b * a.raw.sb + (row0 + r) * a.raw.sr;
      rs[jj] = IN == CSA_FP8_E4M3 && a.raw.scale
                   ? ((const float*)a.raw.scale)[(int64_t)b * a.raw.ssb + (row0 + r) * a.raw.ssr]
                   : 1.f;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        x[jj][v] = load_raw<IN>(a.raw.data, base + min((int)threadIdx.x + v * kCompressThreads, a.dim - 1));
    }
#pragma unroll
    for (int jj = 0; jj < kRowBatch; ++jj) {
      if (r0 + jj < m) {
        const float w = wfun(jj);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float xv = x[jj][v];
          if (IN == CSA_FP8_E4M3) xv *= rs[jj];
          acc[v] = fmaf(w, xv, acc[v]);  // columns beyond dim are never stored
        }
      }
    }
  };
  if (local) {
#pragma unroll
    for (int r0 = 0; r0 < kLocalSoftmaxMax; r0 += kRowBatch)
      if (r0 < m) row_group(r0, [&](int jj) { return zl[r0 + jj]; });  // compile-time index after unrolling
  } else if constexpr (!LOCAL_ONLY) {
    for (int r0 = 0; r0 < m; r0 += kRowBatch) row_group(r0, [&](int jj) { return omega_s[r0 + jj]; });
  }
  const int64_t off = (int64_t)b * a.out_sb + (int64_t)j * a.out_sr;
  const int64_t soff = (int64_t)b * a.out_ssb + (int64_t)j * a.out_ssr;
  store_row<NV>(acc, nv, a.out_dtype, a.out, off, a.out_scale, soff, red);
}


}  // namespace
}  // namespace csa

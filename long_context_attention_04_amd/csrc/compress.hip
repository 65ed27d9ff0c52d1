// (a) KV compression and the stored-format quantisers.
//
// Compression merges each block of m adjacent raw rows into one entry
// (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
// and HCA bullets).  The merge is read as a softmax-weighted sum over the m
// offsets with one logit per offset.  The work is a short weighted reduction
// over rows that are read once: HBM-bound, so each workgroup streams the m
// rows of one output entry with coalesced column-parallel loads and fuses the
// output quantisation (bf16 / fp8 row scale / MXFP4 block scale) into the
// store.
#include "compress_block.h"

#include <algorithm>

namespace csa {

namespace {

template <int NV, int IN>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs a) {
  __shared__ float omega_s[1024];
  __shared__ float red[kCompressThreads / kWave];
  compress_block<NV, IN>(a, blockIdx.y, blockIdx.x, omega_s, red);
}

// Several independent compressions in one launch (grid.z = job): small decode
// steps are latency-bound, so their chains of dependent loads overlap instead of
// running one launch after another.  Each job's (columns per thread, raw format)
// variant is chosen on the host; the switch is uniform per workgroup.
struct CompressJobs {
  CompressArgs job[kMaxCompressJobs];
  int variant[kMaxCompressJobs];  // 3 * log2(NV) + input format (NV in {1, 2, 4})
};

__global__ __launch_bounds__(kCompressThreads) void compress_jobs_kernel(CompressJobs js) {
  __shared__ float omega_s[1024];
  __shared__ float red[kCompressThreads / kWave];
  const int z = blockIdx.z;
  const CompressArgs& a = js.job[z];
  const int b = blockIdx.y, i = blockIdx.x;
  if (b >= a.batch || i >= a.max_blocks) return;
  switch (js.variant[z]) {
    case 0: compress_block<1, CSA_F32>(a, b, i, omega_s, red); break;
    case 1: compress_block<1, CSA_BF16>(a, b, i, omega_s, red); break;
    case 2: compress_block<1, CSA_FP8_E4M3>(a, b, i, omega_s, red); break;
    case 3: compress_block<2, CSA_F32>(a, b, i, omega_s, red); break;
    case 4: compress_block<2, CSA_BF16>(a, b, i, omega_s, red); break;
    case 5: compress_block<2, CSA_FP8_E4M3>(a, b, i, omega_s, red); break;
    case 6: compress_block<4, CSA_F32>(a, b, i, omega_s, red); break;
    case 7: compress_block<4, CSA_BF16>(a, b, i, omega_s, red); break;
    default: compress_block<4, CSA_FP8_E4M3>(a, b, i, omega_s, red); break;
  }
}

// one thread per 32-element block
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const float* __restrict__ x, int64_t nblocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t blk = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const float4* p = (const float4*)(x + blk * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = p[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_scale_exp(amax);
  uint32_t w[4] = {0, 0, 0, 0};
  if (amax > 0.f) {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i / 8] |= f32_to_e2m1(v[i], e) << (4 * (i % 8));
  }
  *(uint4*)(codes + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[blk] = (uint8_t)(e + 127);
}

// one workgroup per row
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const float* __restrict__ x, int cols,
                                                           uint8_t* __restrict__ codes, float* __restrict__ rs) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * cols;
  float amax = 0.f;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(xr[c]));
  amax = block_max(amax, red);
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  for (int c = threadIdx.x; c < cols; c += blockDim.x)
    codes[row * cols + c] = (uint8_t)f32_to_e4m3(__fdiv_rn(xr[c], s));
  if (threadIdx.x == 0) rs[row] = s;
}

}  // namespace

template <int IN>
hipError_t launch_compress_in(const CompressArgs& a, hipStream_t s) {
  dim3 grid(a.max_blocks, a.batch);
  const int nv = (a.dim + kCompressThreads - 1) / kCompressThreads;
  if (nv <= 1) hipLaunchKernelGGL((compress_kernel<1, IN>), grid, dim3(kCompressThreads), 0, s, a);
  else if (nv <= 2) hipLaunchKernelGGL((compress_kernel<2, IN>), grid, dim3(kCompressThreads), 0, s, a);
  else if (nv <= 4) hipLaunchKernelGGL((compress_kernel<4, IN>), grid, dim3(kCompressThreads), 0, s, a);
  else if (nv <= 8) hipLaunchKernelGGL((compress_kernel<8, IN>), grid, dim3(kCompressThreads), 0, s, a);
  else hipLaunchKernelGGL((compress_kernel<16, IN>), grid, dim3(kCompressThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compress_jobs(const CompressArgs* jobs, int n, hipStream_t s) {
  CompressJobs js{};
  int gx = 0, gy = 0, nz = 0;
  for (int j = 0; j < n; ++j) {
    const CompressArgs& a = jobs[j];
    if (a.max_blocks <= 0 || a.batch <= 0) continue;
    const int nv = (a.dim + kCompressThreads - 1) / kCompressThreads;
    if (nv > 4) {  // wide rows: a launch of their own
      const hipError_t e = launch_compress(a, s);
      if (e != hipSuccess) return e;
      continue;
    }
    const int in = a.raw.dtype == CSA_F32 ? 0 : a.raw.dtype == CSA_BF16 ? 1 : 2;
    js.job[nz] = a;
    js.variant[nz] = 3 * (nv <= 1 ? 0 : nv <= 2 ? 1 : 2) + in;
    gx = std::max(gx, a.max_blocks);
    gy = std::max(gy, a.batch);
    ++nz;
  }
  if (nz == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_jobs_kernel, dim3(gx, gy, nz), dim3(kCompressThreads), 0, s, js);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.max_blocks <= 0 || a.batch <= 0) return hipSuccess;
  if (a.raw.dtype == CSA_F32) return launch_compress_in<CSA_F32>(a, s);
  if (a.raw.dtype == CSA_BF16) return launch_compress_in<CSA_BF16>(a, s);
  return launch_compress_in<CSA_FP8_E4M3>(a, s);
}

hipError_t launch_quantize_mxfp4(const float* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, x, nblocks,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const float* x, int64_t rows, int cols, uint8_t* codes, float* row_scale,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)rows), dim3(256), 0, s, x, cols, codes, row_scale);
  return hipGetLastError();
}

}  // namespace csa

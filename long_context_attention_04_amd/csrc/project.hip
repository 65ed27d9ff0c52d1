// Dense projections on either side of the hot path, all "NT" products
// Y[M x N] = X[M x K] . W[N x K]^T with K contiguous in both operands, so MFMA
// operands load straight from memory: lane (i, g) of a 16x16x32 bf16 MFMA takes 8
// consecutive K elements of row i of X (A operand) or of row i of W (B operand).  A
// wave computes one 16 x 16 output tile.
//
// * Indexer query from the query hidden state (b-lab.team summary of DeepSeek-V4,
//   Core Methodological Innovations 1, CSA bullet: the indexer scores with low-rank
//   projections of h_t): c = W_dq h (rank r), q_I = W_uq c, w = W_w h.  c is rounded
//   to bf16 between the two projections (the operand precision of the second).
// * MLA absorbed query and output up-projection, one product per head (reading of
//   the same bullet: attention reads shared latent rows c, head h's key being
//   W_uk[h] c and its value W_uv[h] c): q_lat_h = W_uk[h]^T q_h and o_h = W_uv[h] o_lat_h.
//   The fp32 attention output enters the MFMA as bf16 hi + lo (x = hi + lo to about
//   16 significant bits), two products with the same weight operand.
//
// Sums over K are batch-invariant: K is cut into chunks of 128; each chunk's
// partial sum starts from zero (its MFMAs in order) and the partials are added in
// ascending chunk order, in registers when one wave covers every chunk (many rows)
// or by the reduce kernel when the chunks are spread over waves (few rows, where the
// weight stream must be spread over the chip).  Either way the bits are the same,
// whatever the number of rows.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kProjThreads = 256;  // 4 waves, one output tile each
constexpr int kKChunk = 128;       // K elements per partial sum (4 MFMA steps)

struct NtArgs {
  const void* x;  // X rows: row R at (R / tq) * xsb + (R % tq) * xsr (elements); head z at + z * xsh
  int64_t xsb, xsr, xsh;
  int tq, M, K;
  const uint16_t* w0;  // W rows 0 .. n0-1 (pitch ldw0), then rows n0 .. n0+n1-1 of w1; head z at + z * wsh
  int64_t ldw0;
  int n0;
  const uint16_t* w1;
  int64_t ldw1;
  int n1;
  int64_t wsh;
  float* part;  // [heads][nsplit][M][n0 + n1] partial sums
  int nsplit, cps;  // splits of the chunk range and chunks per split
  // with one split (no reduce launch): columns < n0 go straight to y0 (row R at
  // (R / ytq) * y0sb + (R % ytq) * y0sr, head z at + z * y0sh, fp32 or bf16), the rest to
  // y1 (fp32 [M][n1])
  void* y0;
  int ytq;
  int64_t y0sb, y0sr, y0sh;
  int y0_bf16;
  float* y1;
};

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return *(const v8bf*)p; }

// Eight fp32 values as bf16 hi (round to nearest even) and lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float* p, v8bf* hi, v8bf* lo) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)x[e];
    (*hi)[e] = h;
    (*lo)[e] = (__bf16)(x[e] - (float)h);
  }
}

template <bool XF32>
__global__ __launch_bounds__(kProjThreads) void nt_partial_kernel(NtArgs a) {
  const int N = a.n0 + a.n1;
  const int mtiles = (a.M + 15) / 16, ntiles = (N + 15) / 16;
  const int64_t wid = (int64_t)blockIdx.x * (kProjThreads / kWave) + threadIdx.x / kWave;
  if (wid >= (int64_t)mtiles * ntiles * a.nsplit) return;  // wave-uniform; no barriers below
  const int lane = threadIdx.x % kWave, i = lane % 16, g = lane / 16;
  const int z = blockIdx.y;  // head
  // consecutive waves take consecutive column tiles of one row tile and split
  const int nt = (int)(wid % ntiles);
  const int mt = (int)((wid / ntiles) % mtiles);
  const int sp = (int)(wid / ((int64_t)ntiles * mtiles));
  const int xr = 16 * mt + i, wr = 16 * nt + i;  // this lane's X row and W row
  const bool xlive = xr < a.M, wlive = wr < N;
  const int64_t xo = (xlive ? (int64_t)(xr / a.tq) * a.xsb + (int64_t)(xr % a.tq) * a.xsr : 0) + z * a.xsh + 8 * g;
  const uint16_t* wp = (wr < a.n0 ? a.w0 + (int64_t)wr * a.ldw0 : a.w1 + (int64_t)(wlive ? wr - a.n0 : 0) * a.ldw1) +
                       z * a.wsh + 8 * g;
  const int nch = (a.K + kKChunk - 1) / kKChunk;
  const int c_lo = sp * a.cps, c_hi = min(nch, c_lo + a.cps);
  const v8bf zero = (v8bf){};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = c_lo; c < c_hi; ++c) {
    const int k0 = c * kKChunk;
    const int steps = min(4, (a.K - k0) / 32);  // K is a multiple of 32
    v8bf xa[4], xl[4], wb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool in = s < steps;
      xa[s] = zero;
      xl[s] = zero;
      if (in && xlive) {
        if constexpr (XF32)
          split8((const float*)a.x + xo + k0 + 32 * s, &xa[s], &xl[s]);
        else
          xa[s] = ld8((const uint16_t*)a.x + xo + k0 + 32 * s);
      }
      wb[s] = in && wlive ? ld8(wp + k0 + 32 * s) : zero;
    }
    v4f part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < steps) {
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], wb[s], part, 0, 0, 0);
        if constexpr (XF32) part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl[s], wb[s], part, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += part[r];  // chunks in ascending order
  }
  // C layout: lane (column i, group g) holds rows 4g + r of the tile
  const int col = 16 * nt + i;
  if (col < N) {
    if (a.nsplit == 1) {  // every chunk summed here: the result itself
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * g + r;
        if (row >= a.M) continue;
        if (col < a.n0) {
          const int64_t o = (int64_t)(row / a.ytq) * a.y0sb + (int64_t)(row % a.ytq) * a.y0sr + z * a.y0sh + col;
          if (a.y0_bf16)
            ((__bf16*)a.y0)[o] = (__bf16)acc[r];
          else
            ((float*)a.y0)[o] = acc[r];
        } else {
          a.y1[(int64_t)row * a.n1 + (col - a.n0)] = acc[r];
        }
      }
      return;
    }
    float* out = a.part + ((int64_t)z * a.nsplit + sp) * a.M * N;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      if (row < a.M) out[(int64_t)row * N + col] = acc[r];
    }
  }
}

// Sum of the splits' partials in ascending order, then out: columns < n0 go to
// y0 (rows mapped like X through (y0sb, y0sr, tq), head z at + z * y0sh, as fp32 or
// bf16), columns n0 .. n0+n1-1 to y1 (fp32 [M][n1], one head only).
struct ReduceArgs {
  const float* part;
  int nsplit, M, n0, n1, tq;
  void* y0;
  int64_t y0sb, y0sr;
  int y0_bf16;
  float* y1;
  int64_t y0sh;
};

__global__ __launch_bounds__(256) void nt_reduce_kernel(ReduceArgs a) {
  const int N = a.n0 + a.n1;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)a.M * N) return;
  const int z = blockIdx.y;
  const int row = (int)(id / N), col = (int)(id % N);
  const float* part = a.part + (int64_t)z * a.nsplit * a.M * N + (int64_t)row * N + col;
  const int64_t ss = (int64_t)a.M * N;  // between splits
  // ascending split order, eight loads in flight at a time
  float v = 0.f;
  for (int sp0 = 0; sp0 < a.nsplit; sp0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sp0 + j < a.nsplit ? part[(sp0 + j) * ss] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (sp0 + j < a.nsplit) v += x[j];
  }
  if (col < a.n0) {
    const int64_t o = (int64_t)(row / a.tq) * a.y0sb + (int64_t)(row % a.tq) * a.y0sr + z * a.y0sh + col;
    if (a.y0_bf16)
      ((__bf16*)a.y0)[o] = (__bf16)v;
    else
      ((float*)a.y0)[o] = v;
  } else {
    a.y1[(int64_t)row * a.n1 + (col - a.n0)] = v;
  }
}

// Splits of the K chunks: every chunk its own split when there are few rows (the
// weights are then streamed by many waves), one split otherwise.
int proj_nsplit(int64_t rows, int K) { return rows <= 64 ? (K + kKChunk - 1) / kKChunk : 1; }

hipError_t launch_nt(const NtArgs& a0, int heads, bool xf32, hipStream_t s) {
  NtArgs a = a0;
  const int nch = (a.K + kKChunk - 1) / kKChunk;
  a.cps = (nch + a.nsplit - 1) / a.nsplit;
  const int64_t waves = (int64_t)((a.M + 15) / 16) * ((a.n0 + a.n1 + 15) / 16) * a.nsplit;
  const dim3 grid((unsigned)((waves + kProjThreads / kWave - 1) / (kProjThreads / kWave)), (unsigned)heads);
  if (xf32)
    hipLaunchKernelGGL(nt_partial_kernel<true>, grid, dim3(kProjThreads), 0, s, a);
  else
    hipLaunchKernelGGL(nt_partial_kernel<false>, grid, dim3(kProjThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int heads, hipStream_t s) {
  const int64_t n = (int64_t)a.M * (a.n0 + a.n1);
  hipLaunchKernelGGL(nt_reduce_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t index_query_workspace_bytes(int64_t rows, int d_model, int rank, int n_idx_heads, int idx_dim) {
  const size_t p1 = (size_t)proj_nsplit(rows, d_model) * rows * (rank + n_idx_heads) * sizeof(float);
  const size_t p2 = (size_t)proj_nsplit(rows, rank) * rows * n_idx_heads * idx_dim * sizeof(float);
  return align256(std::max(p1, p2)) + align256((size_t)rows * rank * 2);
}

hipError_t launch_index_query(const IndexQueryArgs& q, hipStream_t s) {
  const int64_t rows = (int64_t)q.batch * q.tq;
  if (rows == 0) return hipSuccess;
  const int HD = q.n_idx_heads * q.idx_dim;
  float* part = (float*)q.ws;
  const size_t p1 = (size_t)proj_nsplit(rows, q.d_model) * rows * (q.rank + q.n_idx_heads) * sizeof(float);
  const size_t p2 = (size_t)proj_nsplit(rows, q.rank) * rows * HD * sizeof(float);
  uint16_t* cbuf = (uint16_t*)((uint8_t*)q.ws + align256(std::max(p1, p2)));
  // projection 1: [c | w] = h . [W_dq ; W_w]^T
  NtArgs a1{};
  a1.x = q.h;
  a1.xsb = q.h_sb;
  a1.xsr = q.h_sr;
  a1.tq = q.tq;
  a1.M = (int)rows;
  a1.K = q.d_model;
  a1.w0 = (const uint16_t*)q.w_dq;
  a1.ldw0 = q.ld_dq;
  a1.n0 = q.rank;
  a1.w1 = (const uint16_t*)q.w_w;
  a1.ldw1 = q.ld_w;
  a1.n1 = q.n_idx_heads;
  a1.part = part;
  a1.nsplit = proj_nsplit(rows, q.d_model);
  a1.y0 = cbuf;  // c: [rows][rank] bf16, row R at R * rank
  a1.ytq = 1;
  a1.y0sb = q.rank;
  a1.y0sr = 0;
  a1.y0sh = 0;
  a1.y0_bf16 = 1;
  a1.y1 = q.w_out;
  hipError_t e = launch_nt(a1, 1, false, s);
  if (e != hipSuccess) return e;
  if (a1.nsplit > 1) {
    ReduceArgs r1{part, a1.nsplit, (int)rows, q.rank, q.n_idx_heads, 1, cbuf, q.rank, 0, 1, q.w_out, 0};  // c: [rows][rank]
    if ((e = launch_reduce(r1, 1, s)) != hipSuccess) return e;
  }
  // projection 2: q_I = c . W_uq^T
  NtArgs a2{};
  a2.x = cbuf;
  a2.xsb = 0;
  a2.xsr = q.rank;
  a2.tq = 1 << 30;  // c rows are contiguous: row R at R * rank
  a2.M = (int)rows;
  a2.K = q.rank;
  a2.w0 = (const uint16_t*)q.w_uq;
  a2.ldw0 = q.ld_uq;
  a2.n0 = HD;
  a2.w1 = a2.w0;
  a2.ldw1 = 0;
  a2.n1 = 0;
  a2.part = part;
  a2.nsplit = proj_nsplit(rows, q.rank);
  a2.y0 = q.q_out;
  a2.ytq = q.tq;
  a2.y0sb = q.q_sb;
  a2.y0sr = q.q_sr;
  a2.y0sh = 0;
  a2.y0_bf16 = q.q_bf16;
  a2.y1 = nullptr;
  if ((e = launch_nt(a2, 1, false, s)) != hipSuccess) return e;
  if (a2.nsplit == 1) return hipSuccess;
  ReduceArgs r2{part, a2.nsplit, (int)rows, HD, 0, q.tq, q.q_out, q.q_sb, q.q_sr, q.q_bf16, nullptr, 0};
  return launch_reduce(r2, 1, s);
}

size_t latent_proj_workspace_bytes(int64_t rows, int heads, int K, int N) {
  return align256((size_t)proj_nsplit(rows, K) * heads * rows * N * sizeof(float));
}

hipError_t launch_latent_proj(const LatentProjArgs& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  // per head z: Y_z[rows x N] = X_z[rows x K] . W_z[N x K]^T, X rows pitched heads * K,
  // W_z at z * N * K, Y rows pitched heads * N
  NtArgs a{};
  a.x = p.x;
  a.xsb = 0;
  a.xsr = (int64_t)p.heads * p.K;
  a.xsh = p.K;
  a.tq = 1 << 30;
  a.M = (int)p.rows;
  a.K = p.K;
  a.w0 = (const uint16_t*)p.w;
  a.ldw0 = p.K;
  a.n0 = p.N;
  a.w1 = a.w0;
  a.ldw1 = 0;
  a.n1 = 0;
  a.wsh = (int64_t)p.N * p.K;
  a.part = (float*)p.ws;
  a.nsplit = proj_nsplit(p.rows, p.K);
  a.y0 = p.y;
  a.ytq = 1 << 30;
  a.y0sb = 0;
  a.y0sr = (int64_t)p.heads * p.N;
  a.y0sh = p.N;
  a.y0_bf16 = p.y_bf16;
  a.y1 = nullptr;
  hipError_t e = launch_nt(a, p.heads, p.x_f32 != 0, s);
  if (e != hipSuccess) return e;
  if (a.nsplit == 1) return hipSuccess;
  ReduceArgs r{a.part, a.nsplit, (int)p.rows, p.N, 0, 1 << 30, p.y, 0, (int64_t)p.heads * p.N, p.y_bf16, nullptr, p.N};
  return launch_reduce(r, p.heads, s);
}

}  // namespace csa

// (c) Per-query top-k selection of compressed blocks.
//
// The indexer's scores choose "the top-k most relevant compressed KV blocks"
// (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
// bullet).  Reading of the order: score descending, then block index
// ascending; the selected set is written in ascending index order, padded
// with -1.
//
// Selection is an exact radix select on an order-preserving 32-bit key of the
// fp32 score (-0 folded onto +0), with ties broken by index, followed by an
// ascending-order compaction.  Integer histograms only, so results are exact
// and do not depend on scheduling.
//  * Rows of up to kTopkLdsMax keys: one workgroup per row, the row resident
//    in LDS, four 8-bit passes, then a block-scan compaction.
//  * Longer rows (1M-token decode: 262,144 blocks per row and few rows):
//    the row is split over many workgroups.  Pass 1 builds a 4096-bin
//    histogram of the top 12 key bits (LDS histogram, then integer atomics
//    into a per-row histogram); the last workgroup of the row to finish picks
//    the threshold bin.  Pass 2 sets a bitmap bit for every key above that
//    bin and appends the keys inside it to a candidate list; the last
//    workgroup of the row resolves the candidates exactly (radix passes over
//    the remaining 20 key bits, then over the index for exact ties), sets
//    their bits and compacts the bitmap into ascending indices.  "Last
//    workgroup" is decided by an atomic counter after a release fence; no
//    workgroup ever waits for another.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace csa {

namespace {

// ------------------------------------------------------------------ block helpers
// Inclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
__device__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp /* >= 16 */, uint32_t* total) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (l >= o) v += u;
  }
  if (l == kWave - 1) tmp[w] = v;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) base += tmp[i];
    tot += tmp[i];
  }
  __syncthreads();
  if (total) *total = tot;
  return v + base;
}

// Given a histogram (bins ascending = keys ascending) and krem >= 1 with
// sum(hist) >= krem, find the bin d holding the krem-th largest key:
// count(bins > d) < krem <= count(bins >= d).  Writes d and count(bins > d).
__device__ void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t krem, uint32_t* tmp,
                                   uint32_t* out_bin, uint32_t* out_above) {
  const int per = nbins / (int)blockDim.x;  // nbins is a multiple of blockDim
  const int lo = threadIdx.x * per;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += hist[lo + i];
  uint32_t tot;
  const uint32_t incl = block_incl_scan(mine, tmp, &tot);
  uint32_t running = tot - incl;  // keys in bins above this thread's range
  for (int d = lo + per - 1; d >= lo; --d) {
    const uint32_t h = hist[d];
    if (running < krem && running + h >= krem) {
      *out_bin = (uint32_t)d;
      *out_above = running;
    }
    running += h;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ LDS path
constexpr int kLdsThreads = 512;

__global__ __launch_bounds__(kLdsThreads) void topk_lds_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ q_pos, int n_cap, int m,
                                                               int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t sh_bin, sh_above;
  const int64_t row = blockIdx.x;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kLdsThreads) out[i] = i < V ? i : -1;
    return;
  }
  const float* srow = scores + row * n_cap;
  for (int i = threadIdx.x; i < V; i += kLdsThreads) keys[i] = float_key(srow[i]);
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < V; i += kLdsThreads) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    {  // 256 bins, 512 threads: threads < 256 own one bin each
      const uint32_t h = threadIdx.x < 256 ? hist[threadIdx.x] : 0u;
      uint32_t tot;
      const uint32_t incl = block_incl_scan(h, tmp, &tot);
      const uint32_t above = tot - incl;  // keys in bins > this bin
      if (threadIdx.x < 256 && above < krem && above + h >= krem) {
        sh_bin = threadIdx.x;
        sh_above = above;
      }
      __syncthreads();
    }
    prefix |= sh_bin << shift;
    mask |= 0xffu << shift;
    krem -= sh_above;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the k-th largest key; take krem of its copies (lowest indices)
  const int seg = (V + kLdsThreads - 1) / kLdsThreads;
  const int lo = min(V, (int)threadIdx.x * seg), hi = min(V, lo + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    gt += key > T;
    eq += key == T;
  }
  const uint32_t eq_before = block_incl_scan(eq, tmp, nullptr) - eq;
  const uint32_t take = eq_before >= krem ? 0u : min(eq, krem - eq_before);
  const uint32_t sel = gt + take;
  uint32_t pos = block_incl_scan(sel, tmp, nullptr) - sel;
  uint32_t taken = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    bool s = key > T;
    if (key == T && taken < take) { s = true; ++taken; }
    if (s) {
      if (pos < (uint32_t)k) out[pos] = i;
      ++pos;
    }
  }
}

// ------------------------------------------------------------------ multi-WG path
constexpr int kBins = 4096;  // top 12 key bits
constexpr int kLThreads = 256;
constexpr int kCandLds = 6144;  // candidates resolved from LDS when they fit

struct RowCtl {  // one per row, 8 words
  uint32_t done1, done2, cand_count, bin, krem, pad0, pad1, pad2;
};

struct LWs {
  uint32_t* hist;    // [rows][kBins]
  RowCtl* ctl;       // [rows]
  uint2* cand;       // [rows][n_cap]  (key, index)
  uint32_t* bitmap;  // [rows][words]
  int words;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline LWs carve(void* ws, int64_t rows, int n_cap) {
  LWs w;
  char* p = (char*)ws;
  w.words = (n_cap + 63) / 64 * 2;
  w.hist = (uint32_t*)p;
  p += align256((size_t)rows * kBins * 4);
  w.ctl = (RowCtl*)p;
  p += align256((size_t)rows * sizeof(RowCtl));
  w.cand = (uint2*)p;
  p += align256((size_t)rows * n_cap * 8);
  w.bitmap = (uint32_t*)p;
  return w;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void topk_clear_kernel(LWs w, int64_t rows) {
  const int64_t n = rows * kBins;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    w.hist[i] = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < rows * 8; i += (int64_t)gridDim.x * blockDim.x)
    ((uint32_t*)w.ctl)[i] = 0;
}

__global__ __launch_bounds__(kLThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ q_pos, int n_cap, int m,
                                                              int k, LWs w) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t sh_last, sh_bin, sh_above;
  const int64_t row = blockIdx.y;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  if (V <= k) return;  // everything visible is selected; pass 2 writes it
  const int start = blockIdx.x * kTopkSlice;
  if (start >= V) return;
  const int end = min(V, start + kTopkSlice);
  const int ngroups = (V + kTopkSlice - 1) / kTopkSlice;
  for (int i = threadIdx.x; i < kBins; i += kLThreads) lh[i] = 0;
  __syncthreads();
  const float* srow = scores + row * n_cap;
  for (int i = start + threadIdx.x; i < end; i += kLThreads) atomicAdd(&lh[float_key(srow[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + row * kBins;
  for (int i = threadIdx.x; i < kBins; i += kLThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&w.ctl[row].done1, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (uint32_t)(ngroups - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  for (int i = threadIdx.x; i < kBins; i += kLThreads) lh[i] = ld_agent(&gh[i]);
  __syncthreads();
  find_threshold_bin(lh, kBins, (uint32_t)k, tmp, &sh_bin, &sh_above);
  if (threadIdx.x == 0) {
    w.ctl[row].bin = sh_bin;
    w.ctl[row].krem = (uint32_t)k - sh_above;
  }
}

// Radix-select the krem-th largest element of `c` (n candidates) whose key bits
// above `lowbits` all equal the threshold bin; returns (key, index) bounds.
__device__ void resolve_candidates(const uint2* c, uint32_t n, uint32_t krem, uint32_t* hist /*[256]*/,
                                   uint32_t* tmp, uint32_t* sh, uint32_t* out_key, uint32_t* out_idx) {
  // key digits: bits 19..12, 11..4, 3..0
  uint32_t prefix = 0, mask = 0;
  const int shifts[3] = {12, 4, 0};
  const uint32_t widths[3] = {0xffu, 0xffu, 0xfu};
  for (int p = 0; p < 3; ++p) {
    const int sh_ = shifts[p];
    hist[threadIdx.x] = 0;  // 256 threads, 256 bins
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kLThreads) {
      const uint32_t key = c[i].x & 0xfffffu;
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh_) & widths[p]], 1u);
    }
    __syncthreads();
    find_threshold_bin(hist, 256, krem, tmp, &sh[0], &sh[1]);
    prefix |= sh[0] << sh_;
    mask |= widths[p] << sh_;
    krem -= sh[1];
    __syncthreads();
  }
  // prefix = low 20 bits of the threshold key; krem copies of it are taken,
  // lowest indices first.  Count copies; when all are taken skip the index passes.
  uint32_t cnt = 0;
  for (uint32_t i = threadIdx.x; i < n; i += kLThreads) cnt += (c[i].x & 0xfffffu) == prefix;
  uint32_t tot;
  block_incl_scan(cnt, tmp, &tot);
  uint32_t idx_bound = 0xffffffffu;  // take every copy with index <= idx_bound
  if (tot != krem) {
    // krem-th smallest index among the copies == krem-th largest of ~index
    uint32_t ip = 0, im = 0;
    for (int p = 0; p < 4; ++p) {
      const int sh_ = 24 - 8 * p;
      hist[threadIdx.x] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n; i += kLThreads) {
        if ((c[i].x & 0xfffffu) != prefix) continue;
        const uint32_t inv = ~c[i].y;
        if ((inv & im) == ip) atomicAdd(&hist[(inv >> sh_) & 0xffu], 1u);
      }
      __syncthreads();
      find_threshold_bin(hist, 256, krem, tmp, &sh[0], &sh[1]);
      ip |= sh[0] << sh_;
      im |= 0xffu << sh_;
      krem -= sh[1];
      __syncthreads();
    }
    idx_bound = ~ip;
  }
  *out_key = prefix;
  *out_idx = idx_bound;
}

__global__ __launch_bounds__(kLThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                                const int32_t* __restrict__ q_pos, int n_cap, int m,
                                                                int k, LWs w, int32_t* __restrict__ idx) {
  __shared__ uint2 cl[kCandLds];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t sh_last;
  const int64_t row = blockIdx.y;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < k; i += kLThreads) out[i] = i < V ? i : -1;
    return;
  }
  const int start = blockIdx.x * kTopkSlice;
  if (start >= V) return;
  const int end = min(V, start + kTopkSlice);
  const int ngroups = (V + kTopkSlice - 1) / kTopkSlice;
  const uint32_t bin = w.ctl[row].bin;
  const float* srow = scores + row * n_cap;
  uint32_t* bm = w.bitmap + row * (int64_t)w.words;
  uint2* cand = w.cand + row * (int64_t)n_cap;
  const int lane = threadIdx.x % kWave;
  for (int base = start + (threadIdx.x / kWave) * kWave; base < end; base += kLThreads) {
    const int i = base + lane;
    const uint32_t key = i < end ? float_key(srow[i]) : 0u;
    const uint32_t kb = key >> 20;
    const bool above = i < end && kb > bin;
    const bool isc = i < end && kb == bin;
    const uint64_t am = __ballot(above);
    const uint64_t cm = __ballot(isc);
    if (lane == 0) {
      bm[base / 32] = (uint32_t)am;
      bm[base / 32 + 1] = (uint32_t)(am >> 32);
    }
    if (cm) {
      uint32_t cbase = 0;
      if (lane == 0) cbase = atomicAdd(&w.ctl[row].cand_count, (uint32_t)__popcll(cm));
      cbase = __shfl(cbase, 0);
      if (isc) {
        const uint32_t r = (uint32_t)__popcll(cm & ((1ull << lane) - 1ull));
        cand[cbase + r] = make_uint2(key, (uint32_t)i);
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&w.ctl[row].done2, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (uint32_t)(ngroups - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  // ---- last workgroup of the row: resolve the threshold bin's candidates
  const uint32_t n = ld_agent(&w.ctl[row].cand_count);
  const uint32_t krem = ld_agent(&w.ctl[row].krem);
  const uint2* src = cand;
  if (n <= (uint32_t)kCandLds) {
    for (uint32_t i = threadIdx.x; i < n; i += kLThreads) {
      uint2 v;
      v.x = ld_agent(&cand[i].x);
      v.y = ld_agent(&cand[i].y);
      cl[i] = v;
    }
    __syncthreads();
    src = cl;
  }
  uint32_t tkey, tidx;
  resolve_candidates(src, n, krem, hist, tmp, sh, &tkey, &tidx);
  for (uint32_t i = threadIdx.x; i < n; i += kLThreads) {
    const uint2 v = src[i];
    const uint32_t lk = v.x & 0xfffffu;
    if (lk > tkey || (lk == tkey && v.y <= tidx)) atomicOr(&bm[v.y >> 5], 1u << (v.y & 31));
  }
  __threadfence();
  __syncthreads();
  // ---- compact the bitmap of [0, V) into ascending indices
  const int nw = (V + 31) / 32;
  const int per = (nw + kLThreads - 1) / kLThreads;
  const int w0 = min(nw, (int)threadIdx.x * per), w1 = min(nw, w0 + per);
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(ld_agent(&bm[i]));
  uint32_t pos = block_incl_scan(cnt, tmp, nullptr) - cnt;
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = ld_agent(&bm[i]);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = i * 32 + b;
      ++pos;
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int n_cap, int k) {
  (void)k;
  if (n_cap <= kTopkLdsMax) return 0;
  const size_t words = (size_t)(n_cap + 63) / 64 * 2;
  return align256((size_t)rows * kBins * 4) + align256((size_t)rows * sizeof(RowCtl)) +
         align256((size_t)rows * n_cap * 8) + align256((size_t)rows * words * 4);
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int batch, int tq, int n_cap, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)batch * tq;
  if (rows == 0) return hipSuccess;
  if (n_cap <= kTopkLdsMax) {
    const size_t lds = (size_t)max(n_cap, 1) * 4;
    hipLaunchKernelGGL(topk_lds_kernel, dim3((unsigned)rows), dim3(kLdsThreads), lds, s, scores, q_pos, n_cap, m, k,
                       idx);
    return hipGetLastError();
  }
  LWs w = carve(ws, rows, n_cap);
  const int64_t nclear = rows * kBins;
  const unsigned cgrid = (unsigned)std::min<int64_t>((nclear + 255) / 256, 1024);
  hipLaunchKernelGGL(topk_clear_kernel, dim3(cgrid), dim3(256), 0, s, w, rows);
  dim3 grid((n_cap + kTopkSlice - 1) / kTopkSlice, (unsigned)rows);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kLThreads), 0, s, scores, q_pos, n_cap, m, k, w);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(kLThreads), 0, s, scores, q_pos, n_cap, m, k, w, idx);
  return hipGetLastError();
}

}  // namespace csa

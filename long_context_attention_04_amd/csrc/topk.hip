// (c) Per-query top-k selection of compressed blocks.
//
// The indexer's scores pick the k compressed blocks each query attends to
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
//  * Longer rows (1M-token decode: 262,144 blocks per row and only 8 rows):
//    two kernels and no communication between workgroups of one kernel
//    (on this chip a device-scope fence writes back / invalidates the XCD's
//    L2 and returning atomics go to the memory-side unit, so "last workgroup"
//    tricks cost far more than a kernel boundary).  Pass 1: every 4096-block
//    slice of a row selects its own exact top-C in LDS (C = 128 for 64
//    slices) and writes it in ascending index order together with its C-th
//    element.  Pass 2: one workgroup per row selects the top-k of the ~8192
//    candidates in LDS; candidate order is ascending index order, so the
//    compaction needs no sort.  The result is exact whenever no truncated
//    slice had its C-th kept element selected (then nothing it dropped can
//    be selected); otherwise the workgroup selects from the whole row itself.
#include "common.h"
#include "kernels.h"
#include "select.h"

#include <algorithm>

namespace csa {

namespace {

__device__ void load_keys(const float* __restrict__ src, int n, uint32_t* keys) {
  const bool vec = (((uintptr_t)src) & 15) == 0;
  const int n4 = vec ? n / 4 : 0;
  for (int base = threadIdx.x; base < n4; base += 8 * blockDim.x) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * blockDim.x;
      if (i < n4) v[j] = ((const float4*)src)[i];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * blockDim.x;
      if (i < n4) {
        keys[4 * i] = float_key(v[j].x);
        keys[4 * i + 1] = float_key(v[j].y);
        keys[4 * i + 2] = float_key(v[j].z);
        keys[4 * i + 3] = float_key(v[j].w);
      }
    }
  }
  for (int i = 4 * n4 + threadIdx.x; i < n; i += blockDim.x) keys[i] = float_key(src[i]);
  __syncthreads();
}

// ------------------------------------------------------------------ LDS path
constexpr int kLdsThreads = 512;

__global__ __launch_bounds__(kLdsThreads) void topk_lds_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ q_pos, int n_cap, int m,
                                                               int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t keys[];
  __shared__ SelShared sh;
  const int64_t row = blockIdx.x;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kLdsThreads) out[i] = i < V ? i : -1;
    return;
  }
  load_keys(scores + row * n_cap, V, keys);
  auto key = [&](int i) { return keys[i]; };
  uint32_t T, krem;
  radix_threshold(key, V, k, sh, &T, &krem);
  compact_selected(key, V, T, krem, sh, [&](int pos, uint32_t r) {
    if (r < (uint32_t)k) out[r] = pos;
  });
}

// ------------------------------------------------------------------ long rows
constexpr int kSlice = kTopkSlice;  // keys per candidate workgroup
constexpr int kCandThreads = 256;
constexpr int kMergeThreads = 1024;
constexpr int kMergeCap = 8192;     // candidates a merge workgroup holds in LDS


__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ __launch_bounds__(kCandThreads) void topk_cand_kernel(const float* __restrict__ scores,
                                                                 const int32_t* __restrict__ q_pos, int n_cap, int m,
                                                                 int k, int C, int nslices, uint2* __restrict__ cand,
                                                                 SliceMeta* __restrict__ meta) {
  __shared__ uint32_t keys[kSlice];
  __shared__ SelShared sh;
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  SliceMeta* mt = meta + row * nslices + g;
  if (V <= k) return;  // the merge writes every visible index
  const int start = g * kSlice;
  const int n = max(0, min(kSlice, V - start));
  uint2* out = cand + (row * nslices + g) * C;
  if (n == 0) {
    if (threadIdx.x == 0) *mt = SliceMeta{0u, 0u, 0u, 0u};
    return;
  }
  load_keys(scores + row * n_cap + start, n, keys);
  if (n <= C) {
    for (int i = threadIdx.x; i < n; i += kCandThreads) out[i] = make_uint2(keys[i], (uint32_t)(start + i));
    if (threadIdx.x == 0) *mt = SliceMeta{(uint32_t)n, 0u, 0u, 0u};
    return;
  }
  auto key = [&](int i) { return keys[i]; };
  uint32_t T, krem;
  radix_threshold(key, n, C, sh, &T, &krem);
  compact_selected(key, n, T, krem, sh, [&](int pos, uint32_t r) {
    if (r < (uint32_t)C) out[r] = make_uint2(keys[pos], (uint32_t)(start + pos));
  });
  // the C-th kept element in (key desc, index asc) order is the last copy of T taken
  if (threadIdx.x == 0) *mt = SliceMeta{(uint32_t)C, 1u, T, (uint32_t)(start + sh.last_pos)};
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const float* __restrict__ scores,
                                                                   const int32_t* __restrict__ q_pos, int n_cap,
                                                                   int m, int k, int C, int nslices, int slice,
                                                                   const uint2* __restrict__ cand,
                                                                   const SliceMeta* __restrict__ meta,
                                                                   int32_t* __restrict__ idx) {
  __shared__ uint32_t ck[kMergeCap];
  __shared__ uint32_t ci[kMergeCap];
  __shared__ uint32_t offs[kMergeCap / 16 + 1];
  __shared__ uint32_t cnts[kMergeCap / 16 + 1];
  __shared__ SelShared sh;
  __shared__ uint32_t bad;
  const int64_t row = blockIdx.x;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kMergeThreads) out[i] = i < V ? i : -1;
    return;
  }
  const float* srow = scores + row * n_cap;
  const int ns = (V + slice - 1) / slice;
  bool full = C == 0;
  if (!full) {
    // gather the slices' lists in slice order (= ascending index order)
    const SliceMeta* mr = meta + row * nslices;
    const uint32_t cnt = threadIdx.x < ns ? mr[threadIdx.x].count : 0u;
    uint32_t tot;
    const uint32_t incl = block_incl_scan(cnt, sh.tmp, &tot);
    if (threadIdx.x < ns) offs[threadIdx.x] = incl - cnt;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int M = (int)tot;
    if (threadIdx.x < ns) cnts[threadIdx.x] = cnt;
    __syncthreads();
    // A row that sees fewer blocks than the capacity has fewer slices: when its
    // candidates are not more than k (and some slice was truncated, since V > k),
    // they cannot decide the selection; the whole row does.
    if (M <= k) full = true;
  }
  if (!full) {
    const SliceMeta* mr = meta + row * nslices;
    const uint2* src = cand + row * nslices * C;
    const uint32_t tot = (uint32_t)(offs[ns - 1] + cnts[ns - 1]);
    const int M = (int)tot;
    const int total = ns * C;  // <= kMergeCap
    for (int base = threadIdx.x; base < total; base += 8 * kMergeThreads) {
      uint2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = base + j * kMergeThreads;
        v[j] = (p < total && (uint32_t)(p % C) < cnts[p / C]) ? src[p] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = base + j * kMergeThreads;
        if (p < total && (uint32_t)(p % C) < cnts[p / C]) {
          const uint32_t o = offs[p / C] + p % C;
          ck[o] = v[j].x;
          ci[o] = v[j].y;
        }
      }
    }
    __syncthreads();
    auto key = [&](int i) { return ck[i]; };
    uint32_t T, krem;
    radix_threshold(key, M, k, sh, &T, &krem);
    sh.last_pos = 0;
    __syncthreads();
    compact_selected(key, M, T, krem, sh, [&](int pos, uint32_t r) {
      if (r < (uint32_t)k) out[r] = (int32_t)ci[pos];
    });
    // exact unless a truncated slice had its C-th kept element selected
    const uint32_t jT = ci[sh.last_pos];
    if (threadIdx.x < ns) {
      const SliceMeta mm = mr[threadIdx.x];
      if (mm.trunc && (mm.last_key > T || (mm.last_key == T && mm.last_idx <= jT))) bad = 1;
    }
    __syncthreads();
    full = bad != 0;
  }
  if (full) {  // select from the whole row (slow path; any input)
    auto key = [&](int i) { return float_key(srow[i]); };
    uint32_t T, krem;
    radix_threshold(key, V, k, sh, &T, &krem);
    compact_selected(key, V, T, krem, sh, [&](int pos, uint32_t r) {
      if (r < (uint32_t)k) out[r] = pos;
    });
  }
}

// Pass 1, one wave per 1024-key slice: the slice's exact top-32 by a one-wave
// radix select (no workgroup barrier), written in ascending index order.
constexpr int kSlice32 = kWaveTopN * kWave;  // 1024
static_assert(kSlice32 == kFusedSlice && kWaveTopC == kFusedC, "one candidate format for both passes");

__global__ __launch_bounds__(256) void topk_cand32_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ q_pos, int n_cap, int m, int k,
                                                          int nslices, uint2* __restrict__ cand,
                                                          SliceMeta* __restrict__ meta) {
  __shared__ WaveSelLds sl[4];
  const int64_t row = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), L = threadIdx.x % kWave;
  const int g = blockIdx.x * 4 + w;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  if (V <= k || g >= nslices) return;  // V <= k: the merge writes every visible index
  const int start = g * kSlice32;
  const int n = max(0, min(kSlice32, V - start));
  SliceMeta* mt = meta + row * nslices + g;
  uint2* out = cand + (row * nslices + g) * kWaveTopC;
  // lane L: positions 16L .. 16L+15 (64 contiguous bytes)
  const float* src = scores + row * n_cap + start + kWaveTopN * L;
  uint32_t kv[kWaveTopN];
  const bool vec = ((((uintptr_t)(scores + row * n_cap + start)) & 15) == 0) && kWaveTopN * L + kWaveTopN <= n;
  if (vec) {
#pragma unroll
    for (int q = 0; q < kWaveTopN / 4; ++q) {
      const float4 f = ((const float4*)src)[q];
      kv[4 * q] = float_key(f.x);
      kv[4 * q + 1] = float_key(f.y);
      kv[4 * q + 2] = float_key(f.z);
      kv[4 * q + 3] = float_key(f.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) kv[j] = kWaveTopN * L + j < n ? float_key(src[j]) : 0u;
  }
  if (n <= kWaveTopC) {  // every slot of the slice's list: its n keys, then empty (key 0) slots
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) {
      const int p = kWaveTopN * L + j;
      if (p < kWaveTopC) out[p] = p < n ? make_uint2(kv[j], (uint32_t)(start + p)) : make_uint2(0u, 0u);
    }
    if (L == 0) *mt = SliceMeta{(uint32_t)n, 0u, 0u, 0u};
    return;
  }
  uint32_t T, tpos;
  wave_top32(kv, sl[w], &T, &tpos);
  if (L < kWaveTopC) {  // one coalesced store of the list
    const uint2 e = sl[w].res[L];
    out[L] = make_uint2(e.x, (uint32_t)start + e.y);
  }
  if (L == 0) *mt = SliceMeta{(uint32_t)kWaveTopC, 1u, T, (uint32_t)start + tpos};
}

// Pass 2 of the 1024-slice scheme, one 1024-thread workgroup per row: slice s's
// list fills slots 32s .. 32s+31 (empty slots hold key 0), so slot order is
// ascending index order and thread t holds slots 8t .. 8t+7 in registers.  The
// threshold is found on the registers, the compaction is one block scan, and
// the exactness certificate is the same as above.
constexpr int kM32PerThread = kMergeCap / kRegSelThreads;  // 8
static_assert(kM32PerThread * kRegSelThreads == kMergeCap && kWaveTopC % kM32PerThread == 0, "slot tiling");

__global__ __launch_bounds__(kRegSelThreads) void topk_merge32_kernel(const float* __restrict__ scores,
                                                                     const int32_t* __restrict__ q_pos, int n_cap,
                                                                     int m, int k, int nslices,
                                                                     const uint2* __restrict__ cand,
                                                                     const SliceMeta* __restrict__ meta,
                                                                     int32_t* __restrict__ idx) {
  __shared__ RegSelLds rs;
  __shared__ SelShared sh;
  __shared__ uint32_t ostage[kMergeCap + kRegSelThreads];  // selected indices by rank, then discard slots
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  // The candidate lists and the slices' metadata are loaded together with the row's
  // position (their addresses do not depend on it: one memory round trip); the slots
  // of slices past the visible ones are cleared once it is known.
  const int qpos = q_pos[row];
  SliceMeta mm{0u, 0u, 0u, 0u};
  if (t < nslices) mm = meta[row * nslices + t];
  uint32_t kv[kM32PerThread], iv[kM32PerThread];
  if (kM32PerThread * t < nslices * kWaveTopC) {
    const uint4* src = (const uint4*)(cand + row * nslices * kWaveTopC) + (kM32PerThread / 2) * t;
#pragma unroll
    for (int q = 0; q < kM32PerThread / 2; ++q) {
      const uint4 v = src[q];
      kv[2 * q] = v.x;
      iv[2 * q] = v.y;
      kv[2 * q + 1] = v.z;
      iv[2 * q + 1] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kM32PerThread; ++j) kv[j] = iv[j] = 0u;
  }
  const int V = min(visible_blocks(qpos, m), n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    for (int i = t; i < k; i += kRegSelThreads) out[i] = i < V ? i : -1;
    return;
  }
  const int ns = (V + kSlice32 - 1) / kSlice32;  // slices holding visible keys
  if (t >= ns) mm = SliceMeta{0u, 0u, 0u, 0u};
  if (kM32PerThread * t >= ns * kWaveTopC) {
#pragma unroll
    for (int j = 0; j < kM32PerThread; ++j) kv[j] = iv[j] = 0u;
  }
  uint32_t lo, hi, M;
  block_key_range(kv, rs, &lo, &hi, &M);
  // A row that sees fewer blocks than the capacity has fewer slices: when its
  // candidates are not more than k (and some slice was truncated, since V > k),
  // they cannot decide the selection; the whole row does.
  bool full = M <= (uint32_t)k;
  if (!full) {
    uint32_t T, krem;
    block_threshold_regs(kv, lo, hi, (uint32_t)k, rs, &T, &krem);
    // compaction in slot order: one scan of (keys > T) | (copies of T) << 16
    uint32_t gtc = 0, eqc = 0;
#pragma unroll
    for (int j = 0; j < kM32PerThread; ++j) {
      gtc += kv[j] > T;
      eqc += kv[j] == T;
    }
    const uint32_t packed = gtc | (eqc << 16);
    uint32_t tot;
    const uint32_t excl = block_scan_regsel(packed, rs.scan[2], &tot) - packed;
    krem = min(krem, tot >> 16);  // "every copy" made a count
    uint32_t eq_seen = excl >> 16;
    uint32_t r = (excl & 0xffffu) + min(eq_seen, krem);
    // the k indices go to LDS (rank order), unwanted stores to this thread's discard
    // slot, then out in one coalesced pass
    uint32_t my_jT = 0;
    bool has_t = false;
#pragma unroll
    for (int j = 0; j < kM32PerThread; ++j) {
      const bool is_eq = kv[j] == T;
      const bool keep = kv[j] > T || (is_eq && eq_seen < krem);
      const bool last = is_eq && eq_seen == krem - 1u;  // the last copy of T taken
      my_jT = last ? iv[j] : my_jT;
      has_t = has_t || last;
      eq_seen += is_eq;
      ostage[keep && r < (uint32_t)k ? r : (uint32_t)kMergeCap + t] = iv[j];
      r += keep;
    }
    if (has_t) rs.jT = my_jT;
    __syncthreads();
    for (int i = t; i < k; i += kRegSelThreads) out[i] = (int32_t)ostage[i];
    // exact unless a truncated slice had its 32nd kept element selected
    const uint32_t jT = rs.jT;
    if (t < ns && mm.trunc && (mm.last_key > T || (mm.last_key == T && mm.last_idx <= jT))) rs.bad = 1u;
    __syncthreads();
    full = rs.bad != 0u;
  }
  if (full) {  // select from the whole row (slow path; any input)
    const float* srow = scores + row * n_cap;
    auto key = [&](int i) { return float_key(srow[i]); };
    uint32_t T, krem;
    radix_threshold(key, V, k, sh, &T, &krem);
    compact_selected(key, V, T, krem, sh, [&](int pos, uint32_t r) {
      if (r < (uint32_t)k) out[r] = pos;
    });
  }
}

// C for a row length: the merge holds nslices * C candidates in LDS.
__host__ inline int cand_per_slice(int n_cap, int k) {
  const int ns = (n_cap + kSlice - 1) / kSlice;
  int C = kMergeCap / ns;
  if (C > 128) C = 128;
  if (C < 16 || ns > kMergeThreads || (int64_t)ns * C < k) return 0;  // whole-row path
  return C;
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int n_cap, int k) {
  if (n_cap <= kTopkLdsMax) return 0;
  const int ns = (n_cap + kSlice - 1) / kSlice;
  const int C = cand_per_slice(n_cap, k);
  const size_t wide = align256((size_t)rows * ns * sizeof(SliceMeta)) + align256((size_t)rows * ns * (C > 0 ? C : 1) * 8);
  const int ns32 = (n_cap + kSlice32 - 1) / kSlice32;
  const size_t narrow = align256((size_t)rows * ns32 * sizeof(SliceMeta)) + align256((size_t)rows * ns32 * kWaveTopC * 8);
  return std::max(wide, narrow);
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int batch, int tq, int n_cap, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)batch * tq;
  if (rows == 0) return hipSuccess;
  if (n_cap <= kTopkLdsMax) {
    const size_t lds = (size_t)std::max(n_cap, 1) * 4;
    hipLaunchKernelGGL(topk_lds_kernel, dim3((unsigned)rows), dim3(kLdsThreads), lds, s, scores, q_pos, n_cap, m, k,
                       idx);
    return hipGetLastError();
  }
  {
    const int ns32 = (n_cap + kSlice32 - 1) / kSlice32;
    if (ns32 <= kMergeThreads && ns32 * kWaveTopC <= kMergeCap && ns32 * kWaveTopC >= k) {
      SliceMeta* meta = (SliceMeta*)ws;
      uint2* cand = (uint2*)((char*)ws + align256((size_t)rows * ns32 * sizeof(SliceMeta)));
      hipLaunchKernelGGL(topk_cand32_kernel, dim3((unsigned)((ns32 + 3) / 4), (unsigned)rows), dim3(256), 0, s, scores,
                         q_pos, n_cap, m, k, ns32, cand, meta);
      hipLaunchKernelGGL(topk_merge32_kernel, dim3((unsigned)rows), dim3(kRegSelThreads), 0, s, scores, q_pos, n_cap,
                         m, k, ns32, cand, meta, idx);
      return hipGetLastError();
    }
  }
  const int ns = (n_cap + kSlice - 1) / kSlice;
  const int C = cand_per_slice(n_cap, k);
  SliceMeta* meta = (SliceMeta*)ws;
  uint2* cand = (uint2*)((char*)ws + align256((size_t)rows * ns * sizeof(SliceMeta)));
  if (C > 0)
    hipLaunchKernelGGL(topk_cand_kernel, dim3(ns, (unsigned)rows), dim3(kCandThreads), 0, s, scores, q_pos, n_cap, m,
                       k, C, ns, cand, meta);
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, s, scores, q_pos, n_cap, m, k, C,
                     ns, kSlice, cand, meta, idx);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused with the indexer
namespace {
__host__ inline int fused_slices(int n_cap) { return (n_cap + kFusedSlice - 1) / kFusedSlice; }
}  // namespace

bool index_topk_fused_ok(const IndexArgs& a, int k) {
  // MXFP4 keys (the indexer that emits candidates), long rows, and a candidate set that
  // fits the merge pass: nslices * 32 entries in LDS, one thread per slice for the scan
  const int ns = fused_slices(a.n_cap);
  return a.k.dtype == CSA_MXFP4 && a.n_cap > kTopkLdsMax && ns <= kMergeThreads &&
         (int64_t)ns * kFusedC <= kMergeCap && (int64_t)ns * kFusedC >= k;
}

size_t index_topk_workspace_bytes(int64_t rows, int n_cap, int k) {
  if (n_cap <= kTopkLdsMax) return 0;
  const int ns = fused_slices(n_cap);
  return align256((size_t)rows * ns * sizeof(SliceMeta)) + align256((size_t)rows * ns * kFusedC * 8);
}

namespace {
CandOut fused_cand_out(const IndexArgs& a, int k, void* ws) {
  const int64_t rows = (int64_t)a.batch * a.tq;
  const int ns = fused_slices(a.n_cap);
  CandOut co;
  co.C = kFusedC;
  co.slice = kFusedSlice;
  co.nslices = ns;
  co.k = k;
  co.meta = (SliceMeta*)ws;
  co.cand = (uint2*)((char*)ws + align256((size_t)rows * ns * sizeof(SliceMeta)));
  return co;
}
}  // namespace

hipError_t launch_index_topk_cand(const IndexArgs& a, int k, void* ws, hipStream_t s, const FusedCompress* fc) {
  if ((int64_t)a.batch * a.tq == 0) return hipSuccess;
  return launch_index_scores_cand(a, fused_cand_out(a, k, ws), s, fc);
}

hipError_t launch_index_topk_merge(const IndexArgs& a, int k, int32_t* idx, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.tq;
  if (rows == 0) return hipSuccess;
  const CandOut co = fused_cand_out(a, k, ws);
  hipLaunchKernelGGL(topk_merge32_kernel, dim3((unsigned)rows), dim3(kRegSelThreads), 0, s, a.scores, a.q_pos,
                     a.n_cap, a.m, k, co.nslices, co.cand, co.meta, idx);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexArgs& a, int k, int32_t* idx, void* ws, hipStream_t s) {
  const hipError_t e = launch_index_topk_cand(a, k, ws, s);
  if (e != hipSuccess) return e;
  return launch_index_topk_merge(a, k, idx, ws, s);
}

}  // namespace csa

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

// Wave-wide min / max of a uint32 with DPP row ops (VALU, no LDS round trip):
// reduce within each 16-lane row, then combine the four rows via readlane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  // quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

struct SelShared {
  uint32_t hist[2][256];
  uint32_t tmp[16];
  uint32_t tmn[16], tmx[16];
  uint32_t bin, above, cnt, last_pos;
  uint32_t nfin;
  __attribute__((aligned(16))) uint32_t fkey[64];
  __attribute__((aligned(16))) uint32_t fpos[64];
  uint32_t T, krem;
};

// Exact threshold of the top-k of n keys (key(i) for i < n, tie order = i
// ascending; 1 <= k < n): the k-th largest key T and the number krem of its
// copies that are taken (the lowest-positioned ones).
// Radix select over the live key range: each pass splits the current range
// [lo, hi] into <= 256 equal bins (not fixed digits, so scores that share
// their top bits still spread out), keeps the bin holding the k-th key, and
// stops as soon as that bin holds <= 64 keys, which one wave then ranks
// exactly by (key desc, position asc).
template <typename KeyFn>
__device__ void radix_threshold(KeyFn key, int n, int k, SelShared& sh, uint32_t* T_out, uint32_t* krem_out) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
  // key range
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int base = threadIdx.x; base < n; base += 8 * blockDim.x) {
    uint32_t kv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * blockDim.x;
      kv[j] = i < n ? key(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (base + j * (int)blockDim.x < n) {
        mn = min(mn, kv[j]);
        mx = max(mx, kv[j]);
      }
  }
  mn = wave_reduce_u32<false>(mn);
  mx = wave_reduce_u32<true>(mx);
  if (lane == 0) {
    sh.tmn[wv] = mn;
    sh.tmx[wv] = mx;
  }
  for (int i = threadIdx.x; i < 512; i += blockDim.x) (&sh.hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t lo = sh.tmn[0], hi = sh.tmx[0];
  for (int i = 1; i < nw; ++i) {
    lo = min(lo, sh.tmn[i]);
    hi = max(hi, sh.tmx[i]);
  }
  uint32_t krem = (uint32_t)k;
  bool finish = false;
  for (int pass = 0; pass < 5 && !finish; ++pass) {
    const uint32_t span = hi - lo;
    if (span == 0) break;  // every key left in range is equal: T = lo
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    uint32_t* hist = sh.hist[pass & 1];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[(pass + 1) & 1][i] = 0;
    for (int base = threadIdx.x; base < n; base += 8 * blockDim.x) {
      uint32_t kv[8];  // all loads first: one memory latency per 8 keys when key() reads memory
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * blockDim.x;
        kv[j] = i < n ? key(i) : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * blockDim.x;
        if (i < n && kv[j] >= lo && kv[j] <= hi) atomicAdd(&hist[(kv[j] - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {  // one wave: lane L owns bins 4L..4L+3; suffix sums by shuffles
      const int L = threadIdx.x;
      const uint32_t h0 = hist[4 * L], h1 = hist[4 * L + 1], h2 = hist[4 * L + 2], h3 = hist[4 * L + 3];
      const uint32_t mine = h0 + h1 + h2 + h3;
      uint32_t suf = mine;  // inclusive suffix over lanes >= L
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t u = __shfl_down(suf, o);
        if (L + o < kWave) suf += u;
      }
      uint32_t run = suf - mine;  // keys in bins above this lane's four
      const uint32_t hh[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int d = 3; d >= 0; --d) {
        if (run < krem && run + hh[d] >= krem) {
          sh.bin = 4 * L + d;
          sh.above = run;
          sh.cnt = hh[d];
        }
        run += hh[d];
      }
      if (L == 0) sh.nfin = 0;
    }
    __syncthreads();
    const uint32_t nlo = lo + (sh.bin << shift);
    const uint32_t nhi = min(hi, nlo + ((1u << shift) - 1u));
    krem -= sh.above;
    finish = sh.cnt <= 64;
    lo = nlo;
    hi = nhi;
  }
  if (finish && hi != lo) {
    // gather the <= 64 keys of [lo, hi] with their positions, then rank them in one wave
    for (int base = threadIdx.x; base < n; base += 8 * blockDim.x) {
      uint32_t kv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * blockDim.x;
        kv[j] = i < n ? key(i) : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + j * blockDim.x;
        if (i < n && kv[j] >= lo && kv[j] <= hi) {
          const uint32_t slot = atomicAdd(&sh.nfin, 1u);
          sh.fkey[slot] = kv[j];
          sh.fpos[slot] = (uint32_t)i;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {  // one wave ranks the <= 64 gathered keys (broadcast reads, 8 at a time)
      const int c = (int)sh.nfin, L = threadIdx.x;
      for (int i = c + L; i < 64; i += kWave) {  // pad to whole groups of 8 with keys that never rank
        sh.fkey[i] = 0u;
        sh.fpos[i] = 0xffffffffu;
      }
      const uint32_t myk = L < c ? sh.fkey[L] : 0u, myp = L < c ? sh.fpos[L] : 0xffffffffu;
      uint32_t rank = 0, gt = 0;
      for (int i0 = 0; i0 < c; i0 += 8) {
        const uint4 k0 = *(const uint4*)&sh.fkey[i0], k1 = *(const uint4*)&sh.fkey[i0 + 4];
        const uint4 p0 = *(const uint4*)&sh.fpos[i0], p1 = *(const uint4*)&sh.fpos[i0 + 4];
        const uint32_t kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        const uint32_t pp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          rank += kk[j] > myk || (kk[j] == myk && pp[j] < myp);
          gt += kk[j] > myk;
        }
      }
      if (L < c && rank == krem - 1) {
        sh.T = myk;
        sh.krem = krem - gt;
      }
    }
    __syncthreads();
    *T_out = sh.T;
    *krem_out = sh.krem;
    return;
  }
  *T_out = lo;  // range collapsed to one key value: take krem copies of it
  *krem_out = krem;
}

// Ascending-order compaction of the selected positions (key > T, or key == T
// among the first krem copies).  emit(pos, rank) is called once per selected
// position with its rank 0..k-1.  Sets sh.last_pos to the position of the last
// copy of T taken.  Each wave owns a contiguous chunk and walks it 64 keys per
// step (lane i <-> key base+i, conflict-free); ballots give in-wave ranks and
// one barrier gives every wave its offsets.
template <typename KeyFn, typename Emit>
__device__ void compact_selected(KeyFn key, int n, uint32_t T, uint32_t krem, SelShared& sh, Emit emit) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int chunk = (n + nw * kWave - 1) / (nw * kWave) * kWave;  // whole 64-key steps per wave
  const int lo = min(n, wv * chunk), hi = min(n, lo + chunk);
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t gt = 0, eq = 0;
  for (int b0 = lo; b0 < hi; b0 += 4 * kWave) {
    uint32_t kv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = b0 + j * kWave + lane;
      kv[j] = i < hi ? key(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = b0 + j * kWave + lane;
      gt += (uint32_t)__popcll(__ballot(i < hi && kv[j] > T));
      eq += (uint32_t)__popcll(__ballot(i < hi && kv[j] == T));
    }
  }
  if (lane == 0) {
    sh.tmn[wv] = gt;
    sh.tmx[wv] = eq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wv; ++w) {
    gt_before += sh.tmn[w];
    eq_before += sh.tmx[w];
  }
  uint32_t taken_before = eq_before >= krem ? krem : eq_before;  // copies of T taken by earlier waves
  uint32_t rank = gt_before + taken_before;
  uint32_t eq_seen = eq_before;
  for (int b0 = lo; b0 < hi; b0 += 4 * kWave) {
    uint32_t kvs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = b0 + j * kWave + lane;
      kvs[j] = i < hi ? key(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
    const int i = b0 + j * kWave + lane;
    const uint32_t kv = kvs[j];
    const bool is_eq = i < hi && kv == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t my_eq_rank = eq_seen + (uint32_t)__popcll(eqm & below);  // copies of T before me
    const bool s = (i < hi && kv > T) || (is_eq && my_eq_rank < krem);
    const uint64_t sm = __ballot(s);
    if (s) {
      emit(i, rank + (uint32_t)__popcll(sm & below));
      if (is_eq && my_eq_rank == krem - 1) sh.last_pos = (uint32_t)i;
    }
    rank += (uint32_t)__popcll(sm);
    eq_seen += (uint32_t)__popcll(eqm);
    }
  }
  __syncthreads();
}

// n fp32 scores -> order-preserving keys in LDS; 8 float4 loads in flight per thread.
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

struct SliceMeta {   // per (row, slice)
  uint32_t count;    // candidates written
  uint32_t trunc;    // 1 when the slice held more than C visible keys
  uint32_t last_key; // C-th kept element (the smallest kept in the order)
  uint32_t last_idx;
};

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
                                                                   int m, int k, int C, int nslices,
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
  const int ns = (V + kSlice - 1) / kSlice;
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
    const uint2* src = cand + row * nslices * C;
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
  return align256((size_t)rows * ns * sizeof(SliceMeta)) + align256((size_t)rows * ns * (C > 0 ? C : 1) * 8);
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
  const int ns = (n_cap + kSlice - 1) / kSlice;
  const int C = cand_per_slice(n_cap, k);
  SliceMeta* meta = (SliceMeta*)ws;
  uint2* cand = (uint2*)((char*)ws + align256((size_t)rows * ns * sizeof(SliceMeta)));
  if (C > 0)
    hipLaunchKernelGGL(topk_cand_kernel, dim3(ns, (unsigned)rows), dim3(kCandThreads), 0, s, scores, q_pos, n_cap, m,
                       k, C, ns, cand, meta);
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, s, scores, q_pos, n_cap, m, k, C,
                     ns, cand, meta, idx);
  return hipGetLastError();
}

}  // namespace csa

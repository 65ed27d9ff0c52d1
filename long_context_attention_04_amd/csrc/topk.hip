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
//  * Rows of up to kTopkLdsMax keys.  For k <= 4096 the row is held in registers (16 to
//    40 keys per thread, 512-thread workgroups, two resident per CU, each walking its
//    rows) and selected with value-linear then key-space histograms and one block scan;
//    otherwise one workgroup per row holds it in LDS: radix passes over the live key
//    range, then a block-scan compaction.
//  * Longer rows (the 1M-token decode: 262,144 blocks per row and only 8 rows): two
//    passes and no communication between workgroups of one kernel (on this chip a
//    device-scope fence writes back / invalidates the XCD's L2 and returning atomics
//    go to the memory-side unit, so "last workgroup" tricks cost far more than a kernel
//    boundary).  Pass 1: every 1024-block slice lists its exact top-32, in ascending
//    index order, with its 32nd (key, index) (topk_cand32_kernel from stored scores, or
//    the MXFP4 indexer itself as it scores).  Pass 2: one 1024-thread workgroup per row
//    selects the top-k of the <= 8192 listed candidates in registers; slot order is
//    index order, so the compaction needs no sort.  The result is certified exact
//    whenever no slice had its 32nd listed entry selected (then nothing it left out can
//    be); otherwise the row is selected again over the other lists plus every key of
//    the failing slices (at most 8), or over the whole row.
//  * Rows longer than 262,144 blocks: the same two passes with 4096-block slices listing
//    up to 128 candidates each, merged in LDS (topk_cand_kernel, topk_merge_kernel).
#include "common.h"
#include "kernels.h"
#include "index_fp4.h"
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
constexpr int kMergeCap = 8192;     // candidates a merge workgroup holds in LDS (4096-key slices)
constexpr int kSliceMergeCap = 8192;  // list slots the 1024-slice merge holds (256 slices of 32)


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

// Pass 1 of the 1024-slice scheme, one wave per slice: the slice's candidate list
// (emit_slice_list), from the scores in memory.
constexpr int kSlice32 = kSliceKeys;  // 1024
static_assert(kSlice32 == kFusedSlice && kSliceSlots == kFusedC, "one candidate format for both passes");

__global__ __launch_bounds__(256) void topk_cand32_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ q_pos, int n_cap, int m, int k,
                                                          int nslices, uint2* __restrict__ cand,
                                                          SliceMeta* __restrict__ meta) {
  __shared__ CutLds cl[4];
  const int64_t row = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), L = threadIdx.x % kWave;
  const int g = blockIdx.x * 4 + w;
  const int V = min(visible_blocks(q_pos[row], m), n_cap);
  if (V <= k || g >= nslices) return;  // V <= k: the merge writes every visible index
  const int start = g * kSlice32;
  const int n = max(0, min(kSlice32, V - start));
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
  emit_slice_list(kv, n, (uint32_t)start, cl[w], cand + (row * nslices + g) * kSliceSlots,
                  meta + row * nslices + g);
}

// Pass 2 of the 1024-slice scheme, one 1024-thread workgroup per row: slice s's
// list fills slots 32s .. 32s+31 (empty slots hold key 0), so slot order is
// ascending index order and thread t holds slots 8t .. 8t+7 in registers.  The
// threshold is found on the registers, the compaction is one block scan, and the
// result is certified exact: every key a slice left out ranks after that slice's
// (last_key, last_idx), so the selection is exact unless such a pair is selected.
// When some are (a slice holding more than kSliceSlots of the row's top-k), the
// row is selected again: with the row's scores when the caller kept them; else,
// for at most kMaxBadSlices such slices, from the other slices' lists plus every
// key of those slices rescored with the indexer's arithmetic; else from the whole
// row rescored.  Rows whose full slices hold too few candidates (short rows) are
// selected from their scores, which the indexer wrote to `row_scores`.
// The merge runs 1024-thread workgroups (8 slots per thread): its phases are chains of
// dependent LDS and cross-lane steps, and 16 waves hide more of their latency than 4
// (256 threads of 32 slots: 13.9 us per call against 8.8 us).
constexpr int kMergeThreads32 = 1024;
constexpr int kMPerThread = kSliceMergeCap / kMergeThreads32;  // 8
static_assert(kMPerThread * kMergeThreads32 == kSliceMergeCap && kSliceSlots % kMPerThread == 0, "slot tiling");
constexpr int kMergeMaxSlices = kSliceMergeCap / kSliceSlots;  // 256
static_assert(kMergeMaxSlices % kWave == 0 && kMergeMaxSlices <= kMergeThreads32, "slice flags per wave");
// A failed certificate rescores up to kMaxBadSlices slices into LDS (ostage after
// the query: kBadKeysOffset words, then kSlice32 keys per slice); more rescore the row.
constexpr int kMaxBadSlices = 8;
constexpr int kBadKeysOffset = 512;
static_assert(sizeof(Fp4QueryLds) <= 4 * kBadKeysOffset, "query stage fits below the rescored keys");
// ostage: selected indices by rank, then one discard slot per thread; or the query and
// the rescored slices
constexpr int kMergeStage = std::max(kSliceMergeCap + kMergeThreads32, kBadKeysOffset + kMaxBadSlices * kSlice32);

struct MergeArgs {
  const float* scores;    // the row scores, when the caller keeps them (else nullptr)
  float* row_scores;      // otherwise: [rows][n_cap] scratch rows
  const int32_t* q_pos;
  int n_cap, m, k, nslices;
  const uint2* cand;
  const SliceMeta* meta;
  int32_t* idx;
  int short_rows;         // 1: rows that index_topk_short_row names have their scores in row_scores
  IndexArgs rescore;      // MXFP4 keys to rescore from (rescore.k.data == nullptr: never needed)
};

template <int NR>  // 0: no rescoring; 4 / 16: the indexer's MFMA layout (heads <= 8 / <= 32)
__global__ __launch_bounds__(kMergeThreads32) void topk_merge_slices_kernel(MergeArgs ma) {
  constexpr int TH = kMergeThreads32;
  __shared__ RegSelLds rs;
  __shared__ SelShared sh;
  __shared__ __attribute__((aligned(16))) uint32_t ostage[kMergeStage];
  __shared__ uint64_t badmask[kMergeMaxSlices / kWave];
  __shared__ int badlist[kMaxBadSlices], badstart[kMaxBadSlices];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nslices = ma.nslices, k = ma.k;
  // The candidate lists and the slices' metadata are loaded together with the row's
  // position (their addresses do not depend on it: one memory round trip).
  const int qpos = ma.q_pos[row];
  SliceMeta mm{0u, 0u, 0u, 0u};
  if (t < nslices) mm = ma.meta[row * nslices + t];
  uint32_t kv[kMPerThread], iv[kMPerThread];
  if (kMPerThread * t < nslices * kSliceSlots) {
    const uint4* src = (const uint4*)(ma.cand + row * nslices * kSliceSlots) + (kMPerThread / 2) * t;
    uint4 v[kMPerThread / 2];
#pragma unroll
    for (int q = 0; q < kMPerThread / 2; ++q) v[q] = src[q];
#pragma unroll
    for (int q = 0; q < kMPerThread / 2; ++q) {
      kv[2 * q] = v[q].x;
      iv[2 * q] = v[q].y;
      kv[2 * q + 1] = v[q].z;
      iv[2 * q + 1] = v[q].w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMPerThread; ++j) kv[j] = iv[j] = 0u;
  }
  const int V = min(visible_blocks(qpos, ma.m), ma.n_cap);
  int32_t* out = ma.idx + row * k;
  if (V <= k) {
    for (int i = t; i < k; i += TH) out[i] = i < V ? i : -1;
    return;
  }
  const float* srow = ma.scores ? ma.scores + row * ma.n_cap : ma.row_scores + row * ma.n_cap;
  bool full = ma.short_rows && index_topk_short_row(V, k);
  int nbad = 0;   // slices whose certificate failed
  int sel_n = 0;  // > 0: select from the union of good lists and rescored bad slices
  if (!full) {
    const int ns = (V + kSlice32 - 1) / kSlice32;  // slices holding visible keys
    if (t >= ns) mm = SliceMeta{0u, 0u, 0u, 0u};
    if (kMPerThread * t >= ns * kSliceSlots) {
#pragma unroll
      for (int j = 0; j < kMPerThread; ++j) kv[j] = iv[j] = 0u;
    }
    uint32_t lo, hi, M;
    block_key_range<kMPerThread, TH>(kv, rs, &lo, &hi, &M);
    full = M <= (uint32_t)k;  // too few candidates to decide (rows of a few slices)
    if (!full) {
      uint32_t T, krem;
      block_threshold_regs<kMPerThread, TH>(kv, lo, hi, (uint32_t)k, rs, &T, &krem);
      // compaction in slot order: one scan of (keys > T) | (copies of T) << 16
      uint32_t gtc = 0, eqc = 0;
#pragma unroll
      for (int j = 0; j < kMPerThread; ++j) {
        gtc += kv[j] > T;
        eqc += kv[j] == T;
      }
      const uint32_t packed = gtc | (eqc << 16);
      uint32_t tot;
      const uint32_t excl = block_scan_regsel<TH>(packed, rs.scan[2], &tot) - packed;
      krem = min(krem, tot >> 16);  // "every copy" made a count
      uint32_t eq_seen = excl >> 16;
      uint32_t r = (excl & 0xffffu) + min(eq_seen, krem);
      // the k indices go to LDS (rank order), unwanted stores to this thread's discard
      // slot, then out in one coalesced pass
      if (__builtin_amdgcn_ballot_w64(eqc != 0u) == 0ull) {  // no copy of T in this wave
#pragma unroll
        for (int j = 0; j < kMPerThread; ++j) {
          const bool keep = kv[j] > T;
          ostage[keep && r < (uint32_t)k ? r : (uint32_t)kSliceMergeCap + t] = iv[j];
          r += keep;
        }
      } else {
        uint32_t my_jT = 0;
        bool has_t = false;
#pragma unroll
        for (int j = 0; j < kMPerThread; ++j) {
          const bool is_eq = kv[j] == T;
          const bool keep = kv[j] > T || (is_eq && eq_seen < krem);
          const bool last = is_eq && eq_seen == krem - 1u;  // the last copy of T taken
          my_jT = last ? iv[j] : my_jT;
          has_t = has_t || last;
          eq_seen += is_eq;
          ostage[keep && r < (uint32_t)k ? r : (uint32_t)kSliceMergeCap + t] = iv[j];
          r += keep;
        }
        if (has_t) rs.jT = my_jT;
      }
      __syncthreads();
      // exact unless some slice's (last_key, last_idx) is selected: such slices are
      // "bad" (waves 0-3 cover the <= 256 slices)
      const uint32_t jT = rs.jT;
      const bool isbad = t < ns && mm.trunc && (mm.last_key > T || (mm.last_key == T && mm.last_idx <= jT));
      const uint64_t bm = __builtin_amdgcn_ballot_w64(isbad);
      if (t < kMergeMaxSlices && t % kWave == 0) badmask[t / kWave] = bm;
      __syncthreads();
      nbad = 0;
#pragma unroll
      for (int i = 0; i < kMergeMaxSlices / kWave; ++i) nbad += __builtin_popcountll(badmask[i]);
      full = nbad != 0;
      if (!full)
        for (int i = t; i < k; i += TH) out[i] = (int32_t)ostage[i];
    }
    // With at most kMaxBadSlices bad slices, select over the union of the good slices'
    // lists and every key of the bad slices (read from the kept scores, or rescored into
    // LDS).  Exact: a good slice's omitted keys rank after the candidates' k-th key, and
    // the union's k-th key ranks at or before it.
    if (full && nbad > 0 && nbad <= kMaxBadSlices && (ma.scores || NR > 0)) {
      {
        if (t < nbad) {  // the t-th bad slice (ascending) and its start in the union
          int seen = 0, id = 0;
          for (int i = 0; i < kMergeMaxSlices / kWave; ++i) {
            uint64_t m = badmask[i];
            while (m) {
              if (seen == t) id = kWave * i + __builtin_ctzll(m);
              ++seen;
              m &= m - 1ull;
            }
          }
          badlist[t] = id;
          badstart[t] = kSliceSlots * id + (kSlice32 - kSliceSlots) * t;
        }
        uint32_t* bkeys = ostage + kBadKeysOffset;
        if (ma.scores) {
          __syncthreads();  // the bad-slice list is visible; ostage is free
          for (int i = t; i < nbad * kSlice32; i += TH) {
            const int key = kSlice32 * badlist[i / kSlice32] + i % kSlice32;
            bkeys[i] = key < V ? float_key(srow[key]) : 0u;
          }
          __syncthreads();
        } else if constexpr (NR > 0) {
          fp4_rescore_tiles<NR>(
              ma.rescore, (int)row, V, *(Fp4QueryLds*)ostage, nbad * (kSlice32 / 32),
              [&](int tile) { return kSlice32 * badlist[tile / (kSlice32 / 32)] + 32 * (tile % (kSlice32 / 32)); },
              [&](int tile, int key, float sc, bool live) {
                bkeys[(tile / (kSlice32 / 32)) * kSlice32 + key % kSlice32] = live ? float_key(sc) : 0u;
              });
        }
        sel_n = kSliceSlots * (ns - nbad) + kSlice32 * nbad;  // > k: it holds every candidate
      }
    } else if constexpr (NR > 0) {
      if (full && !ma.scores)  // the row's scores were not kept: recompute them all
        fp4_rescore_row<NR>(ma.rescore, (int)row, V, *(Fp4QueryLds*)ostage, ma.row_scores + row * ma.n_cap);
    }
  }
  if (full) {  // select again, from the union above or from the whole row (any input)
    const uint2* lists = ma.cand + row * nslices * kSliceSlots;
    const uint32_t* bkeys = ostage + kBadKeysOffset;
    // position v -> (key, index).  Union: the slices in ascending order, kSliceSlots
    // positions for a good slice's list, kSlice32 for a bad slice's keys.
    auto key_at = [&](int v, uint32_t* index) -> uint32_t {
      if (sel_n == 0) {
        *index = (uint32_t)v;
        return float_key(srow[v]);
      }
      int i = 0;
      for (; i < nbad; ++i) {
        const int bs = badstart[i];
        if (v < bs) break;
        if (v < bs + kSlice32) {
          *index = (uint32_t)(kSlice32 * badlist[i] + (v - bs));
          return bkeys[i * kSlice32 + (v - bs)];
        }
      }
      const uint2 e = lists[v - (kSlice32 - kSliceSlots) * i];
      *index = e.y;
      return e.x;
    };
    auto key = [&](int v) {
      uint32_t ix;
      return key_at(v, &ix);
    };
    const int n = sel_n ? sel_n : V;
    uint32_t T, krem;
    radix_threshold(key, n, k, sh, &T, &krem);
    compact_selected(key, n, T, krem, sh, [&](int v, uint32_t r) {
      uint32_t ix;
      key_at(v, &ix);
      if (r < (uint32_t)k) out[r] = (int32_t)ix;
    });
  }
}

// Rows of up to THREADS * NPT keys (a prefill chunk's rows), register-resident: thread t
// holds positions NPT*t .. NPT*t+NPT-1, so slot order is index order.  The threshold is
// found on the registers (block_threshold_regs: value-linear bins first, then key-space
// bins, exact) and the compaction is one block scan, as in the slice-list merge.  A
// present key is made nonzero (0 marks the positions past the row's visible count; only
// the all-ones NaN pattern maps to 0 and is folded onto the next key).
// Workgroups of 512 threads, two resident per CU, each walking rows w, w + grid, ...:
// while one selects (barriers, LDS round trips), the other's work fills the SIMDs.
constexpr int kTopkRegsMaxK = 4096;  // selections staged in LDS before the coalesced write
constexpr int kTopkRegsThreads = 512;
constexpr int kTopkRegsPerCu = 2;

template <int NPT, bool VEC>  // VEC: 16-byte aligned rows (scores 16-byte aligned, n_cap % 4 == 0)
__global__ __launch_bounds__(kTopkRegsThreads, kTopkRegsPerCu * kTopkRegsThreads / kWave / 4) void topk_regs_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int n_cap, int m, int k, int64_t rows,
    int32_t* __restrict__ idx) {
  static_assert(NPT % 4 == 0, "float4 loads");
  constexpr int TH = kTopkRegsThreads;
  __shared__ RegSelLds rs;
  __shared__ uint32_t ostage[kTopkRegsMaxK + TH];  // indices by rank, then discard slots
  const int t = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    // the row's scores as stored (every position below the capacity: the visible count
    // is applied after the loads, so they need not wait for the row's position;
    // positions past the capacity read a position inside it instead)
    const float* src = scores + row * n_cap;
    float4 cur[NPT / 4];
#pragma unroll
    for (int q = 0; q < NPT / 4; ++q) {
      const int p0 = NPT * t + 4 * q;
      if constexpr (VEC) {
        cur[q] = *(const float4*)(src + min(p0, n_cap - 4));
      } else {
        cur[q].x = src[min(p0, n_cap - 1)];
        cur[q].y = src[min(p0 + 1, n_cap - 1)];
        cur[q].z = src[min(p0 + 2, n_cap - 1)];
        cur[q].w = src[min(p0 + 3, n_cap - 1)];
      }
    }
    const int V = min(visible_blocks(q_pos[row], m), n_cap);
    int32_t* out = idx + row * k;
    uint32_t kv[NPT];
#pragma unroll
    for (int q = 0; q < NPT / 4; ++q) {
      const int p0 = NPT * t + 4 * q;
      kv[4 * q] = p0 < V ? max(float_key(cur[q].x), 1u) : 0u;
      kv[4 * q + 1] = p0 + 1 < V ? max(float_key(cur[q].y), 1u) : 0u;
      kv[4 * q + 2] = p0 + 2 < V ? max(float_key(cur[q].z), 1u) : 0u;
      kv[4 * q + 3] = p0 + 3 < V ? max(float_key(cur[q].w), 1u) : 0u;
    }
    if (V <= k) {  // workgroup-uniform
      for (int i = t; i < k; i += TH) out[i] = i < V ? i : -1;
    } else {
      uint32_t lo, hi, M;
      block_key_range<NPT, TH>(kv, rs, &lo, &hi, &M);  // M = V > k (its barrier also ends the previous row's LDS use)
      uint32_t T, krem;
      block_threshold_regs<NPT, TH, false>(kv, lo, hi, (uint32_t)k, rs, &T, &krem);
      // compaction in position order: one scan of (keys > T) | (copies of T) << 16
      uint32_t gtc = 0, eqc = 0;
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        gtc += kv[j] > T;
        eqc += kv[j] == T;
      }
      const uint32_t packed = gtc | (eqc << 16);
      uint32_t tot;
      const uint32_t excl = block_scan_regsel<TH>(packed, rs.scan[2], &tot) - packed;
      krem = min(krem, tot >> 16);  // "every copy" made a count
      uint32_t eq_seen = excl >> 16;
      uint32_t r = (excl & 0xffffu) + min(eq_seen, krem);
      if (__builtin_amdgcn_ballot_w64(eqc != 0u) == 0ull) {  // no copy of T in this wave
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          const bool keep = kv[j] > T;
          ostage[keep && r < (uint32_t)k ? r : (uint32_t)kTopkRegsMaxK + t] = (uint32_t)(NPT * t + j);
          r += keep;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
          const bool is_eq = kv[j] == T;
          const bool keep = kv[j] > T || (is_eq && eq_seen < krem);
          eq_seen += is_eq;
          ostage[keep && r < (uint32_t)k ? r : (uint32_t)kTopkRegsMaxK + t] = (uint32_t)(NPT * t + j);
          r += keep;
        }
      }
      __syncthreads();
      for (int i = t; i < k; i += TH) out[i] = (int32_t)ostage[i];
      __syncthreads();  // ostage and the tables are free for the next row
    }
  }
}
static_assert(40 * kTopkRegsThreads >= kTopkLdsMax, "the register path covers every row the LDS path does");
static_assert(kTopkRegsThreads * 40 < 65536 && kSliceMergeCap < 65536, "scan halves of 16 bits");

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
  const size_t narrow = align256((size_t)rows * ns32 * sizeof(SliceMeta)) + align256((size_t)rows * ns32 * kSliceSlots * 8);
  return std::max(wide, narrow);
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int batch, int tq, int n_cap, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)batch * tq;
  if (rows == 0) return hipSuccess;
  if (n_cap <= kTopkLdsMax && k <= kTopkRegsMaxK) {
    // two resident workgroups per CU, each walking rows w, w + grid, ...
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const dim3 grid((unsigned)std::min<int64_t>(rows, (int64_t)kTopkRegsPerCu * std::max(cus, 1))),
        block(kTopkRegsThreads);
    const bool vec = (((uintptr_t)scores) & 15) == 0 && (n_cap & 3) == 0 && n_cap >= 4;
#define CSA_TOPK_REGS(NPT)                                                                                       \
  if (vec)                                                                                                       \
    hipLaunchKernelGGL((topk_regs_kernel<NPT, true>), grid, block, 0, s, scores, q_pos, n_cap, m, k, rows, idx); \
  else                                                                                                           \
    hipLaunchKernelGGL((topk_regs_kernel<NPT, false>), grid, block, 0, s, scores, q_pos, n_cap, m, k, rows, idx);
    // the fewest keys per thread (a multiple of 4) that hold the row: slots past the
    // row still cost their share of every pass
    if (n_cap <= 16 * kTopkRegsThreads) {
      CSA_TOPK_REGS(16)
    } else if (n_cap <= 24 * kTopkRegsThreads) {
      CSA_TOPK_REGS(24)
    } else if (n_cap <= 32 * kTopkRegsThreads) {
      CSA_TOPK_REGS(32)
    } else if (n_cap <= 36 * kTopkRegsThreads) {
      CSA_TOPK_REGS(36)
    } else {
      CSA_TOPK_REGS(40)
    }
#undef CSA_TOPK_REGS
    return hipGetLastError();
  }
  if (n_cap <= kTopkLdsMax) {
    const size_t lds = (size_t)std::max(n_cap, 1) * 4;
    hipLaunchKernelGGL(topk_lds_kernel, dim3((unsigned)rows), dim3(kLdsThreads), lds, s, scores, q_pos, n_cap, m, k,
                       idx);
    return hipGetLastError();
  }
  {
    const int ns32 = (n_cap + kSlice32 - 1) / kSlice32;
    if (ns32 * kSliceSlots <= kSliceMergeCap && k <= kSliceMergeCap) {
      SliceMeta* meta = (SliceMeta*)ws;
      uint2* cand = (uint2*)((char*)ws + align256((size_t)rows * ns32 * sizeof(SliceMeta)));
      hipLaunchKernelGGL(topk_cand32_kernel, dim3((unsigned)((ns32 + 3) / 4), (unsigned)rows), dim3(256), 0, s, scores,
                         q_pos, n_cap, m, k, ns32, cand, meta);
      MergeArgs ma{};
      ma.scores = scores;
      ma.q_pos = q_pos;
      ma.n_cap = n_cap;
      ma.m = m;
      ma.k = k;
      ma.nslices = ns32;
      ma.cand = cand;
      ma.meta = meta;
      ma.idx = idx;
      hipLaunchKernelGGL(topk_merge_slices_kernel<0>, dim3((unsigned)rows), dim3(kMergeThreads32), 0, s, ma);
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
__host__ inline size_t fused_lists_bytes(int64_t rows, int n_cap) {
  const int ns = fused_slices(n_cap);
  return align256((size_t)rows * ns * sizeof(SliceMeta)) + align256((size_t)rows * ns * kFusedC * 8);
}
}  // namespace

bool index_topk_fused_ok(const IndexArgs& a, int k) {
  // MXFP4 keys (the indexer that emits lists), long rows, and lists that fit the merge
  // pass (nslices * 64 slots in registers, one thread per slice for the certificate)
  const int ns = fused_slices(a.n_cap);
  return a.k.dtype == CSA_MXFP4 && a.n_cap > kTopkLdsMax && ns <= kMergeMaxSlices &&
         (int64_t)ns * kFusedC <= kSliceMergeCap && k <= kSliceMergeCap;
}

// Workspace: the slice lists (and the top-k pass's own needs), then, when the caller
// keeps no scores, one score row per query row.
size_t index_topk_score_offset(int64_t rows, int n_cap, int k) {
  return align256(std::max(topk_workspace_bytes(rows, n_cap, k),
                           n_cap > kTopkLdsMax ? fused_lists_bytes(rows, n_cap) : (size_t)0));
}

size_t index_topk_workspace_bytes(int64_t rows, int n_cap, int k, bool scores_in_ws) {
  const size_t lists = index_topk_score_offset(rows, n_cap, k);
  return scores_in_ws ? lists + align256((size_t)rows * n_cap * sizeof(float)) : lists;
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
  co.row_scores = (float*)((char*)ws + index_topk_score_offset(rows, a.n_cap, k));
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
  MergeArgs ma{};
  ma.scores = a.scores;
  ma.row_scores = co.row_scores;
  ma.q_pos = a.q_pos;
  ma.n_cap = a.n_cap;
  ma.m = a.m;
  ma.k = k;
  ma.nslices = co.nslices;
  ma.cand = co.cand;
  ma.meta = co.meta;
  ma.idx = idx;
  ma.short_rows = 1;
  ma.rescore = a;
  if (a.heads <= 8)
    hipLaunchKernelGGL(topk_merge_slices_kernel<4>, dim3((unsigned)rows), dim3(kMergeThreads32), 0, s, ma);
  else
    hipLaunchKernelGGL(topk_merge_slices_kernel<16>, dim3((unsigned)rows), dim3(kMergeThreads32), 0, s, ma);
  return hipGetLastError();
}

}  // namespace csa

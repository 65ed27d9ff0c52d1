// Exact block-wide selection helpers shared by the top-k kernels and the
// indexer's candidate epilogue: the top-k threshold of n order-preserving keys
// (ties broken by position) and the ascending-position compaction of the
// selected set.  Integer histograms and ballots only, so results are exact and
// independent of scheduling.
#pragma once
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

// ------------------------------------------------------------------ block helpers
// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts inside each
// 16-lane row (zeros shifted in), then the three lower rows' totals.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                 r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x % kWave) / 16;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Inclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
__device__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp /* >= 16 */, uint32_t* total) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_incl_scan(v);
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
__device__ __forceinline__ void radix_threshold(KeyFn key, int n, int k, SelShared& sh, uint32_t* T_out, uint32_t* krem_out) {
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
      const uint32_t incl = wave_incl_scan(mine);
      uint32_t run = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;  // keys in bins above this lane's four
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
__device__ __forceinline__ void compact_selected(KeyFn key, int n, uint32_t T, uint32_t krem, SelShared& sh, Emit emit) {
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

// ------------------------------------------------------------------ one-wave top-32
constexpr int kWaveTopN = 16;  // keys per lane of a one-wave slice selection: 1024 per wave

// The float a key came from (inverse of float_key).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// ------------------------------------------------------------------ slice candidate lists
// A slice of 1024 consecutive keys (one wave, lane L holding positions 16L .. 16L+15)
// hands the row's top-k merge its exact top-kSliceSlots in (key desc, position asc)
// order, listed in position order.  They are found cheaply: a cut keeps every key >=
// tau, tau being the 32nd largest of the 64 lane maxima (so the top 32 all pass, and
// typically about 45 keys do), and the survivors, one per lane in position order, are
// cut again at their own 32nd largest key.  When
// more than kCutMax keys pass the cut (many equal scores), the top-kSliceSlots are
// found by a bit-by-bit threshold instead.  Every key left out ranks after the list's
// last element, so a row's merge is exact unless that element is selected -- which
// needs kSliceSlots of the row's top-k in one slice (a row's top 2048 of 262,144
// blocks put about 8 in a slice, and rarely over 24).
constexpr int kSliceKeys = kWaveTopN * kWave;  // 1024
constexpr int kSliceSlots = 32;
constexpr int kCutMax = kWave;  // survivors of the cut ranked in one pass (one per lane)

struct CutLds {
  __attribute__((aligned(16))) uint2 res[kCutMax + kWave];  // (key, position) staged; then discard slots
};

// Slice list format: kSliceSlots (key, index) pairs in ascending index order, empty
// slots (0, 0) after them; metadata {count, trunc, last_key, last_idx} where trunc
// says some visible key of the slice was left out, and every key left out ranks
// strictly after (last_key, last_idx) in (key desc, index asc) order.

// Exact top-C (C <= kSliceSlots, more than C keys present) of the keys one wave holds,
// in (key desc, position asc) order, staged in position order in cl.res[0..C-1];
// returns the C-th kept key and the position of its last kept copy.  The threshold is
// built bit by bit (the largest value with at least C keys at or above it), which
// needs only a few registers: the path for slices whose keys tie at the cut.
__device__ void wave_topc_exact(const uint32_t (&kv)[kWaveTopN], uint32_t C, CutLds& cl, uint32_t* T_out,
                                uint32_t* tpos_out) {
  const int L = threadIdx.x % kWave;
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) c += kv[j] >= cand;
    T = __builtin_amdgcn_readlane(wave_incl_scan(c), kWave - 1) >= C ? cand : T;
  }
  uint32_t gtc = 0, eqc = 0;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) {
    gtc += kv[j] > T;
    eqc += kv[j] == T;
  }
  const uint32_t krem = C - __builtin_amdgcn_readlane(wave_incl_scan(gtc), kWave - 1);  // copies of T taken
  const uint32_t eq_before = wave_incl_scan(eqc) - eqc;                                 // copies in lanes below
  const uint32_t take = eq_before >= krem ? 0u : min(eqc, krem - eq_before);
  const uint32_t selc = gtc + take;
  uint32_t r = wave_incl_scan(selc) - selc;
  uint32_t seen = 0, tpos = 0;
  bool has_t = false;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) {
    const bool is_eq = kv[j] == T;
    const bool keep = kv[j] > T || (is_eq && seen < take);
    const bool last = is_eq && seen < take && eq_before + seen == krem - 1u;
    tpos = last ? (uint32_t)(kWaveTopN * L + j) : tpos;
    has_t = has_t || last;
    seen += is_eq;
    cl.res[keep ? r : (uint32_t)kCutMax + L] = make_uint2(kv[j], (uint32_t)(kWaveTopN * L + j));
    r += keep;
  }
  *tpos_out = __builtin_amdgcn_readlane(tpos, __builtin_ctzll(__builtin_amdgcn_ballot_w64(has_t)));
  *T_out = T;
}

// The k-th largest (1 <= k <= 64) of the 64 lanes' values, counting repeats: the
// largest v with at least k lanes at or above it, built bit by bit (a compare and a
// ballot count per bit; the result is wave-uniform).
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t x, uint32_t k) {
  uint32_t T = 0u;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    T = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(x >= cand)) >= k ? cand : T;
  }
  return T;
}

// Writes the list of the n <= 1024 keys one wave holds (absent positions hold key 0,
// present keys are > 0) for the slice whose position 0 is index `start`.
__device__ void emit_slice_list(const uint32_t (&kv)[kWaveTopN], int n, uint32_t start, CutLds& cl, uint2* out,
                                SliceMeta* mt) {
  const int L = threadIdx.x % kWave;
  if (n <= kSliceSlots) {  // every key of the slice
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) {
      const int p = kWaveTopN * L + j;
      if (p < kSliceSlots) out[p] = p < n ? make_uint2(kv[j], start + (uint32_t)p) : make_uint2(0u, 0u);
    }
    if (L == 0) *mt = SliceMeta{(uint32_t)n, 0u, 0u, 0u};
    return;
  }
  // tau: the 32nd largest lane maximum, with its 6 low bits cleared.  The maxima are
  // made distinct by putting 63 - lane in those bits (so the 32nd largest is one
  // value, found bit by bit over the wave: one compare and a ballot count per bit);
  // clearing them again keeps every lane at or above the 32nd maximum passing the
  // cut, so at least 32 keys do.
  uint32_t lmx = 0u;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) lmx = max(lmx, kv[j]);
  const uint32_t lmu = (lmx & ~63u) | (uint32_t)(63 - L);
  // (present keys are > 0: "present and >= tau" is one compare against max(tau, 1))
  const uint32_t tau = max(wave_kth_largest(lmu, 32u) & ~63u, 1u);
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) c += kv[j] >= tau;
  const uint32_t incl = wave_incl_scan(c);
  const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
  uint32_t lk, li;
  uint2 e;
  bool keep;
  uint32_t slot;
  if (total <= (uint32_t)kCutMax) {
    // stage the survivors in position order (survivor i in lane i), then keep the
    // top kSliceSlots: keys above the kSliceSlots-th largest survivor key T, and the
    // first (lowest-position, i.e. lowest-lane) copies of T
    uint32_t o = incl - c;
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) {
      const bool in = kv[j] >= tau;
      cl.res[in ? o : (uint32_t)kCutMax + L] = make_uint2(kv[j], (uint32_t)(kWaveTopN * L + j));
      o += in;
    }
    e = (uint32_t)L < total ? cl.res[L] : make_uint2(0u, 0u);  // LDS ops of one wave run in order
    const uint32_t T = wave_kth_largest(e.x, (uint32_t)kSliceSlots);
    const uint64_t below = (1ull << L) - 1ull;
    const uint32_t ngt = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(e.x > T));
    const uint64_t eqm = __builtin_amdgcn_ballot_w64(e.x == T && (uint32_t)L < total);
    const uint32_t eqr = (uint32_t)__builtin_popcountll(eqm & below);  // copies of T in lower lanes
    const uint32_t take = (uint32_t)kSliceSlots - ngt;                  // >= 1: T is the kSliceSlots-th key
    keep = e.x > T || (e.x == T && (uint32_t)L < total && eqr < take);
    const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
    slot = (uint32_t)__builtin_popcountll(km & below);  // position order among the kept
    // the list's last element in (key desc, position asc) order: the take-th copy of T
    const int ll = __builtin_ctzll(__builtin_amdgcn_ballot_w64(e.x == T && (uint32_t)L < total && eqr == take - 1u));
    lk = T;
    li = start + __builtin_amdgcn_readlane(e.y, ll);
  } else {  // many keys at or above tau: the top kSliceSlots by a bit-by-bit threshold
    uint32_t T, tpos;
    wave_topc_exact(kv, (uint32_t)kSliceSlots, cl, &T, &tpos);
    keep = L < kSliceSlots;
    slot = (uint32_t)L;
    e = cl.res[L % kSliceSlots];
    lk = T;
    li = start + tpos;
  }
  if (keep) out[slot] = make_uint2(e.x, start + e.y);
  if (L == 0) *mt = SliceMeta{(uint32_t)kSliceSlots, 1u, lk, li};
}

// ------------------------------------------------------------------ block top-k, keys in registers
// Block sizes of the register-resident selection: 256, 512 or 1024 threads (THREADS
// below).  Fewer threads holding more keys each run the per-wave scans and reductions
// on fewer waves: with 16 waves on a CU's 4 SIMDs every such step is issued 16 times.
constexpr int kRegSelMaxThreads = 1024;
constexpr int kRegSelBins = 1024;     // histogram bins: kRegSelBins / THREADS per thread
constexpr int kRegSelMaxWaves = kRegSelMaxThreads / kWave;

struct RegSelLds {
  // kRegSelBins bins, then one never-read bin per lane that absent keys of the first
  // pass count into (so that pass adds with no per-key branch and no shared address)
  __attribute__((aligned(16))) uint32_t hist[2][kRegSelBins + kWave];
  uint32_t red[3][kRegSelMaxWaves];   // per-wave min, max, count
  uint32_t scan[3][kRegSelMaxWaves];  // per-wave totals of block scans
  uint32_t bin, above, cnt, nfin, T, krem, jT, bad;
  __attribute__((aligned(16))) uint32_t fk[64];
  __attribute__((aligned(16))) uint32_t fp[64];
};

// Combining one value per wave (at most 16 waves): lane i of every wave reads wave i's
// value, then DPP steps inside the first 16-lane row do the rest (lanes 16.. unused).
// Inclusive prefix sum over lanes 0 .. 15 (zeros shifted in).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  return v;
}
// Minimum or maximum over lanes 0 .. 15, as a wave-uniform value.
template <bool MAX>
__device__ __forceinline__ uint32_t row16_reduce(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return __builtin_amdgcn_readlane(v, 0);
}

// Inclusive prefix sum over a block of THREADS threads (one barrier; tmp is not
// reused by the caller until after a later barrier).
template <int THREADS>
__device__ __forceinline__ uint32_t block_scan_regsel(uint32_t v, uint32_t* tmp, uint32_t* total) {
  static_assert(THREADS % kWave == 0 && THREADS <= kRegSelMaxThreads && kRegSelBins % THREADS == 0, "block size");
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), L = threadIdx.x % kWave;
  const uint32_t incl = wave_incl_scan(v);
  if (L == kWave - 1) tmp[w] = incl;
  __syncthreads();
  constexpr int NW = THREADS / kWave;
  const uint32_t wi = row16_incl_scan(L < NW ? tmp[L] : 0u);  // lane i < NW: waves 0 .. i
  *total = __builtin_amdgcn_readlane(wi, NW - 1);
  const uint32_t below = __builtin_amdgcn_readlane(wi, max(w, 1) - 1);  // waves 0 .. w-1 (for w > 0)
  return incl + (w > 0 ? below : 0u);
}

// Min and max present key and the number of present keys of a block holding
// kv[NPT] per thread (0 = absent); also clears rs.hist[0] and rs.bad for
// block_threshold_regs and its caller.
template <int NPT, int THREADS>
__device__ __forceinline__ void block_key_range(const uint32_t (&kv)[NPT], RegSelLds& rs, uint32_t* lo, uint32_t* hi, uint32_t* cnt) {
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t / kWave), L = t % kWave;
  uint32_t mn = 0xffffffffu, mx = 0u, c = 0u;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    mn = kv[j] ? min(mn, kv[j]) : mn;
    mx = max(mx, kv[j]);
    c += kv[j] != 0u;
  }
  mn = wave_reduce_u32<false>(mn);
  mx = wave_reduce_u32<true>(mx);
  c = __builtin_amdgcn_readlane(wave_incl_scan(c), kWave - 1);
  if (L == 0) {
    rs.red[0][w] = mn;
    rs.red[1][w] = mx;
    rs.red[2][w] = c;
  }
#pragma unroll
  for (int i = 0; i < kRegSelBins / THREADS; ++i) rs.hist[0][t + i * THREADS] = 0u;
  if (t == 0) rs.bad = 0u;
  __syncthreads();
  constexpr int NW = THREADS / kWave;
  *lo = row16_reduce<false>(L < NW ? rs.red[0][L] : 0xffffffffu);
  *hi = row16_reduce<true>(L < NW ? rs.red[1][L] : 0u);
  *cnt = __builtin_amdgcn_readlane(row16_incl_scan(L < NW ? rs.red[2][L] : 0u), 15);
}

// Exact threshold of the top-k of the keys a block of THREADS threads holds in
// registers (thread t: kv[j] is the key of slot NPT*t + j, tie order = slot
// ascending; 0 = absent, present keys > 0, more than k present; [lo, hi] the
// present range from block_key_range, whose barrier this call relies on).
// Returns the k-th largest key T and the number krem of its copies taken (the
// lowest-slot ones; 0xffffffff when every copy is taken).  A first pass of 1024
// bins linear in the score, then
// key-space passes of 1024 bins over the bin of the k-th key while it holds
// more than 64 keys; those are ranked exactly by one wave.  A non-decreasing
// map from key to bin keeps every bin a contiguous range of the key order,
// which is all the selection needs to stay exact.
template <int NPT, int THREADS, bool KEEP_BINS = true>
__device__ __forceinline__ void block_threshold_regs(const uint32_t (&kv)[NPT], uint32_t lo, uint32_t hi, uint32_t k, RegSelLds& rs,
                                     uint32_t* T_out, uint32_t* krem_out) {
  constexpr int NW = THREADS / kWave;
  constexpr int BPT = kRegSelBins / THREADS;  // bins per thread in the scan
  const int t = threadIdx.x;
  uint32_t krem = k;
  int buf = 0;
  // one pass: histogram of bins binf(j) (-1 = not counted) into rs.hist[buf], then the
  // bin holding the krem-th key from the top, the keys above it and its count
  // (every_key: binf(j) < 0 goes to this lane's own extra bin instead of being skipped;
  // used by the first pass with kept bins, where few keys are absent)
  auto pass = [&](auto binf, auto every_key, uint32_t* bin, uint32_t* above, uint32_t* cn) {
    const int lane_bin = kRegSelBins + (int)(threadIdx.x % kWave);
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int bj = binf(j);
      if constexpr (decltype(every_key)::value)
        atomicAdd(&rs.hist[buf][bj >= 0 ? bj : lane_bin], 1u);
      else if (bj >= 0)
        atomicAdd(&rs.hist[buf][bj], 1u);
    }
    __syncthreads();
    // thread t scans bins kRegSelBins - 1 - (BPT t + i), i = 0 .. BPT - 1 (descending)
    uint32_t h[BPT], hs = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      h[i] = rs.hist[buf][kRegSelBins - 1 - (BPT * t + i)];
      hs += h[i];
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) rs.hist[buf ^ 1][t + i * THREADS] = 0u;  // the next pass's histogram
    uint32_t tot;
    uint32_t run = block_scan_regsel<THREADS>(hs, rs.scan[buf], &tot) - hs;  // keys in the bins above
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (run < krem && run + h[i] >= krem) {
        rs.bin = (uint32_t)(kRegSelBins - 1 - (BPT * t + i));
        rs.above = run;
        rs.cnt = h[i];
      }
      run += h[i];
    }
    if (t == 0) rs.nfin = 0u;
    __syncthreads();
    *bin = rs.bin;
    *above = rs.above;
    *cn = rs.cnt;
    buf ^= 1;
  };
  bool finish = false, by_bin = false;
  uint32_t fbin = 0, cn_last = 0xffffffffu;  // keys in the final range (unknown before a pass)
  const float xlo = key_float(lo), xhi = key_float(hi);
  const float inv = 1023.99f / (xhi - xlo);
  // the first pass's bins: kept in registers (KEEP_BINS), or recomputed where needed by
  // kernels short of registers (the same expression, so the same bins)
  constexpr bool kKeepBins = KEEP_BINS;
  // -1 for an absent key.  With the bins kept (registers to spare) this is arithmetic
  // rather than a select, so the pass takes no branch per key: the clamp is then done in
  // float, so that an absent key's NaN becomes 0 before the conversion (present keys lie
  // in [lo, hi], at 0 .. 1023.99 before the clamp: the same bins as an integer clamp
  // after the conversion)
  auto vbin = [&](int j) {
    if constexpr (KEEP_BINS) {
      const float v = fminf(fmaxf((key_float(kv[j]) - xlo) * inv, 0.f), (float)(kRegSelBins - 1));
      return (int)v | -(int)(kv[j] == 0u);
    } else {
      return kv[j] ? min(kRegSelBins - 1, max(0, (int)((key_float(kv[j]) - xlo) * inv))) : -1;
    }
  };
  int b[kKeepBins ? NPT : 1];
  auto first_bin = [&](int j) {
    if constexpr (kKeepBins)
      return b[j];
    else
      return vbin(j);
  };
  // NaN and infinite scores, or a span too small to invert, go to the key-space passes
  if (lo != hi && xhi - xlo < __builtin_inff() && inv < __builtin_inff()) {
    if constexpr (kKeepBins) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) b[j] = vbin(j);
    }
    uint32_t above, cn;
    pass(first_bin, std::integral_constant<bool, KEEP_BINS>{}, &fbin, &above, &cn);
    krem -= above;
    cn_last = cn;
    if (cn <= 64u || cn == krem) {
      finish = by_bin = true;
    } else {  // the key range of that bin (a contiguous range of the key order)
      const int w = __builtin_amdgcn_readfirstlane(t / kWave), L = t % kWave;
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (first_bin(j) == (int)fbin) {
          mn = min(mn, kv[j]);
          mx = max(mx, kv[j]);
        }
      mn = wave_reduce_u32<false>(mn);
      mx = wave_reduce_u32<true>(mx);
      if (L == 0) {
        rs.red[0][w] = mn;
        rs.red[1][w] = mx;
      }
      __syncthreads();
      lo = row16_reduce<false>(L < NW ? rs.red[0][L] : 0xffffffffu);
      hi = row16_reduce<true>(L < NW ? rs.red[1][L] : 0u);
    }
  }
  // key-space passes: 32 bits at <= 10 bits per pass end in a single key after 4
  for (int p = 0; p < 4 && !finish && lo != hi; ++p) {
    by_bin = false;
    const int bits = 32 - __builtin_clz(hi - lo);
    const int shift = bits > 10 ? bits - 10 : 0;
    uint32_t bin, above, cn;
    pass([&](int j) { return (kv[j] >= lo && kv[j] <= hi) ? (int)((kv[j] - lo) >> shift) : -1; }, std::false_type{},
         &bin, &above, &cn);
    const uint32_t nlo = lo + (bin << shift);
    hi = min(hi, nlo + ((1u << shift) - 1u));
    lo = nlo;
    krem -= above;
    cn_last = cn;
    finish = cn <= 64u || cn == krem;
  }
  uint32_t T = lo;
  auto in_final = [&](int j) { return by_bin ? first_bin(j) == (int)fbin : (kv[j] >= lo && kv[j] <= hi); };
  if (finish && cn_last == krem) {
    // the final range is taken whole: T is its smallest key, every copy of it taken
    const int w = __builtin_amdgcn_readfirstlane(t / kWave), L = t % kWave;
    uint32_t mn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < NPT; ++j) mn = in_final(j) ? min(mn, kv[j]) : mn;
    mn = wave_reduce_u32<false>(mn);
    if (L == 0) rs.red[0][w] = mn;
    __syncthreads();
    T = row16_reduce<false>(L < NW ? rs.red[0][L] : 0xffffffffu);
    krem = 0xffffffffu;
  } else if (finish && (by_bin || lo != hi)) {
    // gather the <= 64 keys of the final bin with their slots, then rank them in one wave
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const bool in = in_final(j);
      if (in) {
        const uint32_t s = atomicAdd(&rs.nfin, 1u);
        rs.fk[s] = kv[j];
        rs.fp[s] = (uint32_t)(NPT * t + j);
      }
    }
    __syncthreads();
    if (t < kWave) {
      const uint32_t c = rs.nfin;
      if ((uint32_t)t >= c) {  // pad to whole quads with entries that never rank above
        rs.fk[t] = 0u;
        rs.fp[t] = 0xffffffffu;
      }
      const uint32_t myk = rs.fk[t], myp = rs.fp[t];  // entry t (a pad when t >= c)
      uint32_t rank = 0, gt = 0;
      for (uint32_t i = 0; i < c; i += 4) {
        const uint4 k4 = *(const uint4*)&rs.fk[i], p4 = *(const uint4*)&rs.fp[i];
        const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w}, pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // bitwise, not short-circuit: no branch around the loads
          rank += (uint32_t)(kk[q] > myk) | ((uint32_t)(kk[q] == myk) & (uint32_t)(pp[q] < myp));
          gt += kk[q] > myk;
        }
      }
      if ((uint32_t)t < c && rank == krem - 1u) {
        rs.T = myk;
        rs.krem = krem - gt;
      }
    }
    __syncthreads();
    T = rs.T;
    krem = rs.krem;
  }
  *T_out = T;
  *krem_out = krem;
}

}  // namespace
}  // namespace csa

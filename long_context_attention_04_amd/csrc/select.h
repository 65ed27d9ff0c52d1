// Exact block-wide selection helpers shared by the top-k kernels and the
// indexer's candidate epilogue: the top-k threshold of n order-preserving keys
// (ties broken by position) and the ascending-position compaction of the
// selected set.  Integer histograms and ballots only, so results are exact and
// independent of scheduling.
#pragma once
#include "common.h"

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
// ------------------------------------------------------------------ one-wave top-32
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

constexpr int kWaveTopC = 32;  // candidates a one-wave selection keeps
constexpr int kWaveTopN = 16;  // keys per lane: 1024 per wave
constexpr int kWaveTopPre = 4;  // keys per lane after the pre-filter: at most 256 survive it

// Wave-private LDS of one selection.  Every array has one extra slot per lane past
// its end: a lane whose store is not wanted writes there instead, so stores need no
// branch around them (a branch per key costs far more than the store).
struct WaveSelLds {
  __attribute__((aligned(16))) uint32_t hist[256 + kWave];
  __attribute__((aligned(16))) uint32_t fk[64 + kWave];
  __attribute__((aligned(16))) uint32_t fp[64 + kWave];
  __attribute__((aligned(16))) uint2 pre[kWave * kWaveTopPre + kWave];  // (key, position) of pre-filter survivors
  __attribute__((aligned(16))) uint2 res[kWaveTopC + kWave];            // the kept (key, position), by rank
};

// The float a key came from (inverse of float_key).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// The bin of the 32nd key in one histogram pass: hist holds 256 counts (lane L owns
// bins 4L .. 4L+3); returns the bin, and the keys above it and in it.
__device__ __forceinline__ void wave_find_bin(const WaveSelLds& sl, uint32_t krem, uint32_t* bin, uint32_t* above,
                                              uint32_t* cnt) {
  const int L = threadIdx.x % kWave;
  const uint4 h4 = *(const uint4*)&sl.hist[4 * L];
  const uint32_t hh[4] = {h4.x, h4.y, h4.z, h4.w};
  const uint32_t incl = wave_incl_scan(hh[0] + hh[1] + hh[2] + hh[3]);
  uint32_t run = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;  // keys in the bins of lanes > L
  int fd = -1;
  uint32_t ab = 0, cn = 0;
#pragma unroll
  for (int d = 3; d >= 0; --d) {
    const bool f = fd < 0 && run < krem && run + hh[d] >= krem;
    fd = f ? d : fd;
    ab = f ? run : ab;
    cn = f ? hh[d] : cn;
    run += hh[d];
  }
  const uint64_t fm = __builtin_amdgcn_ballot_w64(fd >= 0);  // exactly one lane
  const int fl = __builtin_ctzll(fm);
  *bin = __builtin_amdgcn_readlane(4 * L + fd, fl);
  *above = __builtin_amdgcn_readlane(ab, fl);
  *cnt = __builtin_amdgcn_readlane(cn, fl);
}

// Exact top-32, in (key desc, position asc) order, of the keys one wave holds with
// no workgroup barrier: lane L holds kv[j] in slot NK*L + j, slot order being
// ascending position order, and pos(j) is that key's position; absent slots hold
// 0, every present key is > 0, more than 32 are present and all lie in [lo, hi].
// A histogram select through wave-private LDS: a first pass of 256 bins linear in
// the score over [lo, hi], then radix passes in key space over the bin of the 32nd
// key while it holds more than 64 keys.  When that bin is taken whole, or holds a
// single key value, the threshold is known at once; otherwise its keys are ranked
// exactly.  The kept (key, position) pairs land in sl.res[0..31] in ascending
// position order.  Returns the 32nd kept key and the position of its last kept copy.
template <int NK, typename PosFn>
__device__ void wave_top32_core(const uint32_t (&kv)[NK], PosFn pos, uint32_t lo, uint32_t hi, WaveSelLds& sl,
                                uint32_t* T_out, uint32_t* tpos_out) {
  const int L = threadIdx.x % kWave;
  uint32_t krem = kWaveTopC;  // keys still to take from [lo, hi]
  uint32_t cn = 0xffffffffu;  // keys in [lo, hi] (unknown before a pass)
  const float xlo = key_float(lo), xhi = key_float(hi);
  const float inv = 255.99f / (xhi - xlo);
  // NaN and infinite scores, or a span too small to invert, go to the key-space passes
  if (lo != hi && xhi - xlo < __builtin_inff() && inv < __builtin_inff()) {
    // First pass in value space: 256 bins linear in the score over [lo, hi].  Any
    // non-decreasing map of the keys gives bins that are contiguous ranges of the key
    // order, so the selection stays exact; linear bins spread scores far better than
    // key bits (which bucket by float exponent), so the bin of the 32nd key is small
    // and usually settles the threshold in one pass.
    int bin[NK];
    *(uint4*)&sl.hist[4 * L] = make_uint4(0u, 0u, 0u, 0u);  // LDS ops of one wave run in order
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const float b = (key_float(kv[j]) - xlo) * inv;
      bin[j] = kv[j] ? min(255, max(0, (int)b)) : -1;
      atomicAdd(&sl.hist[bin[j] >= 0 ? bin[j] : 256 + L], 1u);
    }
    uint32_t fbin, ab;
    wave_find_bin(sl, krem, &fbin, &ab, &cn);
    krem -= ab;
    // the key range of that bin
    uint32_t bmx = 0u, bmn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const bool in = bin[j] == (int)fbin;
      bmx = in ? max(bmx, kv[j]) : bmx;
      bmn = in ? min(bmn, kv[j]) : bmn;
    }
    lo = wave_reduce_u32<false>(bmn);
    hi = wave_reduce_u32<true>(bmx);
  }
  // further passes in key space over [lo, hi] while its keys are more than 64
  for (int pass = 0; pass < 4 && cn > 64u && cn != krem && lo != hi; ++pass) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __builtin_clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    *(uint4*)&sl.hist[4 * L] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const bool in = kv[j] >= lo && kv[j] <= hi;
      atomicAdd(&sl.hist[in ? (kv[j] - lo) >> shift : 256u + L], 1u);
    }
    uint32_t bin, ab;
    wave_find_bin(sl, krem, &bin, &ab, &cn);
    const uint32_t nlo = lo + (bin << shift);
    hi = min(hi, nlo + ((1u << shift) - 1u));
    lo = nlo;
    krem -= ab;
  }
  // The threshold T and the copies of it to take: every key of [lo, hi] when the
  // range is taken whole (T = its smallest key), krem copies of a single-valued range,
  // else rank the <= 64 keys of the range exactly.
  uint32_t T = lo;
  const bool all_t = cn == krem;  // take every copy of T
  if (all_t) {
    uint32_t bmn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < NK; ++j) bmn = kv[j] >= lo && kv[j] <= hi ? min(bmn, kv[j]) : bmn;
    T = wave_reduce_u32<false>(bmn);
  } else if (lo != hi) {
    // gather the <= 64 keys of [lo, hi] with their positions, then rank them exactly
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < NK; ++j) c += kv[j] >= lo && kv[j] <= hi;
    uint32_t o = wave_incl_scan(c) - c;
    const uint32_t nfin = __builtin_amdgcn_readlane(o + c, kWave - 1);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const bool in = kv[j] >= lo && kv[j] <= hi;
      const uint32_t at = in ? o : 64u + L;
      sl.fk[at] = kv[j];
      sl.fp[at] = pos(j);
      o += in;
    }
    // pad to whole quads with entries that never rank above
    const uint32_t at = (uint32_t)L >= nfin ? (uint32_t)L : 64u + L;
    sl.fk[at] = 0u;
    sl.fp[at] = 0xffffffffu;
    const uint32_t myk = sl.fk[L], myp = sl.fp[L];  // entry L (a pad when L >= nfin)
    uint32_t rank = 0, gt = 0;
    for (uint32_t i = 0; i < nfin; i += 4) {  // broadcast reads, four entries at a time
      const uint4 k4 = *(const uint4*)&sl.fk[i], p4 = *(const uint4*)&sl.fp[i];
      const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w}, pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // bitwise, not short-circuit: no branch around the loads
        rank += (uint32_t)(kk[q] > myk) | ((uint32_t)(kk[q] == myk) & (uint32_t)(pp[q] < myp));
        gt += kk[q] > myk;
      }
    }
    const bool hit = (uint32_t)L < nfin && rank == krem - 1u;
    const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
    const int hl = __builtin_ctzll(hm);
    T = __builtin_amdgcn_readlane(myk, hl);
    krem -= __builtin_amdgcn_readlane(gt, hl);  // copies of T still to take
  }
  // compaction in slot order (lane-major): keys > T and the first krem copies of T
  uint32_t gtc = 0, eqc = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    gtc += kv[j] > T;
    eqc += kv[j] == T;
  }
  const uint32_t eq_incl = wave_incl_scan(eqc);
  const uint32_t eq_before = eq_incl - eqc;  // copies of T in lanes below
  if (all_t) krem = __builtin_amdgcn_readlane(eq_incl, kWave - 1);
  const uint32_t take = eq_before >= krem ? 0u : min(eqc, krem - eq_before);
  const uint32_t selc = gtc + take;
  uint32_t r = wave_incl_scan(selc) - selc;
  uint32_t seen = 0, tpos = 0;
  bool has_t = false;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const bool is_eq = kv[j] == T;
    const bool keep = kv[j] > T || (is_eq && seen < take);
    const bool last = is_eq && seen < take && eq_before + seen == krem - 1u;
    tpos = last ? pos(j) : tpos;
    has_t = has_t || last;
    seen += is_eq;
    sl.res[keep ? r : (uint32_t)kWaveTopC + L] = make_uint2(kv[j], pos(j));
    r += keep;
  }
  const uint64_t tm = __builtin_amdgcn_ballot_w64(has_t);
  *tpos_out = __builtin_amdgcn_readlane(tpos, __builtin_ctzll(tm));
  *T_out = T;
}

// Exact top-32, in (key desc, position asc) order, of the 1024 keys one wave holds:
// lane L holds kv[j], the key of position 16L + j; absent positions hold 0, every
// present key is > 0 and more than 32 are present.  The kept (key, position) pairs
// land in sl.res[0..31] in ascending position order; returns the 32nd kept key and
// the position of its last kept copy.
// Pre-filter: each of the 32 lane pairs holds a key at least as large as the smallest
// pair maximum tau, so at least as many keys as there are nonempty pairs are >= tau.
// When more than 32 and at most 256 keys are >= tau, the top-32 lies among them:
// they are compacted in position order (4 per lane) and only they are selected from.
// Otherwise the selection runs on all 16 keys per lane.
__device__ void wave_top32(const uint32_t (&kv)[kWaveTopN], WaveSelLds& sl, uint32_t* T_out, uint32_t* tpos_out) {
  const int L = threadIdx.x % kWave;
  uint32_t lmx = 0u, lmn = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) {
    lmx = max(lmx, kv[j]);
    lmn = kv[j] ? min(lmn, kv[j]) : lmn;
  }
  // quad_perm [1,0,3,2]: the other lane of the pair
  const uint32_t pm = max(lmx, (uint32_t)__builtin_amdgcn_update_dpp((int)lmx, (int)lmx, 0xB1, 0xF, 0xF, false));
  const uint32_t tau = wave_reduce_u32<false>(pm ? pm : 0xffffffffu);
  const uint32_t hi = wave_reduce_u32<true>(lmx);
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kWaveTopN; ++j) c += kv[j] >= tau;
  const uint32_t incl = wave_incl_scan(c);
  const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (total > (uint32_t)kWaveTopC && total <= (uint32_t)(kWave * kWaveTopPre)) {
    // empty slots first, then the survivors over them (LDS ops of one wave run in order)
    *(uint4*)&sl.pre[kWaveTopPre * L] = make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)&sl.pre[kWaveTopPre * L + 2] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t o = incl - c;
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j) {
      const bool in = kv[j] >= tau;
      sl.pre[in ? o : (uint32_t)(kWave * kWaveTopPre + L)] = make_uint2(kv[j], (uint32_t)(kWaveTopN * L + j));
      o += in;
    }
    const uint4 a4 = *(const uint4*)&sl.pre[kWaveTopPre * L], b4 = *(const uint4*)&sl.pre[kWaveTopPre * L + 2];
    const uint32_t k4[kWaveTopPre] = {a4.x, a4.z, b4.x, b4.z}, p4[kWaveTopPre] = {a4.y, a4.w, b4.y, b4.w};
    wave_top32_core<kWaveTopPre>(k4, [&](int j) { return p4[j]; }, tau, hi, sl, T_out, tpos_out);
  } else {
    const uint32_t lo = wave_reduce_u32<false>(lmn);
    wave_top32_core<kWaveTopN>(kv, [&](int j) { return (uint32_t)(kWaveTopN * L + j); }, lo, hi, sl, T_out, tpos_out);
  }
}


// ------------------------------------------------------------------ block top-k, keys in registers
constexpr int kRegSelThreads = 1024;  // block size of the register-resident selection
constexpr int kRegSelBins = 1024;     // histogram bins: one per thread
constexpr int kRegSelWaves = kRegSelThreads / kWave;

struct RegSelLds {
  __attribute__((aligned(16))) uint32_t hist[2][kRegSelBins];
  uint32_t red[3][kRegSelWaves];   // per-wave min, max, count
  uint32_t scan[3][kRegSelWaves];  // per-wave totals of block scans
  uint32_t bin, above, cnt, nfin, T, krem, jT, bad;
  __attribute__((aligned(16))) uint32_t fk[64];
  __attribute__((aligned(16))) uint32_t fp[64];
};

// Inclusive prefix sum over a kRegSelThreads block (one barrier; tmp is not
// reused by the caller until after a later barrier).
__device__ __forceinline__ uint32_t block_scan_regsel(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), L = threadIdx.x % kWave;
  const uint32_t incl = wave_incl_scan(v);
  if (L == kWave - 1) tmp[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kRegSelWaves; ++i) {
    const uint32_t x = tmp[i];
    base += i < w ? x : 0u;
    tot += x;
  }
  *total = tot;
  return incl + base;
}

// Min and max present key and the number of present keys of a block holding
// kv[NPT] per thread (0 = absent); also clears rs.hist[0] and rs.bad for
// block_threshold_regs and its caller.
template <int NPT>
__device__ void block_key_range(const uint32_t (&kv)[NPT], RegSelLds& rs, uint32_t* lo, uint32_t* hi, uint32_t* cnt) {
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
  rs.hist[0][t] = 0u;
  if (t == 0) rs.bad = 0u;
  __syncthreads();
  mn = 0xffffffffu, mx = 0u, c = 0u;
#pragma unroll
  for (int i = 0; i < kRegSelWaves; ++i) {
    mn = min(mn, rs.red[0][i]);
    mx = max(mx, rs.red[1][i]);
    c += rs.red[2][i];
  }
  *lo = mn;
  *hi = mx;
  *cnt = c;
}

// Exact threshold of the top-k of the keys a kRegSelThreads block holds in
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
template <int NPT>
__device__ void block_threshold_regs(const uint32_t (&kv)[NPT], uint32_t lo, uint32_t hi, uint32_t k, RegSelLds& rs,
                                     uint32_t* T_out, uint32_t* krem_out) {
  const int t = threadIdx.x;
  uint32_t krem = k;
  int buf = 0;
  // one pass: histogram of bins b[j] (-1 = not counted) into rs.hist[buf], then the
  // bin holding the krem-th key from the top, the keys above it and its count
  auto pass = [&](const int (&b)[NPT], uint32_t* bin, uint32_t* above, uint32_t* cn) {
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      if (b[j] >= 0) atomicAdd(&rs.hist[buf][b[j]], 1u);
    __syncthreads();
    const uint32_t h = rs.hist[buf][kRegSelBins - 1 - t];
    rs.hist[buf ^ 1][t] = 0u;  // the next pass's histogram
    uint32_t tot;
    const uint32_t incl = block_scan_regsel(h, rs.scan[buf], &tot);  // keys in bins >= 1023 - t
    if (incl - h < krem && incl >= krem) {
      rs.bin = (uint32_t)(kRegSelBins - 1 - t);
      rs.above = incl - h;
      rs.cnt = h;
    }
    if (t == 0) rs.nfin = 0u;
    __syncthreads();
    *bin = rs.bin;
    *above = rs.above;
    *cn = rs.cnt;
    buf ^= 1;
  };
  bool finish = false, by_bin = false;
  int b[NPT];
  uint32_t fbin = 0, cn_last = 0xffffffffu;  // keys in the final range (unknown before a pass)
  const float xlo = key_float(lo), xhi = key_float(hi);
  const float inv = 1023.99f / (xhi - xlo);
  // NaN and infinite scores, or a span too small to invert, go to the key-space passes
  if (lo != hi && xhi - xlo < __builtin_inff() && inv < __builtin_inff()) {
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      b[j] = kv[j] ? min(kRegSelBins - 1, max(0, (int)((key_float(kv[j]) - xlo) * inv))) : -1;
    uint32_t above, cn;
    pass(b, &fbin, &above, &cn);
    krem -= above;
    cn_last = cn;
    if (cn <= 64u || cn == krem) {
      finish = by_bin = true;
    } else {  // the key range of that bin (a contiguous range of the key order)
      const int w = __builtin_amdgcn_readfirstlane(t / kWave), L = t % kWave;
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (b[j] == (int)fbin) {
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
      lo = 0xffffffffu;
      hi = 0u;
#pragma unroll
      for (int i = 0; i < kRegSelWaves; ++i) {
        lo = min(lo, rs.red[0][i]);
        hi = max(hi, rs.red[1][i]);
      }
    }
  }
  // key-space passes: 32 bits at <= 10 bits per pass end in a single key after 4
  for (int p = 0; p < 4 && !finish && lo != hi; ++p) {
    by_bin = false;
    const int bits = 32 - __builtin_clz(hi - lo);
    const int shift = bits > 10 ? bits - 10 : 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) b[j] = (kv[j] >= lo && kv[j] <= hi) ? (int)((kv[j] - lo) >> shift) : -1;
    uint32_t bin, above, cn;
    pass(b, &bin, &above, &cn);
    const uint32_t nlo = lo + (bin << shift);
    hi = min(hi, nlo + ((1u << shift) - 1u));
    lo = nlo;
    krem -= above;
    cn_last = cn;
    finish = cn <= 64u || cn == krem;
  }
  uint32_t T = lo;
  auto in_final = [&](int j) { return by_bin ? b[j] == (int)fbin : (kv[j] >= lo && kv[j] <= hi); };
  if (finish && cn_last == krem) {
    // the final range is taken whole: T is its smallest key, every copy of it taken
    const int w = __builtin_amdgcn_readfirstlane(t / kWave), L = t % kWave;
    uint32_t mn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < NPT; ++j) mn = in_final(j) ? min(mn, kv[j]) : mn;
    mn = wave_reduce_u32<false>(mn);
    if (L == 0) rs.red[0][w] = mn;
    __syncthreads();
    T = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < kRegSelWaves; ++i) T = min(T, rs.red[0][i]);
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

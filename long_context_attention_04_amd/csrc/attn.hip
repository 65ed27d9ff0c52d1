// (d) CSA sparse attention and (e) HCA dense attention.
//
// Both attend over compressed entries plus a sliding window of raw local
// entries (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations
// 1: CSA bullet for the top-k compressed blocks, HCA bullet for dense
// attention over the heavily compressed entries and the window).  Readings:
// key = value = the stored (shared, MQA) row; one softmax over the compressed
// entries followed by the window rows, not de-duplicated.
//
// MFMA path (bf16 / fp8 caches, 16..64 heads, dim 512).  A query row's 16..64
// heads share one 512-wide latent row per entry, so attention is a
// [heads x 512] x [512 x n] contraction (QK) followed by [heads x n] x [n x 512]
// (PV), both on bf16 MFMA.  A workgroup takes one query row, one group of 16
// heads and one contiguous split of the entry list, with 8 waves (two per
// SIMD, covering each other's waits).  Each wave is an independent
// flash-decoding worker over every 8th tile of 16 entries:
//  * it loads a tile's rows one whole row per instruction (lane L taking
//    elements 8L .. 8L+7, the cheapest gather for the memory pipeline; the row
//    address is scalar) one tile ahead of use, from selection indices staged
//    in LDS once per workgroup, and stages the tile as bf16 rows in its own
//    LDS area (fp8 rows are widened there);
//  * QK reads the staged rows as the A operand and the workgroup's query heads
//    (staged in LDS once) as B, giving the transposed logits S^T = K Q^T
//    (16x16x32): each lane then holds four entries of one head -- exactly the
//    A-operand layout PV needs for P, so P never moves between lanes;
//  * the online softmax reduces over entries within the wave (register max,
//    then two cross-row lane swaps) and rescales the accumulator lazily: only
//    when a head's running maximum grows by more than 2^8, which keeps every
//    probability <= 256 and skips almost all rescaling work;
//  * P goes to PV as two bf16 terms (hi + lo, ~16 significant bits instead of
//    bf16's 8), stacked along the k axis of one 16x16x32 MFMA per column tile;
//    V is the same staged tile, read transposed with ds_read_b64_tr_b16.
// No workgroup barrier runs inside the entry loop.  At the end the eight waves
// combine their (max, sum, accumulator) through LDS in a fixed order; splits
// are merged by a second kernel with a fixed-order log-sum-exp combine.  The
// split size depends only on the call shape, never on the batch, so results
// are batch-invariant.  fp8 rows keep their per-row scale out of the MFMA: it
// multiplies the logit and the probability used for PV.
//
// Plain path (fp32 caches): a straightforward fp32 VALU kernel, one workgroup
// per (query, head).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;  // 8: two per SIMD
constexpr int kTile = 16;        // entries per wave step
constexpr int kVsPitch = 528;    // bf16 per staged row: 512 + 16 pad (row stride 8 banks mod 32)
// rows of staged tiles that also hold the merge buffer: 4 waves x 16 heads x 512 floats in 16 x 528 bf16 units
constexpr int kMergeRows = kWaves;  // the combine buffer (4 x 16 heads x 512 floats) fits in 8 staged tiles
static_assert(4 * 16 * 512 * 4 <= kMergeRows * kTile * kVsPitch * 2, "combine buffer fits the staging area");
constexpr int kIdxStage = kAttnMaxSplitEntries;  // selection indices a workgroup stages (the largest split)
constexpr int kRing = 1;         // tiles of rows in flight per wave beyond the one staged (register ring)
constexpr int kQPitch = 520;     // bf16 per staged query head row (512 + 8 pad)
constexpr float kRescale = 8.f;  // lazy rescale threshold (log2 units)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowInfo {
  int b, t, pos, w0, n_cmp, n_tot;
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int row) {
  RowInfo r;
  r.b = row / a.tq;
  r.t = row % a.tq;
  r.pos = __builtin_amdgcn_readfirstlane(a.q_pos[row]);  // row is workgroup-uniform in every caller
  r.w0 = max(0, r.pos - a.window + 1);
  const int n_win = a.window > 0 ? r.pos - r.w0 + 1 : 0;
  r.n_cmp = a.idx ? a.k : visible_blocks(r.pos, a.m_hc);
  r.n_tot = r.n_cmp + n_win;
  return r;
}

// Where a query row's entries live: base addresses and row pitches resolved once
// per workgroup, so that locating entry e is plain integer arithmetic (no
// descriptor selected at run time, which would be re-read from memory).
struct EntrySrc {
  const uint8_t* kv0;   // compressed row 0 of this sequence
  const uint8_t* win0;  // first window row of this query
  int64_t kv_rs, raw_rs;  // row pitches in bytes
  const float* kv_sc;   // fp8 row scales (nullptr otherwise)
  const float* win_sc;
  int64_t kv_ss, raw_ss;
  const int32_t* idx_row;  // CSA selection of this query row (nullptr: HCA, entry e is block e)
};

// eb: bytes per element of the caches (a compile-time constant at every call site)
__device__ __forceinline__ EntrySrc entry_src(const AttnArgs& a, const RowInfo& r, int row, int eb) {
  EntrySrc s;
  const int64_t rr0 = (int64_t)r.w0 - __builtin_amdgcn_readfirstlane(a.raw_base[r.b]);  // raw row of the first window entry
  s.kv0 = (const uint8_t*)a.kv.data + (int64_t)r.b * a.kv.sb * eb;
  s.win0 = (const uint8_t*)a.raw.data + ((int64_t)r.b * a.raw.sb + rr0 * a.raw.sr) * eb;
  s.kv_rs = a.kv.sr * eb;
  s.raw_rs = a.raw.sr * eb;
  const bool fp8 = a.kv.dtype == CSA_FP8_E4M3;
  s.kv_sc = fp8 && a.kv.scale ? (const float*)a.kv.scale + (int64_t)r.b * a.kv.ssb : nullptr;
  s.win_sc = fp8 && a.raw.scale ? (const float*)a.raw.scale + (int64_t)r.b * a.raw.ssb + rr0 * a.raw.ssr : nullptr;
  s.kv_ss = a.kv.ssr;
  s.raw_ss = a.raw.ssr;
  s.idx_row = a.idx ? a.idx + (int64_t)row * a.k : nullptr;
  return s;
}

// Byte pointer to entry e of a row's list (nullptr when the slot is empty) and its row scale.
__device__ __forceinline__ const uint8_t* entry_ptr(const EntrySrc& src, const RowInfo& r, int e, float* sc) {
  *sc = 1.f;
  if (e >= r.n_tot) return nullptr;
  if (e < r.n_cmp) {
    const int j = src.idx_row ? src.idx_row[e] : e;
    if (j < 0) return nullptr;
    if (src.kv_sc) *sc = src.kv_sc[(int64_t)j * src.kv_ss];
    return src.kv0 + (int64_t)j * src.kv_rs;
  }
  const int64_t wr = e - r.n_cmp;
  if (src.win_sc) *sc = src.win_sc[wr * src.raw_ss];
  return src.win0 + wr * src.raw_rs;
}

// Eight consecutive elements of an entry row, as stored: bf16 (16 B) or e4m3 (8 B).
// They stay raw in registers while in flight and are widened to bf16 at use.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool FP8>
using Raw8 = typename std::conditional<FP8, u32x2, u32x4>::type;
typedef __attribute__((address_space(1))) const uint8_t gbyte;

template <bool FP8>
__device__ __forceinline__ Raw8<FP8> load_raw8(const gbyte* p, int col) {
  return *(const __attribute__((address_space(1))) Raw8<FP8>*)(p + (FP8 ? col : 2 * col));
}

template <bool FP8>
__device__ __forceinline__ v8bf widen8(Raw8<FP8> r) {
  if constexpr (!FP8) {
    return __builtin_bit_cast(v8bf, r);
  } else {
    v8bf v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = ((i < 4 ? r[0] : r[1]) >> (8 * (i & 3))) & 0xffu;
      v[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(e4m3_to_f32(byte)) >> 16));  // exact
    }
    return v;
  }
}

// Workgroup -> (row, split, head group).  Consecutive workgroup ids go round robin
// over the 8 XCDs.  With at least 8 rows, every workgroup of row r runs on XCD r % 8:
// the row's splits leave their partial results in that XCD's L2, where the split
// merge (placed the same way) reads them, and the head groups of a split share its
// entry rows there.  With fewer rows, the head groups of one (row, split) get ids 8
// apart (same XCD, shared rows) and the (row, split) pairs spread over the XCDs.
__device__ __forceinline__ void decode_block(int id, int nhg, int nsplit_max, int64_t rows, int* row, int* split,
                                             int* hg) {
  if (rows >= 8) {
    const int x = id % 8, j = id / 8;
    const int per_row = nsplit_max * nhg;
    *row = x + 8 * (j / per_row);
    *split = (j % per_row) / nhg;
    *hg = j % nhg;
    return;
  }
  *hg = (id / 8) % nhg;
  const int c = (id / (8 * nhg)) * 8 + id % 8;  // (row, split) pair
  *row = c / nsplit_max;
  *split = c % nsplit_max;
}

__device__ __forceinline__ float lane_max4rows(float x) {  // max over the 4 lanes n, n+16, n+32, n+48
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

__device__ __forceinline__ float lane_sum4rows(float x) {  // fixed-order sum over the same 4 lanes
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);  // (row r) + (row r+2), identical in both rows
  t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void attn_wave_kernel(AttnArgs a, int split, int nsplit_max, int nhg,
                                                             int partial, int64_t rows) {
  int row, s, hg;
  decode_block(blockIdx.x, nhg, nsplit_max, rows, &row, &s, &hg);
  if (row >= rows) return;
  const int e_begin = s * split;
  // the wave index is made visibly uniform, so per-wave control flow is scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int m = lane % 16, g = lane / 16;  // operand role: entry / head m, k group g
  // A CSA row's compressed entries are its k selection slots, known without reading
  // its position: the indices of each wave's first tile are loaded first (that tile's
  // rows are requested before the workgroup barrier), then the split's indices for
  // the LDS stage, all while the position is in flight.
  __shared__ int sidx[kIdxStage];
  const int32_t* idx_row = a.idx ? a.idx + (int64_t)row * a.k : nullptr;
  const int n_sel = idx_row ? max(0, min(split, a.k - e_begin)) : 0;
  const int32_t* isel = idx_row + e_begin;  // this split's indices (used only when n_sel > 0)
  const int j0 = n_sel > 0 ? isel[min(w * kTile + m, n_sel - 1)] : 0;
  constexpr int kStagePer = kIdxStage / kThreads;
  int stv[kStagePer];
#pragma unroll
  for (int q = 0; q < kStagePer; ++q)
    stv[q] = q * kThreads < n_sel ? isel[min(q * kThreads + (int)threadIdx.x, n_sel - 1)] : 0;
  const RowInfo ri = row_info(a, row);
  const int nsplit = max(1, (ri.n_tot + split - 1) / split);
  if (s >= nsplit) return;  // workgroup-uniform: no barrier has been passed yet
  const EntrySrc src = entry_src(a, ri, row, FP8 ? 1 : 2);
  const int e_end = min(ri.n_tot, e_begin + split);
  const int n_here = e_end - e_begin;
  const int h0 = hg * 16;  // first head of this workgroup
  const bool sel = idx_row != nullptr && ri.n_cmp > 0;

  // each wave's staged tile during the loop; the combine buffer (4 x 16 x 512 floats) afterwards
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kMergeRows][kTile][kVsPitch];
  __shared__ __attribute__((aligned(16))) float esl[kWaves][kTile];  // per-entry scale, -1 = empty
  __shared__ float wml[kWaves][16][2];                                // per-wave (max, sum) per head

  // the workgroup's 16 query heads, staged once in LDS (the QK B operand is read from
  // there: registers hold the row ring instead)
  __shared__ __attribute__((aligned(16))) uint16_t Qs[16][kQPitch];
  const uint16_t* qp = (const uint16_t*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr;
  v8bf qv[16 / kWaves];
#pragma unroll
  for (int hh = 0; hh < 16 / kWaves; ++hh) qv[hh] = *(const v8bf*)(qp + (h0 + (16 / kWaves) * w + hh) * 512 + 8 * lane);

  // This wave's tiles: w, w + 8, w + 16, ... of the split.
  const int ntile = (n_here + kTile - 1) / kTile;
  const int nt = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;

  // Row loads: one instruction per entry row, lane L taking elements 8L .. 8L+7 (a
  // whole row per instruction, the cheapest gather for the memory pipeline), so
  // the row address is scalar.  An empty or out-of-range slot reads this query's
  // own row instead (always a valid address) and gets scale -1.  Tile 0 takes its
  // indices from j0, later tiles from the LDS stage.
  const gbyte* dummy = (const gbyte*)qp;
  Raw8<FP8> kr[kRing][kTile];  // [buffer][row]
  float esc[kRing];            // lane m: entry m's scale (-1 = empty)
  auto load_tile = [&](int i, int buf) {
    const int el = (w + kWaves * i) * kTile + m;  // entry offset in the split (operand role)
    const int e = e_begin + el;
    const bool cmp = e < ri.n_cmp;
    const int j = !cmp ? 0 : sel ? (i == 0 ? j0 : sidx[min(el, n_sel - 1)]) : e;
    const int64_t wr = e - ri.n_cmp;
    const bool live = i < nt && e < e_end && (!cmp || j >= 0);
    const gbyte* p = !live ? dummy
                           : cmp ? (const gbyte*)src.kv0 + (int64_t)j * src.kv_rs
                                 : (const gbyte*)src.win0 + wr * src.raw_rs;
    float sc = live ? 1.f : -1.f;
    if constexpr (FP8) {
      const float* sp = nullptr;
      if (live) sp = cmp ? (src.kv_sc ? src.kv_sc + (int64_t)j * src.kv_ss : nullptr)
                         : (src.win_sc ? src.win_sc + wr * src.raw_ss : nullptr);
      const float v = *(const __attribute__((address_space(1))) float*)(sp ? sp : (const float*)qp);
      if (sp) sc = v;
    }
    esc[buf] = sc;
    const uint64_t pu = (uint64_t)(uintptr_t)p;
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)pu, r), hi = __builtin_amdgcn_readlane((uint32_t)(pu >> 32), r);
      const gbyte* pr = (const gbyte*)(uintptr_t)(((uint64_t)hi << 32) | lo);
      kr[buf][r] = load_raw8<FP8>(pr, 8 * lane);
    }
  };
  // the first tile's rows, before the stage and the barrier
  static_assert(kRing == 1, "the prologue issues exactly one tile ahead");
  load_tile(0, 0);
#pragma unroll
  for (int q = 0; q < kStagePer; ++q)
    if (q * kThreads < n_sel && q * kThreads + (int)threadIdx.x < n_sel) sidx[q * kThreads + threadIdx.x] = stv[q];
#pragma unroll
  for (int hh = 0; hh < 16 / kWaves; ++hh) *(v8bf*)&Qs[(16 / kWaves) * w + hh][8 * lane] = qv[hh];
  __syncthreads();  // sidx and Qs visible

  const float sl2 = a.scale * kLog2e;
  float m_run = kNegInf;  // running max of head m (log2 units), same in all four rows
  float l_part = 0.f;     // this lane's share of head m's running sum
  v4f O[32];              // O[ct]: heads 4g + r, latent column 16ct + m
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) O[ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  auto step = [&](int i, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // stage the tile as bf16 rows in the wave's own LDS area (LDS ops of one wave run
    // in order); an empty fp8 row is zeroed (its stand-in may hold NaN codes)
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      v8bf v = widen8<FP8>(kr[buf][r]);
      if (FP8 && __builtin_amdgcn_readlane(__float_as_uint(esc[buf]), r) == __float_as_uint(-1.f)) v = (v8bf){};
      *(v8bf*)&Vs[w][r][8 * lane] = v;
    }
    if (g == 0) esl[w][m] = esc[buf];
    // the register buffer is free: issue tile i+2's rows into it
    __builtin_amdgcn_sched_barrier(0);
    load_tile(i + kRing, buf);
    __builtin_amdgcn_sched_barrier(0);
    // S^T[entry 4g + r][head m] over the full latent width, four independent chains;
    // A = entry m's columns 32kk + 8g .. +7 read back from the staged tile
    v4f c4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) c4[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      __builtin_amdgcn_sched_barrier(0);  // bounded register use: four k blocks at a time
      v8bf kv[4], qb[4];  // A: entry m's columns; B: Q^T, head m's columns 32kk + 8g .. +7
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kv[u] = *(const v8bf*)&Vs[w][m][32 * (4 * k4 + u) + 8 * g];
        qb[u] = *(const v8bf*)&Qs[m][32 * (4 * k4 + u) + 8 * g];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) c4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[u], qb[u], c4[u], 0, 0, 0);
    }
    const v4f acc = (c4[0] + c4[1]) + (c4[2] + c4[3]);
    const float4 ev = *(const float4*)&esl[w][4 * g];
    const float evr[4] = {ev.x, ev.y, ev.z, ev.w};
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = evr[r] >= 0.f ? (FP8 ? acc[r] * evr[r] : acc[r]) * sl2 : kNegInf;
    const float tmax = lane_max4rows(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescale) != 0) {  // wave-uniform
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
      m_run = m_new;
      float ar[4];  // rescale factors of heads 4g + r (held by lanes 4g + r)
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
      // Scale in place, then pass each tile through an identity MFMA (0 * 0 + C == C):
      // every value of O reaching the loop's merge point is then an MFMA result, so
      // the accumulators stay in accumulation registers instead of being copied out
      // and back on every tile.
      // zeros made here (volatile), not hoisted out of the loop into spilled registers
      u32x4 zu;
      asm volatile("v_mov_b32 %0, 0" : "=v"(zu[0]));
      zu[1] = zu[0];
      zu[2] = zu[0];
      zu[3] = zu[0];
      const v8bf zero8 = __builtin_bit_cast(v8bf, zu);
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[ct][r] *= ar[r];
        O[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero8, zero8, O[ct], 0, 0, 0);
        if (ct % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bounded register traffic
      }
    }
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_run);
      l_part += p;
      pv[r] = FP8 ? p * evr[r] : p;
    }
    // P as hi + lo bf16 terms stacked along the MFMA's k axis: lane (head m, g) holds
    // k = 8g .. 8g+3 -> hi of entries 4g .. 4g+3 and k = 8g+4 .. 8g+7 -> lo of the same
    // entries, so one 16x16x32 MFMA per column tile adds P_hi.V + P_lo.V for the tile.
    v8bf pa;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const __bf16 hi = (__bf16)pv[r];
      pa[r] = hi;
      pa[4 + r] = (__bf16)(pv[r] - (float)hi);
    }
    // V operand: lane (m, g) reads staged rows 4g .. 4g+3 at column 16ct + m (the 16 lanes of
    // a group address 4 rows x 4 column quads) and uses the four values for both halves of k.
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      __builtin_amdgcn_sched_barrier(0);
      v8bf vb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v4bf t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf*)&Vs[w][4 * g + m / 4][16 * (4 * c4 + u) + 4 * (m % 4)]);
        vb[u] = __builtin_shufflevector(t, t, 0, 1, 2, 3, 0, 1, 2, 3);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        O[4 * c4 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[u], O[4 * c4 + u], 0, 0, 0);
    }
  };
  // One tile's rows are in flight while the previous one is processed; the two
  // waves sharing a SIMD cover each other's waits.
  for (int i = 0; i < nt; ++i) step(i, std::integral_constant<int, 0>{});

  // ---- combine the eight waves: (max, sum) per head, then the accumulators
  const float l_w = lane_sum4rows(l_part);
  if (g == 0) {
    wml[w][m][0] = m_run;
    wml[w][m][1] = l_w;
  }
  __syncthreads();
  float wt[4];  // this wave's weight for heads 4g + r: 2^(m_w - M), 0 where the wave saw nothing
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, wml[v][h][0]);
    const float mw = wml[w][h][0];
    wt[r] = mw == kNegInf ? 0.f : exp2f(mw - M);
  }
  // per-head totals over the four waves (every thread, from the table above)
  __shared__ float hML[16][2];
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float Mh = kNegInf, Lh = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) Mh = fmaxf(Mh, wml[v][h][0]);
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = wml[v][h][0];
      Lh += mv == kNegInf ? 0.f : wml[v][h][1] * exp2f(mv - Mh);
    }
    hML[h][0] = Mh;
    hML[h][1] = Lh;
  }
  // Two rounds through LDS, every sum in a fixed order: waves 4..7 write their weighted
  // accumulators, waves 0..3 add them to their own (w + 4 onto w) in place, then every
  // thread adds the four buffers for (column, 4-head group) items.  A buffer is
  // [4-head group][column][4 heads]: lane (m, g) stores heads 4g .. 4g+3 of one column
  // as 16 bytes, consecutive lanes at consecutive addresses.  A wave of 0..3 reads and
  // then rewrites only its own lanes' entries (LDS ops of one wave run in order), so
  // the in-place add needs no barrier and no second copy of the accumulator.
  float* mbuf = (float*)&Vs[0][0][0];  // [4][4][512][4] floats (aliases the staging area)
  __syncthreads();                     // all waves are done with their staged tiles
  const int wb = w % 4;
  if (w >= 4) {
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *(float4*)&mbuf[((wb * 4 + g) * 512 + 16 * ct + m) * 4] =
          make_float4(O[ct][0] * wt[0], O[ct][1] * wt[1], O[ct][2] * wt[2], O[ct][3] * wt[3]);
  }
  __syncthreads();
  if (w < 4) {
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      float4* p = (float4*)&mbuf[((wb * 4 + g) * 512 + 16 * ct + m) * 4];
      const float4 x = *p;
      *p = make_float4(O[ct][0] * wt[0] + x.x, O[ct][1] * wt[1] + x.y, O[ct][2] * wt[2] + x.z,
                       O[ct][3] * wt[3] + x.w);
    }
  }
  __syncthreads();
  const int H = a.heads;
  float* obase = partial ? (float*)a.ws + (((int64_t)row * nsplit_max + s) * H + h0) * 512
                         : a.out + ((int64_t)row * H + h0) * 512;
  // item -> (4-head group, column) with the column fastest: a wave reads 64 consecutive
  // 16-byte buffer entries (no bank conflict) and each of its stores covers 64
  // consecutive columns of one head
#pragma unroll
  for (int it = 0; it < 512 * 4 / kThreads; ++it) {
    const int item = threadIdx.x + kThreads * it, hq = item / 512, c = item % 512;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int v = 0; v < 4; ++v) {  // fixed order over the four buffers
      const float4 x = *(const float4*)&mbuf[((v * 4 + hq) * 512 + c) * 4];
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    const float av[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float L = hML[4 * hq + r][1];
      const float fs = partial ? 1.f : (L > 0.f ? __fdiv_rn(1.0f, L) : 0.f);
      if (partial)
        obase[(4 * hq + r) * 512 + c] = av[r];  // kept in this XCD's L2 for the split merge
      else
        __builtin_nontemporal_store(av[r] * fs, &obase[(4 * hq + r) * 512 + c]);  // streamed: read once, elsewhere
    }
  }
  if (threadIdx.x < 16) {
    const int hglob = h0 + threadIdx.x;
    const float Mh = hML[threadIdx.x][0], Lh = hML[threadIdx.x][1];
    if (partial) {
      float* pml = (float*)a.ws + rows * nsplit_max * H * 512 + (((int64_t)row * nsplit_max + s) * H + hglob) * 2;
      pml[0] = Mh;
      pml[1] = Lh;
    } else if (a.lse) {
      a.lse[(int64_t)row * H + hglob] = Lh > 0.f ? (Mh + log2f(Lh)) * kLn2 : kNegInf;
    }
  }
}

// Streaming (non-temporal) float4 store: data written once and read elsewhere, kept out
// of the way of the caches.
__device__ __forceinline__ void nt_store4(float4 x, float4* p) {
  __builtin_nontemporal_store((v4f){x.x, x.y, x.z, x.w}, (v4f*)p);
}

// Fixed-order log-sum-exp merge of the splits of one (row, head); one pass over
// the partials with every split's row in flight at once.
constexpr int kMergeMaxSplits = kAttnMaxSplits;
constexpr int kMergeBatch = 8;  // splits whose partial rows are loaded up front

__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int split, int nsplit_max, int64_t rows) {
  const int row = blockIdx.x, h = blockIdx.y;
  const int H = a.heads;
  // the first kMergeBatch splits' partial rows are loaded before anything else (they
  // depend on nothing), so the position, the (max, sum) pairs and the rows arrive together
  const float4* src = (const float4*)((const float*)a.ws + ((int64_t)row * nsplit_max * H + h) * 512) + threadIdx.x;
  const int64_t sstride = (int64_t)H * 512 / 4;  // float4s between consecutive splits
  float4 pv[kMergeBatch];
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j)
    pv[j] = j < nsplit_max ? src[j * sstride] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float* pml = (const float*)a.ws + rows * nsplit_max * H * 512;
  float ms = kNegInf, ls = 0.f;
  if (threadIdx.x < kWave && (int)threadIdx.x < nsplit_max) {
    const int64_t o = (((int64_t)row * nsplit_max + threadIdx.x) * H + h) * 2;
    ms = pml[o];
    ls = pml[o + 1];
  }
  const RowInfo ri = row_info(a, row);
  const int nsplit = min(kMergeMaxSplits, max(1, (ri.n_tot + split - 1) / split));
  __shared__ float wts[kMergeMaxSplits];
  __shared__ float sh_L, sh_M;
  if (threadIdx.x < kWave) {  // one wave forms the split weights
    const int s = threadIdx.x;
    if (s >= nsplit) ms = kNegInf, ls = 0.f;
    const float M = wave_max(ms);
    const float e = (M == kNegInf || s >= nsplit) ? 0.f : exp2f(ms - M);
    // L = sum over splits in ascending order (fixed, independent of scheduling)
    float L = 0.f;
    for (int i = 0; i < nsplit; ++i) L += __shfl(ls * e, i);
    if (s < kMergeMaxSplits) wts[s] = e;
    if (s == 0) {
      sh_L = L;
      sh_M = M;
    }
  }
  __syncthreads();
  const float L = sh_L;
  const float inv = L > 0.f ? __fdiv_rn(1.0f, L) : 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
    if (j >= nsplit) break;  // splits past this row's count are never read into the sum
    const float wgt = wts[j] * inv;
    acc.x = fmaf(pv[j].x, wgt, acc.x);
    acc.y = fmaf(pv[j].y, wgt, acc.y);
    acc.z = fmaf(pv[j].z, wgt, acc.z);
    acc.w = fmaf(pv[j].w, wgt, acc.w);
  }
  for (int s = kMergeBatch; s < nsplit; ++s) {
    const float wgt = wts[s] * inv;
    const float4 v = src[s * sstride];
    acc.x = fmaf(v.x, wgt, acc.x);
    acc.y = fmaf(v.y, wgt, acc.y);
    acc.z = fmaf(v.z, wgt, acc.z);
    acc.w = fmaf(v.w, wgt, acc.w);
  }
  nt_store4(acc, &((float4*)(a.out + ((int64_t)row * H + h) * 512))[threadIdx.x]);
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)row * H + h] = L > 0.f ? (sh_M + log2f(L)) * kLn2 : kNegInf;
}

// ------------------------------------------------------------------ fp32 VALU path
constexpr int kPlainThreads = 128;
constexpr int kPlainMaxEntries = 8192;

__global__ __launch_bounds__(kPlainThreads) void attn_plain_kernel(AttnArgs a) {
  const int row = blockIdx.x, h = blockIdx.y;
  const RowInfo ri = row_info(a, row);
  const EntrySrc src = entry_src(a, ri, row, 4);
  __shared__ float logit[kPlainMaxEntries];
  __shared__ float qs[512];
  __shared__ float red[kPlainThreads / kWave];
  const int D = a.dim;
  const float* qp = (const float*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr + (int64_t)h * D;
  for (int d = threadIdx.x; d < D; d += kPlainThreads) qs[d] = qp[d];
  __syncthreads();
  float mx = kNegInf;
  for (int e = threadIdx.x; e < ri.n_tot; e += kPlainThreads) {
    float sc;
    const float* p = (const float*)entry_ptr(src, ri, e, &sc);
    float l = kNegInf;
    if (p) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], p[d], dot);
      l = dot * a.scale;
    }
    logit[e] = l;
    mx = fmaxf(mx, l);
  }
  mx = wave_max(mx);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float sum = 0.f;
  for (int e = threadIdx.x; e < ri.n_tot; e += kPlainThreads) {
    const float p = mx == kNegInf ? 0.f : expf(logit[e] - mx);
    logit[e] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  const float inv = sum > 0.f ? __fdiv_rn(1.0f, sum) : 0.f;
  for (int d = threadIdx.x; d < D; d += kPlainThreads) {
    float acc = 0.f;
    for (int e = 0; e < ri.n_tot; ++e) {
      float sc;
      const float* p = (const float*)entry_ptr(src, ri, e, &sc);
      if (p) acc = fmaf(logit[e], p[d], acc);
    }
    a.out[((int64_t)row * a.heads + h) * D + d] = acc * inv;
  }
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)row * a.heads + h] = sum > 0.f ? mx + logf(sum) : kNegInf;
}

hipError_t launch_decode(const AttnArgs& a, int64_t rows, int split, int nsplit_max, hipStream_t s) {
  const int partial = nsplit_max > 1;
  const int nhg = a.heads / 16;
  const int64_t pairs = rows * nsplit_max;
  const int64_t blocks = rows >= 8 ? (rows + 7) / 8 * 8 * nsplit_max * nhg : (pairs + 7) / 8 * 8 * nhg;
  if (a.kv.dtype == CSA_FP8_E4M3)
    hipLaunchKernelGGL(attn_wave_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a, split, nsplit_max,
                       nhg, partial, rows);
  else
    hipLaunchKernelGGL(attn_wave_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a, split, nsplit_max,
                       nhg, partial, rows);
  if (partial)
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)rows, a.heads), dim3(128), 0, s, a, split, nsplit_max, rows);
  return hipGetLastError();
}

}  // namespace

// Splits depend only on the call shape (decode or not) and the entry capacity,
// never on the batch, so each sequence's arithmetic is batch-invariant.  Decode
// cuts a row's list into eight splits of whole 16-entry tiles, at least one tile
// per wave (8 rows x 4 head groups x 8 splits fill the 256 CUs at batch 8); calls
// with many queries per sequence keep each list whole.
int attn_split_size(int tq, int n_entries_max) {
  const int n = max(n_entries_max, 1);
  if (tq != 1) return min(n, kIdxStage);
  const int eighth = ((n + 7) / 8 + kTile - 1) / kTile * kTile;
  return min(kIdxStage, max(kWaves * kTile, eighth));  // at least a tile per wave
}

size_t attn_workspace_bytes(int64_t rows, int heads, int dim, int n_entries_max, int tq) {
  const int split = attn_split_size(tq, n_entries_max);
  const int64_t nsplit = (n_entries_max + split - 1) / split;
  if (nsplit <= 1) return 0;
  return (size_t)rows * nsplit * heads * (dim + 2) * sizeof(float);
}

bool attn_plain_fits(int n_entries_max) { return n_entries_max <= kPlainMaxEntries; }

hipError_t launch_attention(const AttnArgs& a, int n_entries_max, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.tq;
  if (rows == 0) return hipSuccess;
  if (a.kv.dtype == CSA_F32) {
    hipLaunchKernelGGL(attn_plain_kernel, dim3((unsigned)rows, a.heads), dim3(kPlainThreads), 0, s, a);
    return hipGetLastError();
  }
  const int split = attn_split_size(a.tq, n_entries_max);
  const int nsplit_max = max(1, (n_entries_max + split - 1) / split);
  if (nsplit_max > kMergeMaxSplits) return hipErrorInvalidValue;
  return launch_decode(a, rows, split, nsplit_max, s);
}

}  // namespace csa

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
// (PV), both on bf16 MFMA.  A workgroup (4 waves) takes one query row, one
// group of 16 heads and one contiguous split of the entry list.  Each wave is
// an independent flash-decoding worker over every 4th tile of 16 entries:
//  * it loads whole entry rows (each lane 16 x 16 B of one row, the MFMA A
//    layout) two tiles ahead of use, with the selection indices a further
//    tile ahead, so row loads never wait behind an index load;
//  * QK computes the transposed logits S^T = K Q^T (16x16x32), which leaves
//    each lane holding four entries of one head -- exactly the A-operand
//    layout PV needs for P, so P never moves between lanes;
//  * the online softmax reduces over entries within the wave (register max,
//    then two cross-row lane swaps) and rescales the accumulator lazily: only
//    when a head's running maximum grows by more than 2^8, which keeps every
//    probability <= 256 and skips almost all rescaling work;
//  * P goes to PV as two bf16 terms (hi + lo, ~16 significant bits instead of
//    bf16's 8), stacked along the k axis of one 16x16x32 MFMA per column tile;
//    V is the same tile, staged in the wave's own LDS area and read transposed
//    with ds_read_b64_tr_b16.
// No workgroup barrier runs inside the entry loop.  At the end the four waves
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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;        // entries per wave step
constexpr int kVsPitch = 528;    // bf16 per staged row: 512 + 16 pad (row stride 8 banks mod 32)
constexpr int kMbufPitch = 516;  // floats per head row of the merge buffer (512 + 4 pad)
// rows of staged tiles that also hold the merge buffer: 4 x 16 x 516 floats in 16 x 528 bf16 units
constexpr int kMergeRows = (kWaves * 16 * kMbufPitch * 4 + kTile * kVsPitch * 2 - 1) / (kTile * kVsPitch * 2);
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

// Workgroup -> (row, split, head group).  Consecutive workgroup ids go to
// different XCDs (round robin over 8), so the nhg head groups of one
// (row, split) get ids 8 apart: same XCD, same L2, run side by side, and the
// entry rows the first one fetches from HBM are L2 hits for the others.
__device__ __forceinline__ void decode_block(int id, int nhg, int nsplit_max, int* row, int* split, int* hg) {
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
  decode_block(blockIdx.x, nhg, nsplit_max, &row, &s, &hg);
  if (row >= rows) return;
  const RowInfo ri = row_info(a, row);
  const int nsplit = max(1, (ri.n_tot + split - 1) / split);
  if (s >= nsplit) return;
  const EntrySrc src = entry_src(a, ri, row, FP8 ? 1 : 2);
  const int e_begin = s * split, e_end = min(ri.n_tot, e_begin + split);
  const int h0 = hg * 16;  // first head of this workgroup

  // the wave index is made visibly uniform, so per-wave control flow is scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int m = lane % 16, g = lane / 16;  // load role: entry m of a tile; softmax role: head m

  // staged tiles during the loop; the merge buffer (kWaves x 16 x kMbufPitch floats) afterwards
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kMergeRows][kTile][kVsPitch];
  __shared__ __attribute__((aligned(16))) float esl[kWaves][kTile];              // per-entry scale, -1 = empty
  __shared__ float wml[kWaves][16][2];                                            // per-wave (max, sum) per head

  // Q^T as the QK B operand: head h0 + m, latent columns 32kk + 8g .. +7
  const uint16_t* qp = (const uint16_t*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr;
  v8bf qb[16];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) qb[kk] = *(const v8bf*)(qp + (h0 + m) * 512 + 32 * kk + 8 * g);

  // This wave's tiles: w, w + 4, w + 8, ... of the split.
  const int ntile = (e_end - e_begin + kTile - 1) / kTile;
  const int nt = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;
  auto tile_e0 = [&](int i) { return e_begin + (w + kWaves * i) * kTile; };

  // Loads are unconditional: an empty or out-of-range slot reads this query's own
  // row instead (always a valid address), zeroes it, and is masked by a -1 scale.
  const gbyte* dummy = (const gbyte*)qp;
  const bool sel = src.idx_row != nullptr && ri.n_cmp > 0;
  auto load_idx = [&](int i) {
    const int e = tile_e0(i) + m;
    return sel ? src.idx_row[min(e, ri.n_cmp - 1)] : e;
  };
  Raw8<FP8> kr[2][16];
  float esc[2], scl[2];
  bool hs[2] = {false, false};
  auto load_tile = [&](int i, int j, int buf) {
    const int e = tile_e0(i) + m;
    const bool cmp = e < ri.n_cmp;
    const int64_t wr = e - ri.n_cmp;
    const bool live = i < nt && e < e_end && (!cmp || j >= 0);
    const gbyte* p = !live ? dummy
                           : cmp ? (const gbyte*)src.kv0 + (int64_t)j * src.kv_rs
                                 : (const gbyte*)src.win0 + wr * src.raw_rs;
    esc[buf] = live ? 1.f : -1.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) kr[buf][kk] = load_raw8<FP8>(p, 32 * kk + 8 * g);
    if constexpr (FP8) {
      const float* sp = nullptr;
      if (live) sp = cmp ? (src.kv_sc ? src.kv_sc + (int64_t)j * src.kv_ss : nullptr)
                         : (src.win_sc ? src.win_sc + wr * src.raw_ss : nullptr);
      scl[buf] = *(const __attribute__((address_space(1))) float*)(sp ? sp : (const float*)qp);
      hs[buf] = sp != nullptr;  // the stand-in value is never used
    }
  };

  const float sl2 = a.scale * kLog2e;
  float m_run = kNegInf;  // running max of head m (log2 units), same in all four rows
  float l_part = 0.f;     // this lane's share of head m's running sum
  v4f O[32];              // O[ct]: heads 4g + r, latent column 16ct + m
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) O[ct] = (v4f){0.f, 0.f, 0.f, 0.f};

  // pipeline: rows of tiles i+1 and i+2 in flight while tile i is processed; the
  // index of tile i+2 was loaded before tile i+1's rows, so using it never waits on them
  const int j0 = load_idx(0), j1 = load_idx(1);
  int jn2 = load_idx(2);
  load_tile(0, j0, 0);
  load_tile(1, j1, 1);
  auto step = [&](int i, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (g == 0) esl[w][m] = FP8 && hs[buf] ? scl[buf] : esc[buf];
    v8bf kv[16];
    // an fp8 stand-in row may hold NaN codes: zero it (a bf16 one is finite query data)
    const bool dead = FP8 && esc[buf] < 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      kv[kk] = widen8<FP8>(kr[buf][kk]);
      if (dead) kv[kk] = (v8bf){};
    }
    // S^T[entry 4g + r][head m] over the full latent width, four independent chains
    v4f c4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) c4[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      c4[kk % 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[kk], qb[kk], c4[kk % 4], 0, 0, 0);
    // stage the tile for PV (wave-private area; LDS ops of one wave run in order)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) *(v8bf*)&Vs[w][m][32 * kk + 8 * g] = kv[kk];
    // the buffer is free: issue tile i+3's index, then tile i+2's rows
    __builtin_amdgcn_sched_barrier(0);
    {
      const int j2 = jn2;
      jn2 = load_idx(i + 3);
      load_tile(i + 2, j2, buf);
    }
    __builtin_amdgcn_sched_barrier(0);
    const v4f acc = (c4[0] + c4[1]) + (c4[2] + c4[3]);
    const float4 ev = *(const float4*)&esl[w][4 * g];
    const float evr[4] = {ev.x, ev.y, ev.z, ev.w};
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = evr[r] >= 0.f ? acc[r] * evr[r] * sl2 : kNegInf;
    const float tmax = lane_max4rows(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescale) != 0) {  // wave-uniform
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_run == kNegInf ? 0.f : exp2f(m_run - m_new);
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
      const float p = m_run == kNegInf ? 0.f : exp2f(sv[r] - m_run);
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
    typedef __attribute__((address_space(3))) v4bf lds_v4bf;
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
  // Both steps of the loop body are unconditional and an odd last tile is peeled
  // off after the loop, so every path into the loop head has both row buffers in
  // flight: the wait counts the compiler derives then wait for exactly one tile,
  // never for the one behind it.
  int i = 0;
  for (; i + 1 < nt; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
  }
  if (i < nt) step(i, std::integral_constant<int, 0>{});

  // ---- combine the four waves: (max, sum) per head, then the accumulators in column chunks
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
    const float M = fmaxf(fmaxf(wml[0][h][0], wml[1][h][0]), fmaxf(wml[2][h][0], wml[3][h][0]));
    const float mw = wml[w][h][0];
    wt[r] = mw == kNegInf ? 0.f : exp2f(mw - M);
  }
  // reducer role: wave w finalises heads 4w + lane/16, columns 8(lane%16) .. +7 of each chunk
  const int rh = 4 * w + lane / 16, rc = 8 * (lane % 16);
  float Mh = kNegInf, Lh = 0.f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) Mh = fmaxf(Mh, wml[v][rh][0]);
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float mv = wml[v][rh][0];
    Lh += mv == kNegInf ? 0.f : wml[v][rh][1] * exp2f(mv - Mh);
  }
  const int H = a.heads;
  const int hglob = h0 + rh;
  float* orow;
  float fscale;
  if (partial) {
    orow = (float*)a.ws + (((int64_t)row * nsplit_max + s) * H + hglob) * 512;
    fscale = 1.f;
  } else {
    orow = a.out + ((int64_t)row * H + hglob) * 512;
    fscale = Lh > 0.f ? __fdiv_rn(1.0f, Lh) : 0.f;
  }
  // one pass: every wave writes its weighted accumulator (all 512 columns), then each
  // wave sums four heads over the four buffers in a fixed order
  float* mbuf = (float*)&Vs[0][0][0];  // [kWaves][16][kMbufPitch] floats (aliases the staging area)
  __syncthreads();                     // all waves are done with their staged tiles
#pragma unroll
  for (int ct = 0; ct < 32; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) mbuf[(w * 16 + 4 * g + r) * kMbufPitch + 16 * ct + m] = O[ct][r] * wt[r];
  __syncthreads();
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {  // fixed order over waves
      const float4 x0 = *(const float4*)&mbuf[(v * 16 + rh) * kMbufPitch + 128 * ch + rc];
      const float4 x1 = *(const float4*)&mbuf[(v * 16 + rh) * kMbufPitch + 128 * ch + rc + 4];
      acc0.x += x0.x; acc0.y += x0.y; acc0.z += x0.z; acc0.w += x0.w;
      acc1.x += x1.x; acc1.y += x1.y; acc1.z += x1.z; acc1.w += x1.w;
    }
    acc0.x *= fscale; acc0.y *= fscale; acc0.z *= fscale; acc0.w *= fscale;
    acc1.x *= fscale; acc1.y *= fscale; acc1.z *= fscale; acc1.w *= fscale;
    *(float4*)&orow[128 * ch + rc] = acc0;
    *(float4*)&orow[128 * ch + rc + 4] = acc1;
  }
  if (lane % 16 == 0) {
    if (partial) {
      float* pml = (float*)a.ws + rows * nsplit_max * H * 512 + (((int64_t)row * nsplit_max + s) * H + hglob) * 2;
      pml[0] = Mh;
      pml[1] = Lh;
    } else if (a.lse) {
      a.lse[(int64_t)row * H + hglob] = Lh > 0.f ? (Mh + log2f(Lh)) * kLn2 : kNegInf;
    }
  }
}

// Fixed-order log-sum-exp merge of the splits of one (row, head); one pass over
// the partials with every split's row in flight at once.
constexpr int kMergeMaxSplits = 64;

__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int split, int nsplit_max, int64_t rows) {
  const int row = blockIdx.x, h = blockIdx.y;
  const RowInfo ri = row_info(a, row);
  const int nsplit = min(kMergeMaxSplits, max(1, (ri.n_tot + split - 1) / split));
  const int H = a.heads;
  const float* pml = (const float*)a.ws + rows * nsplit_max * H * 512;
  __shared__ float wts[kMergeMaxSplits];
  __shared__ float sh_L, sh_M;
  if (threadIdx.x < kWave) {  // one wave forms the split weights
    const int s = threadIdx.x;
    const int64_t o = (((int64_t)row * nsplit_max + s) * H + h) * 2;
    const float ms = s < nsplit ? pml[o] : kNegInf;
    const float ls = s < nsplit ? pml[o + 1] : 0.f;
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
  const float4* src = (const float4*)((const float*)a.ws + ((int64_t)row * nsplit_max * H + h) * 512) + threadIdx.x;
  const int64_t sstride = (int64_t)H * 512 / 4;  // float4s between consecutive splits
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = wts[s] * inv;
    const float4 v = src[s * sstride];
    acc.x = fmaf(v.x, wgt, acc.x);
    acc.y = fmaf(v.y, wgt, acc.y);
    acc.z = fmaf(v.z, wgt, acc.z);
    acc.w = fmaf(v.w, wgt, acc.w);
  }
  ((float4*)(a.out + ((int64_t)row * H + h) * 512))[threadIdx.x] = acc;
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
  const int64_t blocks = (pairs + 7) / 8 * 8 * nhg;
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
// cuts a row's list into about eight splits of whole 64-entry rounds (one tile
// per wave); calls with many queries per sequence keep each list whole.
int attn_split_size(int tq, int n_entries_max) {
  const int n = max(n_entries_max, 1);
  if (tq != 1) return n;
  const int round = kWaves * kTile;
  return max(round, ((n + 7) / 8 + round - 1) / round * round);
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

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
// heads (two groups, sharing the gathered rows, for calls with many queries per
// sequence) and one contiguous split of the entry list, and walks the split in
// chunks of up to 136 entries that sit whole in LDS (one 1 KB row per entry):
//  * the chunk's rows are all requested at once, one row per wave instruction,
//    straight into LDS (bf16; fp8 rows are widened through registers), so a
//    chunk costs one memory round trip, not one per tile;
//  * QK computes the transposed logits S^T = K Q^T (16x16x32), eight waves over
//    the chunk's 16-entry tiles, with the 16 query heads held in registers as
//    the B operand and K read from LDS;
//  * one max per head over the chunk (online across chunks), then P as two bf16
//    terms (hi + lo, ~16 significant bits) written to LDS in the PV operand
//    layout; per-head sums are added in a fixed order;
//  * PV splits the 512 latent columns over the waves (64 each), reading V
//    transposed with ds_read_b64_tr_b16: every wave's accumulator is final for
//    its columns, so no cross-wave combine is needed.
// Splits are merged by a second kernel with a fixed-order log-sum-exp combine.
// The split and chunk sizes depend only on the call shape, never on the batch,
// so results are batch-invariant.  fp8 rows keep their per-row scale out of the
// MFMA: it multiplies the logit and the probability used for PV.
//
// Plain path (fp32 caches): a straightforward fp32 VALU kernel, one workgroup
// per (query, head).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kTile = 16;  // entries per MFMA tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowInfo {
  int b, t, pos, w0, n_cmp, n_tot;
};

// The row's position and entry counts (row is workgroup-uniform in every caller).
__device__ __forceinline__ RowInfo row_info(const int32_t* q_pos, bool csa, int k, int tq, int window, int m_hc,
                                            int row) {
  RowInfo r;
  r.b = row / tq;
  r.t = row % tq;
  r.pos = __builtin_amdgcn_readfirstlane(q_pos[row]);
  r.w0 = max(0, r.pos - window + 1);
  const int n_win = window > 0 ? r.pos - r.w0 + 1 : 0;
  r.n_cmp = csa ? k : visible_blocks(r.pos, m_hc);
  r.n_tot = r.n_cmp + n_win;
  return r;
}

__device__ __forceinline__ RowInfo row_info(const AttnArgs& a, int row) {
  return row_info(a.q_pos, a.idx != nullptr, a.k, a.tq, a.window, a.m_hc, row);
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
  const uint8_t* kv_bs;   // MXFP4 block scales: dim / 32 bytes per row (nullptr otherwise)
  const uint8_t* win_bs;
  int64_t kv_ss, raw_ss;  // scale row pitches (fp8: floats, MXFP4: bytes)
  const int32_t* idx_row;  // CSA selection of this query row (nullptr: HCA, entry e is block e)
};

// eb, ebr: bytes per stride unit of the compressed and of the raw rows (elements;
// MXFP4 strides are in bytes), compile-time constants at every call site
// rb: raw_base[r.b], the absolute position of the sequence's raw row 0.
__device__ __forceinline__ EntrySrc entry_src(const AttnArgs& a, const RowInfo& r, int row, int eb, int ebr, int rb) {
  EntrySrc s;
  const int64_t rr0 = (int64_t)r.w0 - rb;  // raw row of the first window entry
  s.kv0 = (const uint8_t*)a.kv.data + (int64_t)r.b * a.kv.sb * eb;
  s.win0 = (const uint8_t*)a.raw.data + ((int64_t)r.b * a.raw.sb + rr0 * a.raw.sr) * ebr;
  s.kv_rs = a.kv.sr * eb;
  s.raw_rs = a.raw.sr * ebr;
  const bool fp8 = a.kv.dtype == CSA_FP8_E4M3;
  s.kv_sc = fp8 && a.kv.scale ? (const float*)a.kv.scale + (int64_t)r.b * a.kv.ssb : nullptr;
  s.win_sc = fp8 && a.raw.scale ? (const float*)a.raw.scale + (int64_t)r.b * a.raw.ssb + rr0 * a.raw.ssr : nullptr;
  const bool fp4 = a.kv.dtype == CSA_MXFP4;
  s.kv_bs = fp4 ? (const uint8_t*)a.kv.scale + (int64_t)r.b * a.kv.ssb : nullptr;
  s.win_bs = nullptr;  // MXFP4 caches take bf16 window rows
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
  } else {  // OCP e4m3 -> bf16 in hardware (exact: 3 mantissa bits, exponents within range)
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, true);
    return (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
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

// Row formats of the MFMA path.
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtFp4 = 2;

// Eight MXFP4 elements (one 32-bit word of codes, element 2i in the low nibble of
// byte i) times their block scale 2^(sb - 127), as bf16: exact for every code and
// every scale that keeps the value in the normal range (the products are powers of
// two times at most two significant bits).
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t codes, uint32_t sb) {
  const float sc = __uint_as_float(sb ? sb << 23 : 0x00400000u);  // 2^(sb-127); sb = 0 is 2^-127
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
  return (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
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

// Chunk of a split's entries resident in LDS: up to CH rows of 512 bf16 (1
// KB), 16-byte chunk c of row r stored at position c ^ swz(r) (swz(r) = r mod 16),
// so that the 16 consecutive rows of a QK operand read fall on distinct banks.  The last 16-entry tile of a full chunk reaches 8 rows past the buffer (into
// the region after it): those entries are masked out of QK, and PV zeroes what it
// reads there.
constexpr int kRowBytes = 1024;

// NW waves per head group, HG head groups of 16 per workgroup, chunks of at most CH entries.
template <int NW, int CH, bool QL, int HG>
struct ChunkLds {
  static constexpr int kTiles = (CH + 15) / 16;
  __attribute__((aligned(16))) uint8_t rows[CH][kRowBytes];
  union {
    // QL: the 16 query heads, staged once (same swizzle as the rows) and read into
    // registers before P is first written (otherwise they pass through the rows buffer
    // before the first chunk)
    __attribute__((aligned(16))) uint8_t q[QL ? 16 : 1][kRowBytes];
    // P as the PV A operand: [tile][k group g][head m] -> 4 bf16 hi then 4 bf16 lo
    // of entries 16*tile + 4g .. +3
    __attribute__((aligned(16))) uint4 p[HG][kTiles][4][16];
  };
  float esl[kTiles * 16];     // entry scale (fp8 row scale, else 1); -1 = empty slot
  int32_t sidx[kTiles * 16];  // slots of the chunk
  __attribute__((aligned(16))) float red_max[NW * HG][16];
  __attribute__((aligned(16))) float red_sum[NW * HG][16];
};

__device__ __forceinline__ int swz(int r) { return r & 15; }
__device__ __forceinline__ int swz_off(int r, int chunk16) { return r * kRowBytes + ((chunk16 ^ swz(r)) << 4); }

// One workgroup: one query row, HG groups of 16 heads, one split of its entry list,
// processed in chunks of at most CH entries by NW waves per head group (the head
// groups share the chunk's rows; everything after the gather is per head group, so a
// head's arithmetic is the same for every HG).  For each chunk:
//  * the chunk's selection slots go to LDS, then every wave issues its rows (one
//    row per instruction, straight into LDS for bf16; fp8 rows pass through
//    registers to be widened, with their scales);
//  * QK: S^T = K Q^T on 16x16x32 bf16 MFMA, the waves over the chunk's 16-entry
//    tiles, with the 16 query heads held in registers (B operand) and K read from LDS;
//  * one workgroup max per head (online across chunks), P = exp2(s - max) written
//    to LDS as hi + lo bf16 in the PV operand layout, per-head sums in a fixed order;
//  * PV with the latent columns split over the waves (wave w owns 512 / NW columns
//    of all 16 heads): the accumulator of a wave is final for its columns, so the
//    waves never combine accumulators.
// The scalars the prologue depends on come first in the argument list: they are
// preloaded into scalar registers at launch (the rest of the arguments is read from
// memory, one round trip that overlaps the position and slot loads).
template <int FMT, int NW, int CH, bool QL, int HG>
__global__ __launch_bounds__(NW * HG * kWave) __attribute__((amdgpu_waves_per_eu(2))) void attn_chunk_kernel(
    const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ raw_base, int k, int tq, int window, int m_hc,
    int split, int nsplit_max, int nhg, int rows, AttnArgs a) {
  constexpr int kT = (CH + 15) / 16;             // 16-entry tiles of a full chunk
  constexpr int kQkT = (kT + NW - 1) / NW;       // QK tiles per wave
  constexpr int kCols = 512 / NW, kNT = kCols / 16;  // PV: latent columns per wave, their 16-column tiles
  constexpr int NWT = NW * HG;                   // waves of the workgroup
  constexpr int kRW = (CH + NWT - 1) / NWT;      // rows a wave loads per chunk
  constexpr bool FP8 = FMT == kFmtFp8;
  static_assert(HG == 1 || !QL, "several head groups stage their query heads through the rows buffer");
  int row, s, hg;
  decode_block(blockIdx.x, nhg, nsplit_max, rows, &row, &s, &hg);
  if (row >= rows) return;
  // wave wt of the workgroup is wave w of head group hgl: every wave loads rows, a head
  // group's NW waves share its QK tiles and split its PV columns
  const int wt = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int hgl = HG > 1 ? wt / NW : 0, w = HG > 1 ? wt % NW : wt;
  const int m = lane % 16, g = lane / 16;
  const int t = threadIdx.x;
  const int e_begin = s * split;
  const int nch = (split + CH - 1) / CH;  // chunk size depends on the split only
  const int csz = (split + nch - 1) / nch;
  // A CSA row's compressed entries are its k selection slots, known without its
  // position: the first chunk's slots are requested before the position, so the two
  // memory round trips overlap.
  const int32_t* idx_row = idx ? idx + (int64_t)row * k : nullptr;
  int jn = -1;
  if (idx_row && t < csz && e_begin + t < k) jn = idx_row[e_begin + t];
  const int rb = __builtin_amdgcn_readfirstlane(raw_base[row / tq]);
  const RowInfo ri = row_info(q_pos, idx != nullptr, k, tq, window, m_hc, row);
  // (computed before the early exit below: its argument reads then join the
  // position's round trip)
  const EntrySrc src = entry_src(a, ri, row, FMT == kFmtBf16 ? 2 : 1, FMT == kFmtFp8 ? 1 : 2, rb);
  const int partial = nsplit_max > 1;
  const int nsplit = max(1, (ri.n_tot + split - 1) / split);
  if (s >= nsplit) return;  // workgroup-uniform, before any barrier
  const int e_end = min(ri.n_tot, e_begin + split);
  const int h0 = (hg * HG + hgl) * 16;

  __shared__ ChunkLds<NW, CH, QL, HG> L;
  uint8_t* const rowb = &L.rows[0][0];  // the chunk's rows as one byte array

  // the 16 query heads as the QK B operand: lane (head m, group g) holds columns
  // 32kk + 8g .. +7 of head m, kk = 0 .. 15 (requested after the first chunk's rows)
  const uint16_t* qp = (const uint16_t*)a.q.data + (int64_t)ri.b * a.q.sb + (int64_t)ri.t * a.q.sr;
  v8bf qb[16];
  const gbyte* dummy = (const gbyte*)qp;  // a finite 1 KB row for empty bf16 slots
  if constexpr (!QL) {
    // the 16 query heads pass through the (still free) rows buffer once, before the
    // first chunk: one 16 KB read per workgroup, overlapping the first slots' load
    static_assert(CH >= 16 * HG, "query heads fit the rows buffer");
#pragma unroll
    for (int hh = (16 / NW) * wt; hh < (16 / NW) * (wt + 1); ++hh)
      __builtin_amdgcn_global_load_lds((const gbyte*)(qp + (hg * HG * 16 + hh) * 512) + 16 * (lane ^ swz(hh)),
                                       (__attribute__((address_space(3))) void*)&L.rows[hh][0], 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qb[kk] = *(const v8bf*)&rowb[swz_off(16 * hgl + m, 4 * kk + g)];
    __syncthreads();  // the rows buffer is free again
  }

  const float sl2 = a.scale * kLog2e;
  // running (max, sum) of heads 4g + r (the PV layout) and max of head m (the QK layout)
  float mrun[4], lrun[4], mrun_q = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) mrun[r] = kNegInf, lrun[r] = 0.f;
  v4f O[kNT];  // O[nt]: heads 4g + r, latent column kCols * w + 16nt + m
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) O[nt] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int c0 = e_begin; c0 < e_end; c0 += csz) {
    const int cn = min(csz, e_end - c0);  // entries of this chunk
    const int nmt = (cn + 15) / 16;       // 16-entry tiles
    // the chunk's slots (-1 = empty); esl marks live entries (fp8: the row scale,
    // filled in with the row)
    if (t < nmt * 16) {
      const int e = c0 + t;
      int j = -1;
      if (t < cn) j = e >= ri.n_cmp ? 0 : idx_row ? jn : e;
      L.sidx[t] = j;
      L.esl[t] = j >= 0 ? 1.f : -1.f;
    }
    __syncthreads();
    // rows: wave wt loads rows wt, wt + NWT, ... of the chunk's tiles (lane i holds
    // the slot of the wave's i-th row, so no row waits on an LDS read)
    const int nrows = min(nmt * 16, CH);
    const int jw = lane < (nrows - wt + NWT - 1) / NWT ? L.sidx[wt + NWT * lane] : -1;
    // fp8 / MXFP4 rows pass through registers: all of the wave's rows are requested
    // first, then widened into LDS once the query heads and next slots are in flight
    // (MXFP4 caches take bf16 window rows, which go straight to LDS)
    uint32_t rc[kRW][FP8 ? 2 : 1];  // the lane's 8 elements as stored
    uint32_t rs[kRW];               // fp8: row scale bits; MXFP4: block scale byte
    if constexpr (FMT == kFmtBf16) {
      for (int r = wt, ri8 = 0; r < nrows; r += NWT, ++ri8) {
        const int e = c0 + r;
        const int j = __builtin_amdgcn_readlane(jw, ri8);
        const gbyte* rp = j < 0 ? dummy
                                : e < ri.n_cmp ? (const gbyte*)src.kv0 + (int64_t)j * src.kv_rs
                                               : (const gbyte*)src.win0 + (int64_t)(e - ri.n_cmp) * src.raw_rs;
        // lane l fills LDS chunk l of the row with the row's chunk l ^ swz(r)
        __builtin_amdgcn_global_load_lds(rp + 16 * (lane ^ swz(r)), (__attribute__((address_space(3))) void*)&L.rows[r][0],
                                         16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRW; ++i) {
        const int r = wt + NWT * i, e = c0 + r;
        rc[i][0] = 0u;
        if constexpr (FP8) rc[i][1] = 0u;
        rs[i] = FP8 ? __float_as_uint(1.f) : 127u;
        const int j = __builtin_amdgcn_readlane(jw, i);
        if (r < nrows && j >= 0) {  // wave-uniform
          const bool cmp = e < ri.n_cmp;
          const int64_t er = cmp ? j : e - ri.n_cmp;
          const gbyte* rp = (const gbyte*)(cmp ? src.kv0 : src.win0) + er * (cmp ? src.kv_rs : src.raw_rs);
          if constexpr (FP8) {
            const u32x2 v = *(const __attribute__((address_space(1))) u32x2*)(rp + 8 * lane);
            rc[i][0] = v[0];
            rc[i][1] = v[1];
            const float* sp = cmp ? src.kv_sc : src.win_sc;
            if (sp) rs[i] = __float_as_uint(sp[er * (cmp ? src.kv_ss : src.raw_ss)]);
          } else if (cmp) {
            rc[i][0] = *(const __attribute__((address_space(1))) uint32_t*)(rp + 4 * lane);
            rs[i] = *(const __attribute__((address_space(1))) uint8_t*)(src.kv_bs + er * src.kv_ss + lane / 4);
          } else {  // bf16 window row
            __builtin_amdgcn_global_load_lds(rp + 16 * (lane ^ swz(r)),
                                             (__attribute__((address_space(3))) void*)&L.rows[r][0], 16, 0, 0);
          }
        }
      }
    }
    if (c0 == e_begin) {
      if constexpr (QL) {  // the 16 query heads to LDS, 16 / NW per wave
#pragma unroll
        for (int hh = (16 / NW) * w; hh < (16 / NW) * (w + 1); ++hh)
          __builtin_amdgcn_global_load_lds((const gbyte*)(qp + (h0 + hh) * 512) + 16 * (lane ^ swz(hh)),
                                           (__attribute__((address_space(3))) void*)&L.q[hh][0], 16, 0, 0);
      }
    }
    // the next chunk's slots, requested while this chunk's rows are in flight
    jn = -1;
    if (idx_row && t < csz && c0 + csz + t < min(k, e_end)) jn = idx_row[c0 + csz + t];
    if constexpr (FMT != kFmtBf16) {
#pragma unroll
      for (int i = 0; i < kRW; ++i) {
        const int r = wt + NWT * i;
        if (r < nrows) {
          if constexpr (FP8) {
            *(v8bf*)&rowb[swz_off(r, lane)] = widen8<true>((u32x2){rc[i][0], rc[i][1]});
            if (lane == 0 && __builtin_amdgcn_readlane(jw, i) >= 0) L.esl[r] = __uint_as_float(rs[i]);
          } else if (!(c0 + r >= ri.n_cmp && __builtin_amdgcn_readlane(jw, i) >= 0)) {  // not a window row
            *(v8bf*)&rowb[swz_off(r, lane)] = fp4x8_to_bf16(rc[i][0], rs[i]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // rows (and the first time, the query heads) in LDS
    if (QL && c0 == e_begin) {
      const uint8_t* qs = &L.q[0][0];
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) qb[kk] = *(const v8bf*)&qs[swz_off(m, 4 * kk + g)];
    }

    // ---- QK: tiles w, w + NW, ... of the chunk; lane (head m, g) gets entries 16mt + 4g + r
    float sv[kQkT][4];
    float lmax = kNegInf;
#pragma unroll
    for (int ti = 0; ti < kQkT; ++ti) {
      const int mt = w + NW * ti;
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[ti][r] = kNegInf;
      if (mt < nmt) {  // wave-uniform
        v4f c4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c4[u] = (v4f){0.f, 0.f, 0.f, 0.f};
        const int er = 16 * mt + m;  // the row this lane reads (A operand: entry m of the tile)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          v8bf kv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) kv[u] = *(const v8bf*)&rowb[swz_off(er, 4 * (4 * k4 + u) + g)];
#pragma unroll
          for (int u = 0; u < 4; ++u) c4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[u], qb[4 * k4 + u], c4[u], 0, 0, 0);
        }
        const v4f acc = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        const float4 ev = *(const float4*)&L.esl[16 * mt + 4 * g];
        const float evr[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[ti][r] = evr[r] >= 0.f ? (FP8 ? acc[r] * evr[r] : acc[r]) * sl2 : kNegInf;
          lmax = fmaxf(lmax, sv[ti][r]);
        }
      }
    }
    lmax = lane_max4rows(lmax);
    if (g == 0) L.red_max[wt][m] = lmax;
    __syncthreads();
    // chunk maxima, the same in every wave (fixed order)
    float mc_q = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) mc_q = fmaxf(mc_q, L.red_max[NW * hgl + v][m]);
    const float mnew_q = fmaxf(mrun_q, mc_q);
    mrun_q = mnew_q;
    float lsum = 0.f;
#pragma unroll
    for (int ti = 0; ti < kQkT; ++ti) {
      const int mt = w + NW * ti;
      if (mt < nmt) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = mnew_q == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sv[ti][r] - mnew_q);
          lsum += p;
          pv[r] = FP8 ? p * L.esl[16 * mt + 4 * g + r] : p;
        }
        // P as hi + lo bf16 (about 16 significant bits): k = 8g .. 8g+3 hi, 8g+4 .. 8g+7 lo
        v8bf pa;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 hi = (__bf16)pv[r];
          pa[r] = hi;
          pa[4 + r] = (__bf16)(pv[r] - (float)hi);
        }
        L.p[hgl][mt][g][m] = __builtin_bit_cast(uint4, pa);
      }
    }
    lsum = lane_sum4rows(lsum);
    if (g == 0) L.red_sum[wt][m] = lsum;
    __syncthreads();  // P and the per-wave sums visible
    // running statistics of heads 4g + r and the accumulator rescale
    float mcv[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, lsv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < NW; ++v) {  // heads 4g .. 4g+3: one 16-byte read per table and wave
      const float4 mx = *(const float4*)&L.red_max[NW * hgl + v][4 * g];
      const float4 sm = *(const float4*)&L.red_sum[NW * hgl + v][4 * g];
      mcv[0] = fmaxf(mcv[0], mx.x), mcv[1] = fmaxf(mcv[1], mx.y), mcv[2] = fmaxf(mcv[2], mx.z), mcv[3] = fmaxf(mcv[3], mx.w);
      lsv[0] += sm.x, lsv[1] += sm.y, lsv[2] += sm.z, lsv[3] += sm.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mc = mcv[r], ls = lsv[r];
      const float mn = fmaxf(mrun[r], mc);
      const float alpha = mrun[r] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mrun[r] - mn);
      lrun[r] = lrun[r] * alpha + ls;
      mrun[r] = mn;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) O[nt][r] *= alpha;
    }
    // ---- PV: O[16 heads x this wave's kCols columns] += P V over the chunk's tiles
    typedef __attribute__((address_space(3))) v4bf lds_v4bf;
    // operands of tile ks: P (16 B per lane) and kNT transposed V reads (rows
    // 16ks + 4g .. +3, columns kCols*w + 16nt .. +15: lane m addresses row m / 4,
    // columns 4(m % 4) .. +3 and receives column m of the four rows); two operand
    // sets alternate, so tile ks + 1's reads are in flight during tile ks's MFMAs
    const auto pv_load = [&](int ks, v8bf& pa, v4bf (&tv)[kNT]) {
      pa = __builtin_bit_cast(v8bf, L.p[hgl][ks][g][m]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int col = kCols * w + 16 * nt + 4 * (m % 4);
        tv[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf*)&rowb[swz_off(16 * ks + 4 * g + m / 4, col / 8) + 2 * (col % 8)]);
      }
    };
    // P hi and P lo in two 16x16x16 MFMAs on the same transposed V read (no operand
    // copies).  Only a chunk's last tile can reach past the buffer (CH not a multiple of
    // 16): there the lanes that read past it take zeros (whatever lies after the buffer
    // must not reach other entries' heads, e.g. a NaN in one head's query).
    typedef short v4s __attribute__((ext_vector_type(4)));
    const auto pv_mfma = [&](int ks, const v8bf& pa, const v4bf (&tv)[kNT]) {
      const v4s ph = __builtin_bit_cast(v4s, __builtin_shufflevector(pa, pa, 0, 1, 2, 3));
      const v4s pl = __builtin_bit_cast(v4s, __builtin_shufflevector(pa, pa, 4, 5, 6, 7));
      const auto run = [&](auto masked) {
        const bool past = decltype(masked)::value && 16 * ks + 4 * g + m / 4 >= CH;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const v4s vb = past ? (v4s){0, 0, 0, 0} : __builtin_bit_cast(v4s, tv[nt]);
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, O[nt], 0, 0, 0);
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, O[nt], 0, 0, 0);
        }
      };
      if (16 * ks + 16 > CH)  // wave-uniform
        run(std::true_type{});
      else
        run(std::false_type{});
    };
    {
      v8bf pa0, pa1;
      v4bf tv0[kNT], tv1[kNT];
      pv_load(0, pa0, tv0);
      int ks = 0;
      for (; ks + 1 < nmt; ks += 2) {
        pv_load(ks + 1, pa1, tv1);
        pv_mfma(ks, pa0, tv0);
        if (ks + 2 < nmt) pv_load(ks + 2, pa0, tv0);
        pv_mfma(ks + 1, pa1, tv1);
      }
      if (ks < nmt) pv_mfma(ks, pa0, tv0);
    }
    __syncthreads();  // the chunk's rows, P and tables are free for the next chunk
  }

  // ---- output: this wave's kCols columns of the 16 heads
  const int H = a.heads;
  if (partial) {
    float* obase = (float*)a.ws + (((int64_t)row * nsplit_max + s) * H + h0) * 512;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) obase[(4 * g + r) * 512 + kCols * w + 16 * nt + m] = O[nt][r];
    if (w == 0 && m == 0) {
      float* pml = (float*)a.ws + (int64_t)rows * nsplit_max * H * 512 + (((int64_t)row * nsplit_max + s) * H + h0) * 2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pml[(4 * g + r) * 2] = mrun[r];
        pml[(4 * g + r) * 2 + 1] = lrun[r];
      }
    }
  } else {
    float* obase = a.out + ((int64_t)row * H + h0) * 512;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float fs = lrun[r] > 0.f ? __fdiv_rn(1.0f, lrun[r]) : 0.f;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        __builtin_nontemporal_store(O[nt][r] * fs, &obase[(4 * g + r) * 512 + kCols * w + 16 * nt + m]);
    }
    if (a.lse && w == 0 && m == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.lse[(int64_t)row * H + h0 + 4 * g + r] = lrun[r] > 0.f ? (mrun[r] + log2f(lrun[r])) * kLn2 : kNegInf;
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
    const float le = ls * e;
    float L = 0.f;
    for (int i = 0; i < nsplit; ++i) L += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(le), i));
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
  const EntrySrc src = entry_src(a, ri, row, 4, 4, a.raw_base[ri.b]);
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
  const int64_t pairs = rows * nsplit_max;
  // CSA decode: 8 waves and chunks of 136 entries (one workgroup per CU; a split of 272
  // entries is two chunks).  Many queries per sequence, and HCA: two head groups of 4
  // waves each share chunks of 128 entries (whole tiles; a 640-entry list is five
  // chunks), the query heads staged once through the rows buffer into registers before
  // the first chunk (one workgroup per CU).  With 16 or 48 heads: one head group, chunks
  // of 64 (many queries) or 56 (HCA decode; 75 KB of LDS), two workgroups per CU.  Measured on
  // the 2k prefill chunks (CSA / HCA us per call): one head group, 56-entry chunks
  // 799 / 747, 64-entry 706 / 711; two head groups with 64-entry chunks 704 / 716 (the
  // gather is halved, the time is not: the per-chunk chain bounds it), 96-entry 645 /
  // 619, 128-entry 576 / 602; the query heads read from LDS at every chunk instead of
  // held in registers (LDS for 112-entry chunks at most) 668 / 634.  HCA decode at
  // batch 64: one head group with 56-entry chunks 61.9 us per step, two with 128-entry
  // chunks 56.7 (96-entry 56.8); the hybrid pair's HCA layer 53.1 -> 48.4 us.
  const int fmt = a.kv.dtype == CSA_FP8_E4M3 ? kFmtFp8 : a.kv.dtype == CSA_MXFP4 ? kFmtFp4 : kFmtBf16;
  const bool many = a.tq != 1;
  // HCA (dense over every visible block; long lists at large batch) takes a 4-wave shape
  // per head group.  The shape is chosen by the call kind and the head count, never by
  // the batch, so results stay batch-invariant.
  const bool hca = a.idx == nullptr;
  // calls with many queries per sequence and HCA calls, with 32 or 64 heads: two head
  // groups per workgroup share one gather of the rows
  const int hgw = (many || hca) && a.heads % 32 == 0 ? 2 : 1;
  const int nhg = a.heads / 16 / hgw;
  const int64_t blocks = rows >= 8 ? (rows + 7) / 8 * 8 * nsplit_max * nhg : (pairs + 7) / 8 * 8 * nhg;
  const dim3 grid((unsigned)blocks);
#define CSA_ATTN_LAUNCH(F, NW, CH, QL, HG)                                                                          \
  hipLaunchKernelGGL((attn_chunk_kernel<F, NW, CH, QL, HG>), grid, dim3(NW * HG * kWave), 0, s, a.q_pos, a.idx,    \
                     a.raw_base, a.k, a.tq, a.window, a.m_hc, split, nsplit_max, nhg, (int)rows, a)
#define CSA_ATTN_SHAPES(F)                                  \
  if (hgw > 1) CSA_ATTN_LAUNCH(F, 4, 128, false, 2);         \
  else if (many) CSA_ATTN_LAUNCH(F, 4, 64, false, 1);       \
  else if (hca) CSA_ATTN_LAUNCH(F, 4, 56, true, 1);         \
  else CSA_ATTN_LAUNCH(F, 8, 136, true, 1);
  if (fmt == kFmtFp8) {
    CSA_ATTN_SHAPES(kFmtFp8)
  } else if (fmt == kFmtFp4) {
    CSA_ATTN_SHAPES(kFmtFp4)
  } else {
    CSA_ATTN_SHAPES(kFmtBf16)
  }
#undef CSA_ATTN_SHAPES
#undef CSA_ATTN_LAUNCH
  if (partial)
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)rows, a.heads), dim3(128), 0, s, a, split, nsplit_max, rows);
  return hipGetLastError();
}

}  // namespace

// Splits depend only on the call kind, the call shape (decode or not) and the entry
// capacity, never on the batch, so each sequence's arithmetic is batch-invariant.
// CSA decode cuts a row's list into eight splits of whole 16-entry tiles, at least
// eight tiles each (8 rows x 4 head groups x 8 splits fill the 256 CUs at batch 8);
// HCA decode (dense lists, large batches) into quarters, which halves the split
// partials the merge reads (batch 64: 69 -> 61 us per step; the hybrid pair's HCA
// layer at batch 32: 61 -> 53 us); calls with many queries per sequence keep each list
// whole.  HCA never cuts more splits than CSA at the same list length, so the CSA
// workspace size bounds both.
int attn_split_size(int tq, int n_entries_max, bool dense) {
  const int n = max(n_entries_max, 1);
  if (tq != 1) return min(n, kAttnMaxSplitEntries);
  const int parts = dense ? 4 : 8;
  const int part = ((n + parts - 1) / parts + kTile - 1) / kTile * kTile;
  return min(kAttnMaxSplitEntries, max(8 * kTile, part));
}

size_t attn_workspace_bytes(int64_t rows, int heads, int dim, int n_entries_max, int tq) {
  const int split = attn_split_size(tq, n_entries_max, false);  // the larger of the two policies
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
  const int split = attn_split_size(a.tq, n_entries_max, a.idx == nullptr);
  const int nsplit_max = max(1, (n_entries_max + split - 1) / split);
  if (nsplit_max > kMergeMaxSplits) return hipErrorInvalidValue;
  return launch_decode(a, rows, split, nsplit_max, s);
}

}  // namespace csa

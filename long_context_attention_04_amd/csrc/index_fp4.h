// MXFP4 lightning-indexer scoring pieces shared by the indexer kernel and the
// top-k merge's rescoring fallback: one code path, so a block rescored later
// gets bitwise the score the indexer gave it.
//
// The indexer scores compressed blocks from low-rank projections of the query
// (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
// bullet) with the query-key path in FP4 (same page, item 4, Quantization-Aware
// Training).  Reading of the score: I = sum_h w_h * relu(<q_h, kappa_j>).
//
// Operand layout.  A 32-key tile is scored by one scaled FP4 MFMA.  Each lane
// loads one 16-byte MX block (32 e2m1 codes) and its e8m0 scale: exactly one
// operand slot, so block scales are applied by the matrix core.  Up to 8 heads
// use a block-diagonal 16x16x128 MFMA (heads in rows 0-7 over K 0-63 and again
// in rows 8-15 over K 64-127; keys 0-15 of the tile in K 0-63, keys 16-31 in
// K 64-127): 32 keys per MFMA with a 4-register accumulator.  Up to 32 heads
// use the 32x32x64 MFMA (rows = heads, columns = keys).
#pragma once
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kFp4Unroll = 8;                        // 32-key tiles per wave
constexpr int kFp4KeysPerWave = 32 * kFp4Unroll;     // 256
constexpr int kFp4KeysPerWG = 4 * kFp4KeysPerWave;   // 1024: one candidate slice
// Query element pairs per thread of the 256 that quantise it: heads * 32 pairs.
template <int NR>
struct Fp4Pairs {
  static constexpr int n = NR == 4 ? 1 : 4;  // heads <= 8 : heads <= 32
};

// The MXFP4 query of one row and its head weights, in LDS.
struct Fp4QueryLds {
  __attribute__((aligned(16))) uint32_t code[32][2][4];  // [head][K block][16 B of e2m1 codes]
  uint32_t scale[32][2];                                 // e8m0
  float w[32];
};

// The row's fp32 query as element pairs; t in [0, 256) is the thread's index in the
// 256-thread group that quantises it (thread -> head, K block, pair; the 16 threads of
// a 32-element block are 16 adjacent lanes).
// NP pairs per thread cover NP * 8 heads (NP = 1 for heads <= 8, 4 for heads <= 32).
template <int NP>
__device__ __forceinline__ void fp4_query_load(const IndexArgs& a, int b, int t_q, int t, float2 (&x)[NP]) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pi = 256 * i + t;
    const int h = pi / 32, blk = (pi / 16) % 2, pr = pi % 16;
    x[i] = h < a.heads ? *(const float2*)((const float*)a.q.data + (int64_t)b * a.q.sb + (int64_t)t_q * a.q.sr +
                                          h * 64 + 32 * blk + 2 * pr)
                       : make_float2(0.f, 0.f);
  }
}

// Quantises the loaded pairs to MXFP4 into LDS (same t as fp4_query_load; called by
// whole waves of the 256-thread group).
template <int NP>
__device__ __forceinline__ void fp4_query_quantize(const IndexArgs& a, int t, const float2 (&xs)[NP], Fp4QueryLds& ql) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (256 * i < a.heads * 32) {  // uniform
      const int pi = 256 * i + t;
      const int h = pi / 32, blk = (pi / 16) % 2, pr = pi % 16;
      const float2 x = xs[i];
      float amax = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
      const int e = mx_scale_exp(amax);
      const uint32_t byte = amax > 0.f ? (f32_to_e2m1(x.x, e) | (f32_to_e2m1(x.y, e) << 4)) : 0u;
      // four adjacent pairs form one dword of codes
      const uint32_t b1 = __shfl_down(byte, 1, 16), b2 = __shfl_down(byte, 2, 16), b3 = __shfl_down(byte, 3, 16);
      if (h < a.heads) {
        if ((pr & 3) == 0) ql.code[h][blk][pr / 4] = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
        if (pr == 0) ql.scale[h][blk] = (uint32_t)(e + 127);
      }
    }
  }
}

// A lane's role in the tile MFMA.  NR: accumulator rows that can hold a real head,
// 4 (heads <= 8, block-diagonal 16x16x128) or 16 (heads <= 32, 32x32x64).
template <int NR>
struct Fp4Lane {
  static constexpr bool kDiag = NR == 4;
  static constexpr int kPair = kDiag ? 16 : 32;  // the lane holding the same key's other heads
  int m;   // key within the 32-key tile this lane loads
  int kb;  // K block (32 elements) of that key
  __device__ __forceinline__ explicit Fp4Lane(int l)
      : m(kDiag ? 16 * (l / 32) + l % 16 : l % 32), kb(kDiag ? (l / 16) % 2 : l / 32) {}
};

// The query A operand and its e8m0 scale for lane l (from LDS, after the quantising
// group's barrier), and this lane's accumulator rows' head weights.
template <int NR>
__device__ __forceinline__ void fp4_query_operand(const Fp4QueryLds& ql, int heads, int l, v8i* A, int* sa,
                                                  float (&wv)[NR]) {
  constexpr bool kDiag = NR == 4;
  const int qrow = kDiag ? l % 16 : l % 32, qblk = kDiag ? l / 16 : l / 32;
  const bool qlive = kDiag ? (qrow < 8) == (qblk < 2) : true;  // off-diagonal blocks are zero
  const int qh = kDiag ? qrow % 8 : qrow;
  *A = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
  *sa = 127;
  if (qlive && qh < heads) {
    const uint4 qv = *(const uint4*)&ql.code[qh][qblk % 2][0];
    (*A)[0] = (int)qv.x;
    (*A)[1] = (int)qv.y;
    (*A)[2] = (int)qv.z;
    (*A)[3] = (int)qv.w;
    *sa = (int)ql.scale[qh][qblk % 2];
  }
  // accumulator rows r hold heads 8*(r/4) + 4*kb + r%4 (both layouts)
  const int kb = kDiag ? (l / 16) % 2 : l / 32;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int h = 8 * (r / 4) + 4 * kb + (r % 4);
    wv[r] = h < heads ? ql.w[h] : 0.f;
  }
}

// The score of this lane's key (tile key Fp4Lane::m), identical in lanes l and
// l ^ kPair: one MFMA, ReLU, head weights, one cross-lane add.
template <int NR>
__device__ __forceinline__ float fp4_tile_score(const v8i& A, int sa, const float (&wv)[NR], v4i c, int sbk) {
  const v8i Bop = {c[0], c[1], c[2], c[3], 0, 0, 0, 0};
  // ReLU as one integer max on the bits (a negative float is a negative integer; -0 and
  // every negative value give +0); the float max form costs a canonicalize too
  const auto relu = [](float x) { return __int_as_float(max(__float_as_int(x), 0)); };
  float part = 0.f;
  if constexpr (NR == 4) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bop, acc, 4, 4, 0, sa, 0, sbk);
#pragma unroll
    for (int r = 0; r < 4; ++r) part = fmaf(wv[r], relu(acc[r]), part);
  } else {
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bop, acc, 4, 4, 0, sa, 0, sbk);
#pragma unroll
    for (int r = 0; r < NR; ++r) part = fmaf(wv[r], relu(acc[r]), part);
  }
  // part of lane l plus part of lane l ^ kPair: a lane swap within the VALU (no LDS
  // round trip); the sum is the same in both lanes (addition commutes)
  const uint32_t x = __float_as_uint(part);
  const auto t = Fp4Lane<NR>::kPair == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                                          : __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Scores of chosen 32-key tiles of one row (only keys < V; the rest score as
// absent) recomputed by a whole workgroup (a multiple of 256 threads) with the
// indexer's arithmetic, tile by tile: tile_key(i) is the first key of tile i (a
// multiple of 32, as in the indexer), store(i, key, score, live) is called once per
// key by the lane holding it.  Used when a selection needs scores the indexer did
// not write.  Starts and ends with a workgroup barrier (the caller's LDS is free to
// reuse before; ql and whatever store wrote are readable by the workgroup after).
template <int NR, typename TileKey, typename Store>
__device__ __forceinline__ void fp4_rescore_tiles(const IndexArgs& a, int row, int V, Fp4QueryLds& ql, int ntile, TileKey tile_key,
                                  Store store) {
  const int b = row / a.tq, t_q = row % a.tq;
  const int t = threadIdx.x, l = t % kWave, w = t / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (t < 256) {
    float2 qx[Fp4Pairs<NR>::n];
    fp4_query_load(a, b, t_q, t, qx);
    fp4_query_quantize(a, t, qx, ql);
    if (t < a.heads) ql.w[t] = a.w[(int64_t)row * a.heads + t];
  }
  __syncthreads();
  v8i A;
  int sa;
  float wv[NR];
  fp4_query_operand<NR>(ql, a.heads, l, &A, &sa, wv);
  const Fp4Lane<NR> ln(l);
  constexpr int kU = NR == 4 ? 4 : 2;  // tiles in flight per wave: their loads are issued together
  for (int t0 = w; t0 < ntile; t0 += kU * nw) {
    v4i c[kU];
    int sbk[kU], key[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tile = t0 + u * nw;
      key[u] = tile < ntile ? tile_key(tile) + ln.m : V;
      const bool live = key[u] < V;
      const int64_t kk = live ? key[u] : 0;
      c[u] = live ? *(const v4i*)((const uint8_t*)a.k.data + (int64_t)b * a.k.sb + kk * a.k.sr + 16 * ln.kb)
                  : (v4i){0, 0, 0, 0};
      sbk[u] = live ? ((const uint8_t*)a.k.scale)[(int64_t)b * a.k.ssb + kk * a.k.ssr + ln.kb] : 127;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tile = t0 + u * nw;  // wave-uniform
      if (tile < ntile) {
        const float s = fp4_tile_score<NR>(A, sa, wv, c[u], sbk[u]);
        if (ln.kb == 0) store(tile, key[u], s, key[u] < V);
      }
    }
  }
  __syncthreads();
}

// Every visible score of one row (keys 0 .. V-1) recomputed and written to srow.
template <int NR>
__device__ __forceinline__ void fp4_rescore_row(const IndexArgs& a, int row, int V, Fp4QueryLds& ql, float* srow) {
  fp4_rescore_tiles<NR>(
      a, row, V, ql, (V + 31) / 32, [](int tile) { return 32 * tile; },
      [&](int, int key, float s, bool live) {
        if (live) srow[key] = s;
      });
  __threadfence();
  __syncthreads();
}

}  // namespace
}  // namespace csa

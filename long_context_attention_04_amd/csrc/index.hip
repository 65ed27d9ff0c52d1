// (b) Lightning-indexer scores.
//
// The indexer scores compressed blocks from low-rank projections of the
// query (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1,
// CSA bullet), with the QK path in FP4 (same page, item 4, Quantization-Aware
// Training).  Reading of the score: I = sum_h w_h * relu(<q_h, kappa_j>).
//
// Three kernels, one per key format:
//  * MXFP4 keys: the key stream is the dominant HBM traffic of long-context
//    decode (34 B per key).  Each wave streams 32 keys per step straight into
//    the B operand of one scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
//    lane l carries key l%32's 32-element block l/32 (16 B of codes) and that
//    block's e8m0 scale, so the block scales are applied by the matrix core and
//    no dequantisation happens on the VALU.  Query heads are the MFMA rows
//    (quantised to MXFP4 in-kernel once per workgroup).  ReLU, head weights and
//    the cross-head sum are a short epilogue (one cross-lane add).
//  * BF16 keys: bf16 MFMA 16x16x32 with (query, head) pairs as rows, keys as
//    columns; one kernel for few queries per sequence (decode: the key stream
//    dominates) and a 32-query x 256-key tile kernel for many (a prefill chunk: a
//    dense contraction of many queries against the same keys).
//  * F32 keys: plain fp32 VALU kernel (small shapes).
#include <type_traits>

#include "common.h"
#include "compress_block.h"
#include "kernels.h"
#include "index_fp4.h"
#include "select.h"

namespace csa {

namespace {

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ fp32 VALU
constexpr int kPlainThreads = 256;

__global__ __launch_bounds__(kPlainThreads) void index_plain_kernel(IndexArgs a) {
  extern __shared__ float qs[];  // [heads * dim]
  const int row = blockIdx.y;
  const int b = row / a.tq, t = row % a.tq;
  const int HD = a.heads * a.dim;
  const int64_t qoff = (int64_t)b * a.q.sb + (int64_t)t * a.q.sr;
  for (int i = threadIdx.x; i < HD; i += kPlainThreads) qs[i] = load_elem(a.q.data, a.q.dtype, qoff + i);
  __syncthreads();
  const int j = blockIdx.x * kPlainThreads + threadIdx.x;
  if (j >= a.n_cap) return;
  const int V = visible_blocks(a.q_pos[row], a.m);
  float score = kNegInf;
  if (j < V) {
    const int64_t koff = (int64_t)b * a.k.sb + (int64_t)j * a.k.sr;
    score = 0.f;
    for (int h = 0; h < a.heads; ++h) {
      float dot = 0.f;
      for (int d = 0; d < a.dim; ++d) dot = fmaf(qs[h * a.dim + d], load_elem(a.k.data, a.k.dtype, koff + d), dot);
      score = fmaf(a.w[(int64_t)row * a.heads + h], fmaxf(dot, 0.f), score);
    }
  }
  a.scores[(int64_t)row * a.n_cap + j] = score;
}

// ------------------------------------------------------------------ bf16 MFMA
// heads == 8, dim == 64.  Workgroup tile: 16 queries x 128 keys; each of the 4
// waves takes 32 keys (2 column tiles of 16) for all 16 queries (8 row tiles
// of 2 queries x 8 heads).
constexpr int kBfQT = 16;
constexpr int kBfKT = 128;

__global__ __launch_bounds__(256) void index_bf16_kernel(IndexArgs a) {
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * kBfQT;
  const int kbase = blockIdx.x * kBfKT;
  const int wave = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int g = l / 16, n = l % 16;

  int Vmax = 0;
  for (int i = 0; i < kBfQT && q0 + i < a.tq; ++i) Vmax = max(Vmax, visible_blocks(a.q_pos[b * a.tq + q0 + i], a.m));

  // B operands: key = kbase + 32*wave + 16*nt + n ; k-step ks covers dims 32*ks + 8*g .. +7
  v8bf B[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = kbase + 32 * wave + 16 * nt + n;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (key < Vmax) {
        const uint16_t* p = (const uint16_t*)a.k.data + (int64_t)b * a.k.sb + (int64_t)key * a.k.sr + 32 * ks + 8 * g;
        B[nt][ks] = *(const v8bf*)p;
      } else {
        for (int e = 0; e < 8; ++e) B[nt][ks][e] = (__bf16)0.f;
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < kBfQT / 2; ++mt) {
    const int qa = q0 + 2 * mt;  // row tile = queries qa, qa+1; row m -> query qa + m/8, head m%8
    if (qa >= a.tq) break;
    // A operand: row m = n (lane%16), dims 32*ks + 8*g .. +7
    const int qq = qa + n / 8, hh = n % 8;
    v8bf A[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (qq < a.tq) {
        const int64_t off = (int64_t)b * a.q.sb + (int64_t)qq * a.q.sr + hh * 64 + 32 * ks + 8 * g;
        A[ks] = *(const v8bf*)((const uint16_t*)a.q.data + off);
      } else {
        for (int e = 0; e < 8; ++e) A[ks][e] = (__bf16)0.f;
      }
    }
    // this lane's output rows: m = 4g + r -> query qa + (g >= 2), heads 4*(g&1) + r
    const int myq = qa + (g >> 1);
    float wv[4];
    const int Vq = myq < a.tq ? visible_blocks(a.q_pos[b * a.tq + myq], a.m) : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r] = myq < a.tq ? a.w[((int64_t)b * a.tq + myq) * 8 + 4 * (g & 1) + r] : 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], B[nt][1], c, 0, 0, 0);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(wv[r], fmaxf(c[r], 0.f), part);
      const float other = __shfl_xor(part, 16);
      const float tot = (g & 1) ? other + part : part + other;  // heads 0-3 first, then 4-7
      const int key = kbase + 32 * wave + 16 * nt + n;
      if ((g & 1) == 0 && myq < a.tq && key < a.n_cap)
        a.scores[((int64_t)b * a.tq + myq) * a.n_cap + key] = key < Vq ? tot : kNegInf;
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA, many queries
// heads == 8, dim == 64, many queries per sequence (a prefill chunk): a dense
// [queries*8 x 64] x [64 x keys] contraction.  Workgroup tile: 72 queries x 1024
// keys, 8 waves.  The 72 queries' heads are staged once in LDS (A operand); each wave
// holds its 128 keys in registers as the B operand for all 36 row tiles, so a key is
// loaded once per workgroup.  The epilogue (ReLU, head weights, the sum over heads)
// is the same arithmetic in the same order as index_bf16_kernel: bit-identical
// scores.  The tile is sized so that the whole grid is resident at once (2,048
// queries over 16,896 keys: 29 x 17 = 493 workgroups, two per CU by LDS): the
// staging round trip is paid once, not once per round.
constexpr int kPfQ = 72;        // queries per workgroup
constexpr int kPfNT = 8;        // 16-key column tiles per wave (a multiple of 4)
constexpr int kPfWaves = 8;
constexpr int kPfKeys = kPfWaves * 16 * kPfNT;  // keys per workgroup (1024)
static_assert(kPfQ % 4 == 0 && kPfQ * 8 * 8 % (64 * kPfWaves) == 0, "query quads; whole staging rounds");
constexpr int kPfMinTq = 32;  // chunks of fewer queries take index_bf16_kernel

// 4x4 transpose across the four lanes of each lane quad: lane i holds x[0..3] = M[i][.];
// afterwards lane i holds M[.][i].  Two exchange stages (partner lane i ^ 1, then i ^ 2),
// each one DPP move and selects per exchanged pair.
__device__ __forceinline__ void quad_transpose4(float (&x)[4]) {
  const int i = threadIdx.x & 3;
  {
    const bool odd = i & 1;
    const float r0 = dpp_f32<0xB1>(odd ? x[0] : x[1]), r1 = dpp_f32<0xB1>(odd ? x[2] : x[3]);
    x[0] = odd ? r0 : x[0];
    x[1] = odd ? x[1] : r0;
    x[2] = odd ? r1 : x[2];
    x[3] = odd ? x[3] : r1;
  }
  {
    const bool hi = i & 2;
    const float r0 = dpp_f32<0x4E>(hi ? x[0] : x[2]), r1 = dpp_f32<0x4E>(hi ? x[1] : x[3]);
    x[0] = hi ? r0 : x[0];
    x[2] = hi ? x[2] : r0;
    x[1] = hi ? r1 : x[1];
    x[3] = hi ? x[3] : r1;
  }
}

// max(x, 0) as one integer max on the bits (a negative float is a negative integer;
// -0 and every negative value give +0): the float max form costs a canonicalize too
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// (a 128-register budget: the MFMA accumulators then stay in VGPRs, so the epilogue
// reads them without AGPR copies)
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(4))) void index_bf16_tile_kernel(IndexArgs a) {
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * kPfQ;
  const int kbase = blockIdx.x * kPfKeys;
  const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t / kWave), l = t % kWave;
  const int g = l / 16, n = l % 16;
  // A operand rows (query q0 + r / 8, head r % 8): 64 bf16 = 8 chunks of 16 B,
  // chunk c of row r at position c ^ (r & 7) (conflict-free operand reads)
  __shared__ __attribute__((aligned(16))) uint4 qs[kPfQ * 8][8];
  __shared__ __attribute__((aligned(16))) float wsh[kPfQ][8];
  __shared__ int vsh[kPfQ];
  const int nq = min(kPfQ, a.tq - q0);
#pragma unroll
  for (int i = 0; i < kPfQ * 8 * 8 / (64 * kPfWaves); ++i) {
    const int idx = t + 64 * kPfWaves * i, r = idx / 8, c = idx % 8, q = r / 8, h = r % 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (q < nq)
      v = *(const uint4*)((const uint16_t*)a.q.data + (int64_t)b * a.q.sb + (int64_t)(q0 + q) * a.q.sr + h * 64 + 8 * c);
    qs[r][c ^ (r & 7)] = v;
  }
  for (int i = t; i < kPfQ * 8; i += 64 * kPfWaves) {
    const int q = i / 8, h = i % 8;
    wsh[q][h] = q < nq ? a.w[((int64_t)b * a.tq + q0 + q) * 8 + h] : 0.f;
  }
  if (t < kPfQ) vsh[t] = t < nq ? visible_blocks(a.q_pos[b * a.tq + q0 + t], a.m) : 0;
  __syncthreads();
  int vmax = 0;
  for (int q = 0; q < kPfQ; ++q) vmax = max(vmax, vsh[q]);
  const int kw = kbase + 16 * kPfNT * wave;  // this wave's first key
  float* srow_base = a.scores + ((int64_t)b * a.tq + q0) * a.n_cap;
  const bool rows16 = (a.n_cap & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;  // 16-byte aligned rows
  if (kw >= vmax) {  // no query of the tile sees these keys: -inf only
    for (int q = 0; q < nq; ++q)
      for (int i = l; i < 16 * kPfNT; i += kWave)
        if (kw + i < a.n_cap) srow_base[(int64_t)q * a.n_cap + kw + i] = kNegInf;
    return;
  }
  // B operand: key kw + 16nt + n, dims 32ks + 8g .. +7 (keys no query of the tile sees are zero)
  v8bf B[kPfNT][2];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const int key = kw + 16 * nt + n;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      B[nt][ks] = key < vmax ? *(const v8bf*)((const uint16_t*)a.k.data + (int64_t)b * a.k.sb + (int64_t)key * a.k.sr +
                                              32 * ks + 8 * g)
                             : (v8bf){};
  }
  // Query quads: two row tiles per quad, X = heads 0-3 and Y = heads 4-7 of its four
  // queries (row r: query 4it + r / 4, head r % 4, or 4 + r % 4), so that lane (key n,
  // g) holds all eight heads of query 4it + g for key kw + 16nt + n and sums them
  // without a lane exchange.  Heads 0-3 and 4-7 are summed in separate chains and then
  // added, as in index_bf16_kernel.
  for (int it = 0; it < kPfQ / 4; ++it) {
    if (4 * it >= nq) break;  // wave-uniform
    const int myq = 4 * it + g;
    const int Vq = vsh[myq];
    float* srow = srow_base + (int64_t)myq * a.n_cap;
    // X row 8(4it + n/4) + n%4 holds dims chunk 4ks + g at position 4ks + c0 (c0 = g ^ n%4);
    // the Y row, 4 further, at 4(1 - ks) + c0: one address plus constant offsets
    const uint4* ap = &qs[8 * (4 * it + n / 4) + n % 4][g ^ (n % 4)];
    v8bf AX[2], AY[2];
    AX[0] = __builtin_bit_cast(v8bf, ap[0]);
    AX[1] = __builtin_bit_cast(v8bf, ap[4]);
    AY[0] = __builtin_bit_cast(v8bf, ap[4 * 8 + 4]);
    AY[1] = __builtin_bit_cast(v8bf, ap[4 * 8]);
    const float4 w0 = *(const float4*)&wsh[myq][0], w1 = *(const float4*)&wsh[myq][4];
    const float wx[4] = {w0.x, w0.y, w0.z, w0.w}, wy[4] = {w1.x, w1.y, w1.z, w1.w};
    const int vrel = Vq - kw - n;  // (one register for the eight visibility tests)
    // a whole quad of 128 in-range keys in 16-byte aligned rows takes vector stores
    // with no per-lane test (wave-uniform)
    const bool whole = rows16 && 4 * it + 4 <= nq && kw + 16 * kPfNT <= a.n_cap;
    // tiles 4c .. 4c+3 at a time (four scores live per lane)
#pragma unroll
    for (int c = 0; c < kPfNT / 4; ++c) {
      float x[4];  // this lane's scores: query 4it + g, keys kw + 16(4c + i) + n
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nt = 4 * c + i;
        v4f cx = (v4f){0.f, 0.f, 0.f, 0.f}, cy = cx;
        cx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(AX[0], B[nt][0], cx, 0, 0, 0);
        cy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(AY[0], B[nt][0], cy, 0, 0, 0);
        cx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(AX[1], B[nt][1], cx, 0, 0, 0);
        cy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(AY[1], B[nt][1], cy, 0, 0, 0);
        float px = 0.f, py = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          px = fmaf(wx[r], relu_bits(cx[r]), px);
          py = fmaf(wy[r], relu_bits(cy[r]), py);
        }
        x[i] = 16 * nt < vrel ? px + py : kNegInf;  // key kw + 16nt + n < Vq
      }
      // scores are written once and read by another kernel: streamed past the caches
      if (whole) {
        // a 4x4 transpose across each lane quad gives lane n = 4j + i the four
        // consecutive keys 64c + 16i + 4j .. +3: one 16-byte store per lane writes 256
        // contiguous bytes of each query row
        quad_transpose4(x);
        __builtin_nontemporal_store((v4f){x[0], x[1], x[2], x[3]},
                                    (v4f*)&srow[kw + 64 * c + 16 * (n & 3) + 4 * (n >> 2)]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kw + 16 * (4 * c + i) + n;
          if (myq < nq && key < a.n_cap) __builtin_nontemporal_store(x[i], &srow[key]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ MXFP4 MFMA
// heads <= 32, dim == 64.  Each wave scores 8 tiles of 32 keys (256 keys, one
// scaled FP4 MFMA per tile; index_fp4.h), a workgroup 1024 keys: one candidate
// slice.  The query is quantised to MXFP4 once per workgroup into LDS while the
// keys are in flight.  Short waves, many per SIMD, keep the memory pipe full.

// ------------------------------------------------------------------ in-launch key compression
// The wave scoring keys g0 .. g0+255 of sequence b compresses every key of that
// range that this step completes (blocks klo .. khi-1 of indexer-key job fc.key, at
// most kFusedCompressMaxNew of them): lane l computes element l of the 64 (the
// compression's per-column arithmetic), the MXFP4 block scale and codes follow the
// compression store's arithmetic (32 consecutive lanes per block), and the wave
// stores the key to memory and, for its own scoring, to LDS (new key i: nkc[i] = 8
// dwords of codes, nks[i] = the two scale bytes), where the lanes holding that key's
// operand pick it up in place of what they loaded.  The first key's raw values are
// loaded early and combined after the wave's scoring pass, whose score for that key
// is then replaced: the key's tile is scored again with every other key's operand
// zero (one key's score depends on its own column only, so the bits are those a
// pass over the stored key gives).
__device__ __forceinline__ void compress_raw_load(const FusedCompress& fc, int b, int g,
                                                  float (&x)[kFusedCompressMaxM]) {
  const int64_t row0 = (int64_t)g * fc.key.m - fc.key.raw_base[b];
  const int l = threadIdx.x % kWave;
  if (fc.key_in == 0) compress_element_load<CSA_F32>(fc.key, b, row0, l, x);
  else if (fc.key_in == 1) compress_element_load<CSA_BF16>(fc.key, b, row0, l, x);
  else compress_element_load<CSA_FP8_E4M3>(fc.key, b, row0, l, x);
}

__device__ __forceinline__ void compress_own_keys(const FusedCompress& fc, int b, int klo, int khi,
                                                  const float (&x0)[kFusedCompressMaxM], uint32_t (*nkc)[8],
                                                  uint32_t (*nks)[2]) {
  const CompressArgs& k = fc.key;
  const int l = threadIdx.x % kWave;
  float wz[kFusedCompressMaxM];
#pragma unroll
  for (int r = 0; r < kFusedCompressMaxM; ++r)
    if (r < k.m) wz[r] = k.logits[r];
  local_softmax(k.m, wz);
  for (int g = klo; g < khi; ++g) {
    float x[kFusedCompressMaxM];
    if (g == klo) {
#pragma unroll
      for (int r = 0; r < kFusedCompressMaxM; ++r) x[r] = x0[r];
    } else {
      compress_raw_load(fc, b, g, x);
    }
    const float v = compress_element_combine(k.m, x, wz);
    float am = fabsf(v);
    for (int o = 16; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 32));
    const int e = mx_scale_exp(am);
    const uint32_t nib = am > 0.f ? f32_to_e2m1(v, e) : 0u;
    // dword q of the 32 code bytes holds elements 8q .. 8q+7, element 8q+d in nibble d
    uint32_t word = nib;
#pragma unroll
    for (int d = 1; d < 8; ++d) word |= (uint32_t)__shfl_down((int)nib, d, 8) << (4 * d);
    uint8_t* codes = (uint8_t*)k.out + (int64_t)b * k.out_sb + (int64_t)g * k.out_sr;
    if (l % 8 == 0) {
      *(uint32_t*)(codes + 4 * (l / 8)) = word;
      nkc[g - klo][l / 8] = word;
    }
    if (l % 32 == 0) {
      ((uint8_t*)k.out_scale)[(int64_t)b * k.out_ssb + (int64_t)g * k.out_ssr + l / 32] = (uint8_t)(e + 127);
      nks[g - klo][l / 32] = (uint32_t)(e + 127);
    }
  }
}

// With CAND set, each workgroup also writes its 1024-key slice's candidate list
// (emit_slice_list: every key at or above a cheap cut, else the exact top-32) with
// the slice's metadata.  The keys go through LDS once; three waves then exit (freeing
// their registers for the next workgroups' key loads) and one wave builds the list.
// Scores are written where a.scores points; without it, only short rows' scores go to
// co.row_scores (their selection reads them).
template <int NR, bool CAND>  // NR: accumulator rows that can hold a real head: 4 (heads <= 8) or 16 (heads <= 32)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NR == 4 ? 6 : 4))) void index_mxfp4_kernel(
    IndexArgs a, CandOut co, FusedCompress fc) {
  // Workgroup order (a 1-D grid): the KV compressions first (they run alongside the
  // scoring instead of after it), then row by row, each row's slices from the last one
  // down, so the slice holding a row's newest keys (which it compresses before
  // scoring) starts first.  Consecutive workgroups stream consecutive key ranges.
  const int rows = fc.rows, nextra = fc.kv.batch > 0 ? fc.kv.max_blocks : 0;
  const int id = blockIdx.x;
  if (id < rows * nextra) {  // a KV compression workgroup (decode: row == sequence)
    __shared__ float cred[kCompressThreads / kWave];
    const int b = id % rows, i = id / rows;
    if (b >= fc.kv.batch) return;
    if (fc.kv_in == 0) compress_block<2, CSA_F32, true>(fc.kv, b, i, nullptr, cred);
    else if (fc.kv_in == 1) compress_block<2, CSA_BF16, true>(fc.kv, b, i, nullptr, cred);
    else compress_block<2, CSA_FP8_E4M3, true>(fc.kv, b, i, nullptr, cred);
    return;
  }
  const int sid = id - rows * nextra;
  const int row = sid / fc.nslices;
  const int b = row / a.tq, t = row % a.tq;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = threadIdx.x % kWave;
  const int slice = fc.nslices - 1 - sid % fc.nslices;
  const int g0 = slice * kFp4KeysPerWG + wave * kFp4KeysPerWave;
  const Fp4Lane<NR> ln(l);

  // the row's position, its query and head weights, and (in-launch key compression)
  // the blocks this step completes, then the keys
  const int qp = a.q_pos[row];
  const bool kjob = fc.key.batch > 0;
  const int jf = kjob ? fc.key.block_first[b] : 0, jcnt = kjob ? fc.key.block_count[b] : 0;
  float2 qx[Fp4Pairs<NR>::n];
  fp4_query_load(a, b, t, threadIdx.x, qx);
  __shared__ Fp4QueryLds ql;
  if (threadIdx.x < a.heads) ql.w[threadIdx.x] = a.w[(int64_t)row * a.heads + threadIdx.x];
  const int V = visible_blocks(qp, a.m);
  // the key codes (16 B per lane: key m's block kb) and their e8m0 scales of visible
  // keys, read once (issued as soon as the position is known; earlier, they would
  // hold back the query and position loads queued behind them)
  const int kfirst = g0 + ln.m;
  const uint8_t* kc = (const uint8_t*)a.k.data + (int64_t)b * a.k.sb + 16 * ln.kb;
  const uint8_t* ks = (const uint8_t*)a.k.scale + (int64_t)b * a.k.ssb + ln.kb;
  v4i c[kFp4Unroll];
  int sbk[kFp4Unroll];
#pragma unroll
  for (int u = 0; u < kFp4Unroll; ++u) {
    const bool live = kfirst + 32 * u < V;
    const int64_t key = min(kfirst + 32 * u, a.n_cap - 1);
    c[u] = live ? __builtin_nontemporal_load((const v4i*)(kc + key * a.k.sr)) : (v4i){0, 0, 0, 0};
    sbk[u] = live ? __builtin_nontemporal_load(ks + key * a.k.ssr) : 127;
  }
  // keys of blocks this step completes (the loads above may have read stale codes for
  // them): the wave compresses and stores them after its scoring pass, then rescores
  const int klo = max(jf, g0), khi = min(jf + min(jcnt, fc.key.max_blocks), g0 + kFp4KeysPerWave);
  const bool own_new = kjob && klo < khi;  // wave-uniform
  fp4_query_quantize(a, threadIdx.x, qx, ql);
  __syncthreads();
  if (!CAND && g0 >= a.n_cap) return;

  v8i A;
  int sa;
  float wv[NR];
  fp4_query_operand<NR>(ql, a.heads, l, &A, &sa, wv);
  // operands of keys completed by this step (not yet stored when loaded) are zeroed
  // before any MFMA sees them: stale bytes may hold a NaN scale, which would spoil the
  // tile's other columns
  if (own_new) {  // wave-uniform (rare: the wave holding the step's newest keys)
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int g = kfirst + 32 * u;
      const bool drop = g >= klo && g < khi;
      c[u] = drop ? (v4i){0, 0, 0, 0} : c[u];
      sbk[u] = drop ? 127 : sbk[u];
    }
  }
  // 3) scores
  float sc[kFp4Unroll];  // the wave's scores: tile u, key g0 + 32u + m (in lanes l and l ^ kPair)
#pragma unroll
  for (int u = 0; u < kFp4Unroll; ++u) {
    sc[u] = fp4_tile_score<NR>(A, sa, wv, c[u], sbk[u]);
    // keep one accumulator tile live at a time: occupancy (many waves hiding each
    // other's memory latency) matters more here than MFMA back-to-back issue
    __builtin_amdgcn_sched_barrier(0);
  }
  if (own_new) {  // the step's new keys: compress, store, rescore their tiles
    __shared__ uint32_t nkc[4][kFusedCompressMaxNew][8], nks[4][kFusedCompressMaxNew][2];
    float xr[kFusedCompressMaxM];
    compress_raw_load(fc, b, klo, xr);
    compress_own_keys(fc, b, klo, khi, xr, nkc[wave], nks[wave]);
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int g = kfirst + 32 * u;
      const bool mine = g >= klo && g < khi;
      if (__builtin_amdgcn_ballot_w64(mine) == 0) continue;  // wave-uniform
      v4i cn = {0, 0, 0, 0};
      int sn = 127;
      if (mine) {
        const uint32_t* wc = nkc[wave][g - klo] + 4 * ln.kb;
        cn = (v4i){(int)wc[0], (int)wc[1], (int)wc[2], (int)wc[3]};
        sn = (int)nks[wave][g - klo][ln.kb];
      }
      const float s_new = fp4_tile_score<NR>(A, sa, wv, cn, sn);
      sc[u] = mine ? s_new : sc[u];
    }
  }
  const int Vc = min(V, a.n_cap);
  float* srow = a.scores ? a.scores + (int64_t)row * a.n_cap
                         : (CAND && Vc > co.k && index_topk_short_row(Vc, co.k) ? co.row_scores + (int64_t)row * a.n_cap
                                                                                : nullptr);
  if (srow) {  // kb == 0 lanes store tile u, kb == 1 lanes tile u + 4: one store for two tiles
    const int gend = min(g0 + kFp4KeysPerWave, a.n_cap);
#pragma unroll
    for (int u = 0; u < kFp4Unroll / 2; ++u) {
      const int us = ln.kb ? u + kFp4Unroll / 2 : u;
      const int key = g0 + 32 * us + ln.m;
      const float v = ln.kb ? sc[u + kFp4Unroll / 2] : sc[u];
      if (key < gend) __builtin_nontemporal_store(key < V ? v : kNegInf, &srow[key]);  // streamed
    }
  }
  if constexpr (CAND) {
    if (Vc <= co.k || index_topk_short_row(Vc, co.k)) return;  // selected from the scores, not from lists
    __shared__ __attribute__((aligned(16))) uint32_t skeys[kFusedSlice];
    __shared__ CutLds cl;
    const int start = slice * kFusedSlice;
    const int n = max(0, min(kFusedSlice, Vc - start));  // visible keys of this slice
    if (ln.kb == 0) {  // these lanes hold every key of the wave's tiles once
#pragma unroll
      for (int u = 0; u < kFp4Unroll; ++u) skeys[wave * kFp4KeysPerWave + 32 * u + ln.m] = float_key(sc[u]);
    }
    __syncthreads();
    // one wave builds the list, the others free their registers now; the builder's index
    // rotates with the workgroup so the builders of a CU's workgroups use all four SIMDs
    if (wave != (int)(blockIdx.x % 4)) return;
    uint32_t kv[kWaveTopN];
#pragma unroll
    for (int q = 0; q < kWaveTopN / 4; ++q) {
      const uint4 v4 = *(const uint4*)&skeys[kWaveTopN * l + 4 * q];
      kv[4 * q] = v4.x;
      kv[4 * q + 1] = v4.y;
      kv[4 * q + 2] = v4.z;
      kv[4 * q + 3] = v4.w;
    }
    if (n < kFusedSlice) {  // positions past the visible ones are absent (wave-uniform test)
#pragma unroll
      for (int j = 0; j < kWaveTopN; ++j)
        if (kWaveTopN * l + j >= n) kv[j] = 0u;
    }
    emit_slice_list(kv, n, (uint32_t)start, cl, co.cand + ((int64_t)row * co.nslices + slice) * kFusedC,
                    co.meta + (int64_t)row * co.nslices + slice);
  }
}

// No in-launch compression: every workgroup scores.
FusedCompress no_compress(int nslices, int rows) {
  FusedCompress f{};
  f.key.batch = 0;
  f.kv.batch = 0;
  f.nslices = nslices;
  f.rows = rows;
  return f;
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s) {
  const int rows = a.batch * a.tq;
  if (rows == 0 || a.n_cap == 0) return hipSuccess;
  if (a.k.dtype == CSA_MXFP4) {
    const int nslices = (a.n_cap + kFp4KeysPerWG - 1) / kFp4KeysPerWG;
    const dim3 grid((unsigned)(nslices * rows));
    const CandOut none{};
    if (a.heads <= 8)
      hipLaunchKernelGGL((index_mxfp4_kernel<4, false>), grid, dim3(256), 0, s, a, none, no_compress(nslices, rows));
    else
      hipLaunchKernelGGL((index_mxfp4_kernel<16, false>), grid, dim3(256), 0, s, a, none, no_compress(nslices, rows));
  } else if (a.k.dtype == CSA_BF16 && a.q.dtype == CSA_BF16 && a.heads == 8 && a.dim == 64 && a.tq >= kPfMinTq) {
    // many queries per sequence: the 32-query tile kernel (same arithmetic, same order)
    dim3 grid((a.n_cap + kPfKeys - 1) / kPfKeys, (a.tq + kPfQ - 1) / kPfQ, a.batch);
    hipLaunchKernelGGL(index_bf16_tile_kernel, grid, dim3(64 * kPfWaves), 0, s, a);
  } else if (a.k.dtype == CSA_BF16 && a.q.dtype == CSA_BF16 && a.heads == 8 && a.dim == 64) {
    dim3 grid((a.n_cap + kBfKT - 1) / kBfKT, (a.tq + kBfQT - 1) / kBfQT, a.batch);
    hipLaunchKernelGGL(index_bf16_kernel, grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((a.n_cap + kPlainThreads - 1) / kPlainThreads, rows);
    const size_t lds = (size_t)a.heads * a.dim * sizeof(float);
    hipLaunchKernelGGL(index_plain_kernel, grid, dim3(kPlainThreads), lds, s, a);
  }
  return hipGetLastError();
}

static_assert(kFp4KeysPerWG == kFusedSlice, "one indexer workgroup per candidate slice");

hipError_t launch_index_scores_cand(const IndexArgs& a, const CandOut& c, hipStream_t s, const FusedCompress* fc) {
  const int rows = a.batch * a.tq;
  if (rows == 0 || a.n_cap == 0) return hipSuccess;
  const int nslices = (a.n_cap + kFp4KeysPerWG - 1) / kFp4KeysPerWG;
  FusedCompress f = fc ? *fc : no_compress(nslices, rows);
  f.nslices = nslices;
  f.rows = rows;
  const int extra = f.kv.batch > 0 ? f.kv.max_blocks : 0;  // KV compression workgroups per row
  const dim3 grid((unsigned)((nslices + extra) * rows));
  if (a.heads <= 8)
    hipLaunchKernelGGL((index_mxfp4_kernel<4, true>), grid, dim3(256), 0, s, a, c, f);
  else
    hipLaunchKernelGGL((index_mxfp4_kernel<16, true>), grid, dim3(256), 0, s, a, c, f);
  return hipGetLastError();
}

}  // namespace csa


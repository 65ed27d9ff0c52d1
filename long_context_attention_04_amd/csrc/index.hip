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
//    columns; used by decode and by prefill chunks (where it is a dense
//    contraction of many queries against the same keys).
//  * F32 keys: plain fp32 VALU kernel (small shapes).
#include "common.h"
#include "compress_block.h"
#include "kernels.h"
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

// ------------------------------------------------------------------ MXFP4 MFMA
// heads <= 32, dim == 64.  Each wave scores one group of kFp4Unroll*32 keys:
// it issues every key load of its group, the workgroup quantises the query
// once (cooperatively, into LDS) while they are in flight, then each wave runs
// one MFMA per 32 keys.  Short waves, many per SIMD,
// keep the memory pipe full (a wave's own load latency overlaps the others').
constexpr int kFp4Unroll = 8;
constexpr int kFp4KeysPerWave = 32 * kFp4Unroll;
constexpr int kFp4KeysPerWG = 4 * kFp4KeysPerWave;

// The query of row (b, t), quantised to MXFP4 by a 256-thread workgroup into LDS:
// thread -> (head, K block, element pair); the 16 threads of a 32-element block are
// 16 adjacent lanes.  qcode[h][blk] = 16 B of e2m1 codes, qscale[h][blk] = e8m0.
// Loaded first (query_pairs), quantised later (quantize_query_mxfp4), so the load
// is not queued behind the key loads issued in between.
constexpr int kQueryPairsMax = 4;  // heads * 32 pairs over 256 threads (heads <= 32)
__device__ __forceinline__ void query_pairs(const IndexArgs& a, int b, int t, float2 (&x)[kQueryPairsMax]) {
#pragma unroll
  for (int i = 0; i < kQueryPairsMax; ++i) {
    const int pi = 256 * i + (int)threadIdx.x;
    const int h = pi / 32, blk = (pi / 16) % 2, pr = pi % 16;
    x[i] = h < a.heads ? *(const float2*)((const float*)a.q.data + (int64_t)b * a.q.sb + (int64_t)t * a.q.sr + h * 64 +
                                          32 * blk + 2 * pr)
                       : make_float2(0.f, 0.f);
  }
}
__device__ __forceinline__ void quantize_query_mxfp4(const IndexArgs& a, const float2 (&xs)[kQueryPairsMax],
                                                     uint32_t (*qcode)[2][4], uint32_t (*qscale)[2]) {
#pragma unroll
  for (int i = 0; i < kQueryPairsMax; ++i) {
    if (256 * i >= a.heads * 32) break;  // uniform
    const int pi = 256 * i + (int)threadIdx.x;
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
      if ((pr & 3) == 0) qcode[h][blk][pr / 4] = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
      if (pr == 0) qscale[h][blk] = (uint32_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------ in-launch key compression
// The wave scoring keys g0 .. g0+255 of sequence b compresses every key of that
// range that this step completes (blocks klo .. khi-1 of indexer-key job fc.key, at
// most kFusedCompressMaxNew of them): lane l computes element l of the 64 (the
// compression's per-column arithmetic), the MXFP4 block scale and codes follow the
// compression store's arithmetic (32 consecutive lanes per block), and the wave
// stores the key to memory and, for its own scoring, to LDS (new key i: nkc[i] = 8
// dwords of codes, nks[i] = the two scale bytes), where the lanes holding that key's
// operand pick it up in place of what they loaded.  The first key's raw values are
// loaded before the wave's key loads (compress_raw_load) and combined after them.
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

// ------------------------------------------------------------------ slice top-32
// With CAND set, each workgroup also selects the exact top-32 of its 1024-key
// slice in (key desc, index asc) order -- key being the order-preserving integer
// form of the score, the order the top-k uses -- and writes them in ascending
// index order with the slice's metadata (count, truncated?, 32nd element).  The
// keys go through LDS once; three waves then exit (freeing their registers for
// the next workgroups' key loads) and one wave runs a barrier-free radix select.
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
  // the position and (in-launch key compression) the step's new blocks: one round trip
  const int qp = a.q_pos[row];
  const bool kjob = fc.key.batch > 0;
  const int jf = kjob ? fc.key.block_first[b] : 0, jcnt = kjob ? fc.key.block_count[b] : 0;
  const int V = visible_blocks(qp, a.m);
  const int slice = fc.nslices - 1 - sid % fc.nslices;
  const int g0 = slice * kFp4KeysPerWG + wave * kFp4KeysPerWave;
  // The key (within a 32-key tile) and K block this lane loads.  Up to 8 heads use a
  // block-diagonal 16x16x128 MFMA: query heads fill rows 0-7 over K 0-63 and rows
  // 8-15 over K 64-127, keys 0-15 of the tile fill K 0-63 and keys 16-31 K 64-127, so
  // one MFMA scores 32 keys with a 4-register accumulator; up to 32 heads use the
  // 32x32x64 MFMA (rows = heads, columns = keys).
  constexpr bool kDiag = NR == 4;
  const int m = kDiag ? 16 * (l / 32) + l % 16 : l % 32;
  const int kb = kDiag ? (l / 16) % 2 : l / 32;
  __shared__ __attribute__((aligned(16))) uint32_t qcode[32][2][4];  // [head][K block][16 B of e2m1 codes]
  __shared__ uint32_t qscale[32][2];
  __shared__ float wsh[32];

  // 1) the query (loaded first: it must not queue behind the keys), then the key codes
  //    (16 B per lane: key m's block kb) and their e8m0 scales, whose latency
  //    overlaps the query quantisation below
  float2 qx[kQueryPairsMax];
  query_pairs(a, b, t, qx);
  // keys of blocks this step completes (the loads below may read stale codes for them):
  // the wave compresses them first, stores them, and takes them from LDS before scoring
  const int klo = max(jf, g0), khi = min(jf + min(jcnt, fc.key.max_blocks), g0 + kFp4KeysPerWave);
  const bool own_new = kjob && klo < khi;  // wave-uniform
  __shared__ uint32_t nkc[4][kFusedCompressMaxNew][8], nks[4][kFusedCompressMaxNew][2];
  if (own_new) {
    float xr[kFusedCompressMaxM];
    compress_raw_load(fc, b, klo, xr);
    compress_own_keys(fc, b, klo, khi, xr, nkc[wave], nks[wave]);
  }
  const int kfirst = g0 + m;
  const uint8_t* kc = (const uint8_t*)a.k.data + (int64_t)b * a.k.sb + (int64_t)kfirst * a.k.sr + 16 * kb;
  const uint8_t* ks = (const uint8_t*)a.k.scale + (int64_t)b * a.k.ssb + (int64_t)kfirst * a.k.ssr + kb;
  const int64_t cstep = 32 * a.k.sr, sstep = 32 * a.k.ssr;
  v4i c[kFp4Unroll];
  int sbk[kFp4Unroll];
#pragma unroll
  for (int u = 0; u < kFp4Unroll; ++u) {
    const bool live = kfirst + 32 * u < V;
    c[u] = live ? __builtin_nontemporal_load((const v4i*)(kc + u * cstep)) : (v4i){0, 0, 0, 0};  // read once
    sbk[u] = live ? __builtin_nontemporal_load(ks + u * sstep) : 127;
  }
  // head weights, after the key loads (their wait must not hold the keys back)
  if (threadIdx.x < a.heads) wsh[threadIdx.x] = a.w[(int64_t)row * a.heads + threadIdx.x];
  // 2) the query, quantised to MXFP4 once per workgroup
  quantize_query_mxfp4(a, qx, qcode, qscale);

  __syncthreads();
  if (!CAND && g0 >= a.n_cap) return;
  // A operand: row l%16 (diagonal) or l%32, K block l/16 or l/32 (32 e2m1 codes each)
  const int qrow = kDiag ? l % 16 : l % 32, qblk = kDiag ? l / 16 : l / 32;
  const bool qlive = kDiag ? (qrow < 8) == (qblk < 2) : true;  // off-diagonal blocks are zero
  const int qh = kDiag ? qrow % 8 : qrow;
  v8i A = {0, 0, 0, 0, 0, 0, 0, 0};
  int sa = 127;
  if (qlive && qh < a.heads) {
    const uint4 qv = *(const uint4*)&qcode[qh][qblk % 2][0];
    A[0] = (int)qv.x; A[1] = (int)qv.y; A[2] = (int)qv.z; A[3] = (int)qv.w;
    sa = (int)qscale[qh][qblk % 2];
  }
  if (own_new) {  // the new keys' operands, from LDS (after the barrier above)
#pragma unroll
    for (int u = 0; u < kFp4Unroll; ++u) {
      const int g = kfirst + 32 * u;
      if (g >= klo && g < khi && g < V) {
        const uint32_t* wc = nkc[wave][g - klo] + 4 * kb;
        c[u] = (v4i){(int)wc[0], (int)wc[1], (int)wc[2], (int)wc[3]};
        sbk[u] = (int)nks[wave][g - klo][kb];
      }
    }
  }
  // head weights of this lane's accumulator rows h = 8*(r/4) + 4*kb + r%4 (both layouts:
  // a diagonal lane's rows 4*(l/16) + r hold heads 4*((l/16)%2) + r)
  float wv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int h = 8 * (r / 4) + 4 * kb + (r % 4);
    wv[r] = h < a.heads ? wsh[h] : 0.f;
  }
  // 3) scores
  float* srow = a.scores + (int64_t)row * a.n_cap;
  const int gend = min(g0 + kFp4KeysPerWave, a.n_cap);
  float sc[kFp4Unroll];  // the wave's scores: tile u, key g0 + 32u + m (in lanes l and l ^ kPair)
  constexpr int kPair = kDiag ? 16 : 32;  // the lane holding the same key's other heads
#pragma unroll
  for (int u = 0; u < kFp4Unroll; ++u) {
    v8i Bop = {c[u][0], c[u][1], c[u][2], c[u][3], 0, 0, 0, 0};
    float part = 0.f;
    if constexpr (kDiag) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bop, acc, 4, 4, 0, sa, 0, sbk[u]);
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(wv[r], fmaxf(acc[r], 0.f), part);
    } else {
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bop, acc, 4, 4, 0, sa, 0, sbk[u]);
#pragma unroll
      for (int r = 0; r < NR; ++r) part = fmaf(wv[r], fmaxf(acc[r], 0.f), part);
    }
    const float other = __shfl_xor(part, kPair);
    sc[u] = part + other;  // the same value in lane l and lane l ^ kPair
    if (u >= kFp4Unroll / 2) {  // kb == 0 lanes store tile u - 4, kb == 1 lanes tile u: one store for two tiles
      const int us = kb ? u : u - kFp4Unroll / 2;
      const int key = g0 + 32 * us + m;
      const float v = kb ? sc[u] : sc[u - kFp4Unroll / 2];
      if (key < gend) __builtin_nontemporal_store(key < V ? v : kNegInf, &srow[key]);  // streamed
    }
    // keep one accumulator tile live at a time: occupancy (many waves hiding each
    // other's memory latency) matters more here than MFMA back-to-back issue
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (CAND) {
    const int Vc = min(V, a.n_cap);
    if (Vc <= co.k) return;  // every visible key is selected: the merge needs no candidates
    __shared__ __attribute__((aligned(16))) uint32_t skeys[kFusedSlice];
    __shared__ WaveSelLds sl;
    const int start = slice * kFusedSlice;
    const int n = max(0, min(kFusedSlice, Vc - start));  // visible keys of this slice
    if (kb == 0) {  // these lanes hold every key of the wave's tiles once
#pragma unroll
      for (int u = 0; u < kFp4Unroll; ++u) skeys[wave * kFp4KeysPerWave + 32 * u + m] = float_key(sc[u]);
    }
    __syncthreads();
    if (wave != 0) return;  // one wave selects; the others free their registers now
    SliceMeta* mt = co.meta + (int64_t)row * co.nslices + slice;
    uint2* out = co.cand + ((int64_t)row * co.nslices + slice) * kWaveTopC;
    uint32_t kv[kWaveTopN];
#pragma unroll
    for (int q = 0; q < kWaveTopN / 4; ++q) {
      const uint4 v4 = *(const uint4*)&skeys[kWaveTopN * l + 4 * q];
      kv[4 * q] = v4.x;
      kv[4 * q + 1] = v4.y;
      kv[4 * q + 2] = v4.z;
      kv[4 * q + 3] = v4.w;
    }
#pragma unroll
    for (int j = 0; j < kWaveTopN; ++j)
      if (kWaveTopN * l + j >= n) kv[j] = 0u;  // positions past the visible ones are absent
    if (n <= kWaveTopC) {  // every slot of the slice's list: its n keys, then empty (key 0) slots
#pragma unroll
      for (int j = 0; j < kWaveTopN; ++j) {
        const int p = kWaveTopN * l + j;
        if (p < kWaveTopC) out[p] = p < n ? make_uint2(kv[j], (uint32_t)(start + p)) : make_uint2(0u, 0u);
      }
      if (l == 0) *mt = SliceMeta{(uint32_t)n, 0u, 0u, 0u};
      return;
    }
    uint32_t T, tpos;
    wave_top32(kv, sl, &T, &tpos);
    if (l < kWaveTopC) {  // one coalesced store of the list
      const uint2 e = sl.res[l];
      out[l] = make_uint2(e.x, (uint32_t)start + e.y);
    }
    if (l == 0) *mt = SliceMeta{(uint32_t)kWaveTopC, 1u, T, (uint32_t)start + tpos};
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

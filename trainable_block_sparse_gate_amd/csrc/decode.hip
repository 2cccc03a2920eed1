// Decode path for gfx950 (review, section 3-7: score cached block
// summaries, keep the Top-K per query group, read the kept blocks of the
// paged KV cache, run the block-sparse decode kernel; GQA groups share one
// selection).
//
//   pool:    summary of block j = mean of its 64 keys, summed in token order
//            in fp32 (one thread per (block, channel), reads and writes
//            coalesced along the channel).
//   scores:  s_j = (fmaf chain over channels of qbar * summary) / sqrt(d),
//            qbar = sum of the group's query heads in head order / G, all
//            in fp32 in exactly this order, so the Top-K decision is taken
//            on values the oracle reproduces bit for bit.  Summaries are
//            tiled (summary_index), so a thread reads its block's channels
//            as a few 16-byte pieces, all in flight at once, while each
//            wave-wide read is 1 KB of contiguous memory.
//   attend:  split-K over the kept blocks of every (sequence, kv head):
//            each wave of a workgroup streams its own share of 64-token
//            K/V blocks (16-byte coalesced loads, several passes in flight
//            in registers), keeps an fp32 online softmax per query head
//            with the block's log gate added; the waves merge into an
//            unnormalised partial per split, and a second kernel merges
//            the partials with a log-sum-exp combine in a fixed order.
// Pages cited by title: "review" is the page "SAS: Simple Attention
// Sparsification via End-to-End Optimization of Context Ranking Review";
// "paper text" is the page "SAS: Simple Attention Sparsification via
// End-to-End Optimization of Context Ranking" that holds the paper's text.
#include <mutex>
#include <type_traits>

#include "sas_device.h"
#include "sas_launch.h"
#include "select.h"
#include "tile_stage.h"

namespace sas {

__device__ inline const __bf16 *kv_row(const DecodeParams &p, const __bf16 *cache, int b, int g,
                                       int tok) {
  if (p.paged) {
    const int page = p.page_table[(long)b * p.max_pages + tok / kBlock];
    return cache + (((long)page * p.hkv + g) * kBlock + (tok % kBlock)) * p.D;
  }
  return cache + (((long)b * p.hkv + g) * p.max_seqlen + tok) * p.D;
}

// The fp8 e4m3 code of the nearest e4m3 value to x (1 sign bit, 4 exponent
// bits with bias 7, 3 mantissa bits, no infinities, 0x7f = NaN): below 2^-6
// the format's spacing is 2^-9, in [2^e, 2^(e+1)) it is 2^(e-3); x over its
// spacing is rounded to the nearest integer, ties to even (exact in fp32);
// 480 and beyond, infinities and NaN give NaN.
__device__ inline uint8_t e4m3_code(float x) {
  const uint8_t sgn = (__float_as_uint(x) >> 31) ? 0x80 : 0;
  const float a = fabsf(x);
  if (!(a < 480.f)) return sgn | 0x7f;  // NaN, infinities, >= 480
  const int e = a >= 0x1p-6f ? (int)((__float_as_uint(a) >> 23) & 255u) - 127 : -7;
  const float spacing = e >= -6 ? __uint_as_float((uint32_t)(e - 3 + 127) << 23) : 0x1p-9f;
  const float n = rintf(a / spacing);  // ties to even
  const float r = n * spacing;
  if (r >= 480.f) return sgn | 0x7f;
  if (r < 0x1p-6f) return sgn | (uint8_t)(int)n;  // subnormal (or zero): mantissa n
  const int er = (int)((__float_as_uint(r) >> 23) & 255u) - 127;
  const uint32_t mant = (__float_as_uint(r) >> 20) & 7u;
  return sgn | (uint8_t)((er + 7) << 3) | (uint8_t)mant;
}

// Element index of channel e of block j's summary in row `row`.  Summaries
// are stored in tiles of 64 consecutive blocks; inside a tile, 16-byte piece
// l (channels [l EPP, (l + 1) EPP), EPP = 16 / element size) of the 64 blocks
// lies side by side in block order:
//   [row][j / 64][e / EPP][j % 64][e % EPP]
// so one wave reading piece l of 64 consecutive blocks (a block per lane)
// reads 1 KB of contiguous memory.
__device__ inline long summary_index(const DecodeParams &p, int stride, int row, int j, int e) {
  const int epp = p.sum_kind == kSumBf16 ? 8 : p.sum_kind == kSumFp8 ? 16 : 4;
  const int np = p.D / epp;
  return (((long)row * (stride / 64) + j / 64) * np + e / epp) * (64 * epp) +
         (j % 64) * epp + e % epp;
}
__device__ inline long summary_index(const DecodeParams &p, int row, int j, int e) {
  return summary_index(p, p.nblk_stride, row, j, e);
}

// A block summary (the fp32 mean) stored as fp32, or rounded to the nearest
// bf16 / fp8 e4m3 value (ties to even), into `dst` (block or super-block
// summaries).
__device__ inline void store_summary(const DecodeParams &p, void *dst, long idx, float v) {
  if (p.sum_kind == kSumBf16)
    static_cast<__bf16 *>(dst)[idx] = (__bf16)v;
  else if (p.sum_kind == kSumFp8)
    static_cast<uint8_t *>(dst)[idx] = e4m3_code(v);
  else
    static_cast<float *>(dst)[idx] = v;
}
__device__ inline void store_summary(const DecodeParams &p, long idx, float v) {
  store_summary(p, p.ksum, idx, v);
}

__device__ inline float e4m3_value(uint32_t b);

// The stored block summary at idx as fp32 (exact).
__device__ inline float load_summary(const DecodeParams &p, long idx) {
  if (p.sum_kind == kSumBf16) return (float)static_cast<const __bf16 *>(p.ksum)[idx];
  if (p.sum_kind == kSumFp8) return e4m3_value(static_cast<const uint8_t *>(p.ksum)[idx]);
  return static_cast<const float *>(p.ksum)[idx];
}

// Summary of super-block J (hierarchical selection; review 7-2: a coarse
// retrieval narrows the candidates): the mean of its kCoarseBlocks stored
// block summaries, summed in block order in fp32, stored like them.
__device__ inline void store_coarse(const DecodeParams &p, int row, int J, int e) {
  float acc = 0.f;
  for (int b = 0; b < kCoarseBlocks; ++b)
    acc = acc + load_summary(p, summary_index(p, row, kCoarseBlocks * J + b, e));
  store_summary(p, p.csum, summary_index(p, p.cstride, row, J, e), acc / (float)kCoarseBlocks);
}

// Super-block summaries of every complete super-block (kCoarseBlocks J +
// kCoarseBlocks - 1 < the history count): one thread per (super-block,
// channel).
__global__ __launch_bounds__(128) void pool_coarse_kernel(DecodeParams p) {
#pragma clang fp contract(off)
  const int J = blockIdx.x, row = blockIdx.y;
  const int e = threadIdx.x;
  const int nsup = ((p.seqlens[row / p.hkv] - 1) / kBlock) / kCoarseBlocks;
  if (J >= nsup || e >= p.D) return;
  store_coarse(p, row, J, e);
}

// ------------------------------------------------------------------ pool
__global__ __launch_bounds__(128) void pool_keys_kernel(DecodeParams p) {
#pragma clang fp contract(off)
  const int j = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int e = threadIdx.x;
  const int nhist = (p.seqlens[b] - 1) / kBlock;
  if (j >= nhist || e >= p.D) return;
  const __bf16 *k = static_cast<const __bf16 *>(p.k);
  const __bf16 *row = kv_row(p, k, b, g, j * kBlock);  // a block never crosses a page
  float acc = 0.f;
  for (int t = 0; t < kBlock; ++t) acc = acc + (float)row[(long)t * p.D + e];
  store_summary(p, summary_index(p, bg, j, e), acc / (float)kBlock);
}

// ------------------------------------------------------------------ append
// One decode step's cache maintenance (review section 3-7: summaries are
// kept per block as the cache grows).  The new token's key and value go to
// position L - 1 of its (sequence, kv head) row; when that token opens a new
// block, the block before it has just become history and gets its summary,
// summed exactly as pool_keys_kernel sums it.  One thread per channel.
__global__ __launch_bounds__(128) void append_kernel(DecodeParams p, const __bf16 *k_new,
                                                     const __bf16 *v_new, __bf16 *kc,
                                                     __bf16 *vc) {
#pragma clang fp contract(off)
  const int bg = blockIdx.x;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int e = threadIdx.x;
  if (e >= p.D) return;
  const int tok = p.seqlens[b] - 1;
  const long src = ((long)b * p.hkv + g) * p.D + e;
  const long dst = (kv_row(p, kc, b, g, tok) - kc) + e;
  kc[dst] = k_new[src];
  vc[dst] = v_new[src];
  if (tok > 0 && tok % kBlock == 0) {
    const int j = tok / kBlock - 1;
    const __bf16 *row = kv_row(p, kc, b, g, j * kBlock);
    float acc = 0.f;
    for (int t = 0; t < kBlock; ++t) acc = acc + (float)row[(long)t * p.D + e];
    store_summary(p, summary_index(p, bg, j, e), acc / (float)kBlock);
    // block j completes super-block j / kCoarseBlocks (this thread wrote
    // the channel's last summary itself, so it reads it back)
    if (p.csum && (j + 1) % kCoarseBlocks == 0) store_coarse(p, bg, j / kCoarseBlocks, e);
  }
}

// ------------------------------------------------------------------ select
// The fp32 value of an fp8 e4m3 code (exact): (1 + m / 8) 2^(e - 7) for
// exponent field e > 0, m 2^-9 for e = 0; 0x7f / 0xff are NaN.  The code's
// exponent and mantissa fields placed at the top of an fp32 pattern are the
// fp32 number 2^-120 times the value (a normal fp32 for e > 0, a subnormal
// m 2^-129 for e = 0), so one exact multiplication by 2^120 decodes both.
// The NaN codes are substituted by integer arithmetic, with no comparison
// (a comparison per value leaves a lane mask per value in scalar registers
// when many are decoded at once): nan = 1 exactly when the low seven bits
// are all ones.
__device__ inline float e4m3_value(uint32_t b) {
  const uint32_t v = __float_as_uint(
      __uint_as_float(((b & 0x80u) << 24) | ((b & 0x7fu) << 20)) * 0x1p120f);
  const uint32_t nan = ((b & 0x7fu) + 1u) >> 7;
  return __uint_as_float(v ^ ((v ^ 0x7fc00000u) & (0u - nan)));
}

// The EPL values of a 16-byte piece of summaries, as fp32 (bf16 widened,
// fp8 decoded; exact in every case).  fp8 goes through the hardware
// conversion of code pairs, which decodes gfx950's e4m3 (bias 7, no
// infinities) to the same fp32 value as e4m3_value for every non-NaN code
// (checked for all 256 codes on the device); it returns a negative NaN for
// the two NaN codes, which are mapped to the positive quiet NaN e4m3_value
// gives them.
template <typename TS>
__device__ inline void piece_values(const u32x4 &w, float (&out)[16 / sizeof(TS)]) {
  if constexpr (sizeof(TS) == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = __uint_as_float(w[k]);
  } else if constexpr (sizeof(TS) == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = __uint_as_float(w[k] << 16);
      out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
      const float v[4] = {lo[0], lo[1], hi[0], hi[1]};
      // bit 7 of byte e set exactly when code e has its low seven bits all
      // ones (NaN); that bit moved to the sign flips the NaN to positive
      // (integer arithmetic: a comparison per value would leave a lane mask
      // per value in scalar registers)
      const uint32_t nan = ((w[k] & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[4 * k + e] = __uint_as_float(__float_as_uint(v[e]) ^ ((nan << (24 - 8 * e)) & 0x80000000u));
    }
  }
}

// The row's merge: the chunks' candidates (in block order: chunk by chunk, each in block
// order) hold the row's Top-K, since every block of it is among its own
// chunk's Top-K; an exact Top-K over them with the same order gives the
// row's.  The normaliser combines the chunks' (max, sum) pairs in chunk
// order.  Writes the kept blocks ascending with log g = s - lse, the
// current block (log g 0), then -1 padding.  R candidates per thread.
template <int R, int NT>
__device__ inline void merge_row(const DecodeParams &p, const SelectParams &sp, int row, float *red,
                                 int *cnt, SelectScratch &sel, uint64_t *runs) {
  constexpr int NWV = NT / kWave;
  const int tid = threadIdx.x;
  const int b = row / p.hkv;
  const int cur = ((p.seqlens[b] - 1) / kBlock) / p.coarse_div;  // history count
  const int kh = p.Kb - 1;
  const int ncand = sp.nchunk * kh;
  const int2 *cand = sp.cand + (long)row * ncand;
  float sv[R];
  int jv[R];
  uint32_t valid = 0u;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int x = R * tid + c;
    const int2 e = x < ncand ? cand[x] : make_int2(-1, 0);
    jv[c] = e.x;
    sv[c] = __int_as_float(e.y);
    if (e.x >= 0) valid |= 1u << c;
  }
  // the normaliser: chunks tid, tid + NT, ... by thread tid (the first PC
  // held in registers across the max, the rest, if any, read again), the
  // sums added in a fixed order
  const float2 *part = sp.part + (long)row * sp.nchunk;
  constexpr int PC = 4;
  float2 pv[PC];
#pragma unroll
  for (int u = 0; u < PC; ++u)
    pv[u] = tid + u * NT < sp.nchunk ? part[tid + u * NT] : make_float2(-INFINITY, 0.f);
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < PC; ++u) M = fmaxf(M, pv[u].x);
  for (int c = tid + PC * NT; c < sp.nchunk; c += NT) M = fmaxf(M, part[c].x);
  M = block_max<NWV>(M, red);
  float Lt = 0.f;
#pragma unroll
  for (int u = 0; u < PC; ++u)
    if (pv[u].y > 0.f) Lt += pv[u].y * expf(pv[u].x - M);
  for (int c = tid + PC * NT; c < sp.nchunk; c += NT) {
    const float2 q = part[c];
    if (q.y > 0.f) Lt += q.y * expf(q.x - M);
  }
  const float Lsum = block_sum<NWV>(Lt, red);
  const float lse = (cur == 0 || M == -INFINITY) ? -INFINITY : M + logf(Lsum);
  int nvalid_local = __popc(valid), nvalid;
  block_scan_int<NWV>(nvalid_local, nvalid, cnt);
  const int k = min(kh, cur);
  const bool keep_all = k >= nvalid;
  int32_t *oidx = sp.sel_idx + (long)row * p.Kb;
  float *olg = sp.sel_lg + (long)row * p.Kb;
  if constexpr (R == 1) {
    // one candidate per thread: the Top-K by ranks (entry order = thread
    // order = block order)
    if (k > 0) {
      const bool keep = keep_all ? (valid & 1u) != 0 : rank_keep<NT>(sv[0], valid & 1u, k, runs);
      int total;
      const int pos = block_scan_flag<NWV>(keep, total, cnt);
      if (keep) {
        oidx[pos] = jv[0];
        olg[pos] = lse == -INFINITY ? -INFINITY : sv[0] - lse;
      }
    }
  } else {
    Threshold th{0u, 0u, k};
    if (!keep_all && k > 0)
      th = radix_threshold<NT>(k, sel, [&](auto &&f) {
#pragma unroll
        for (int c = 0; c < R; ++c)
          if ((valid >> c) & 1u) f(order_key(sv[c]));
      });
    if (k > 0) {
      int pos, total;
      const uint32_t takem = kept_mask<R, NWV>(sv, valid, keep_all, th, cnt, pos, total);
#pragma unroll
      for (int c = 0; c < R; ++c)
        if ((takem >> c) & 1u) {
          oidx[pos] = jv[c];
          olg[pos] = lse == -INFINITY ? -INFINITY : sv[c] - lse;
          ++pos;
        }
    }
  }
  if (tid == 0) {
    oidx[k] = cur;
    olg[k] = 0.f;
    sp.gate_lse[row] = lse;
  }
  for (int x = k + 1 + tid; x < p.Kb; x += NT) {
    oidx[x] = -1;
    olg[x] = -INFINITY;
  }
}

// Decode selection: workgroup (chunk c, row b * hkv + g) takes history
// blocks [256 V c, 256 V (c + 1)) of the row, V consecutive blocks per
// thread.  A block's D values are NL 16-byte pieces (summary_index) that
// its thread requests all at once (a block of fp32 summaries is 32
// requests, bf16 16, fp8 8), before the query mean is formed; with one
// block per thread a wave's request for piece l is 1 KB of contiguous
// memory.  Each score is the fixed fp32
// order
//   qbar_e = (q_{gG} + ... + q_{gG+G-1})_e / G,
//   s_j    = (fmaf chain over e of qbar_e * summary_je) / sqrtf(d)
// (so every score is the one the oracle computes).  The workgroup writes the
// scores and keeps the chunk's exact Top-K (the Kb - 1 largest scores,
// earlier block on ties) in block order with the chunk's max and sum of
// exp(s - max).  (A single launch whose last chunk merges its row needs a
// device-scope release per workgroup, which writes back the L2 of its XCD:
// measured 15 times slower than the second launch.)
template <int D, int G, int V, typename TS, int NT>
__global__ __launch_bounds__(NT) void select_kernel(DecodeParams p, SelectParams sp) {
#pragma clang fp contract(off)
  constexpr int NWV = NT / kWave;
  constexpr int BB = D * (int)sizeof(TS);  // bytes of one block's summary
  constexpr int NL = BB / 16;              // 16-byte pieces per block
  constexpr int EPL = 16 / (int)sizeof(TS);
  static_assert(BB % 16 == 0, "a block's summary is whole 16-byte pieces");
  __shared__ __attribute__((aligned(16))) float qbar[D];
  __shared__ float red[NWV];
  __shared__ int cnt[NWV];
  __shared__ SelectScratch sel;
  __shared__ uint64_t runs[NT];
  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / p.hkv, g = row % p.hkv;
  const int tid = threadIdx.x;
  const int nhist = ((p.seqlens[b] - 1) / kBlock) / p.coarse_div;  // blocks or super-blocks
  const int kh = p.Kb - 1;
  const int lo = NT * V * c, n = max(0, min(nhist - lo, NT * V));  // valid blocks in the chunk
  const int j0 = lo + V * tid;  // this thread's first block
  uint32_t valid = 0u;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (j0 + v < nhist) valid |= 1u << v;

  float sv[V];
#pragma unroll
  for (int v = 0; v < V; ++v) sv[v] = -INFINITY;
  if (n > 0) {  // uniform: the chunk holds blocks of this row
    const __bf16 *q = static_cast<const __bf16 *>(p.q);
    float qv[G];  // the heads' values requested before the summaries
    if (tid < D) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) qv[hh] = (float)q[((long)b * p.hq + g * G + hh) * D + tid];
    }
    // block j's piece l at the row's uniform base plus a 32-bit byte offset
    // (a row of summaries spans nblk_stride * BB bytes): tile j / 64 of NL
    // KB, piece l's KB in it, the block's 16 bytes in that; blocks past the
    // history re-read its last block (their scores are discarded), so every
    // thread's requests issue without a branch
    const char *rbase =
        static_cast<const char *>(p.ksum) + (long)row * p.nblk_stride * (long)BB;
    auto load_block = [&](int j, u32x4 (&w)[NL]) {
      const int jj = min(j, nhist - 1);
      const unsigned off = (unsigned)(jj / 64) * (unsigned)(NL * 1024) + 16u * (unsigned)(jj % 64);
#pragma unroll
      for (int l = 0; l < NL; ++l)
        w[l] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(rbase + (off + 1024u * (unsigned)l)));
    };
    u32x4 w[NL];
    load_block(j0, w);
    if (tid < D) {
      float acc = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) acc = acc + qv[hh];
      qbar[tid] = acc / (float)G;
    }
    barrier_keep_requests();  // qbar visible; the summary requests stay in flight
    float *out = p.scores + (long)row * p.nblk_stride;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (v > 0) {  // one block's pieces in registers at a time
        __builtin_amdgcn_sched_barrier(0);
        load_block(j0 + v, w);
      }
      float a = 0.f;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        float x[EPL];
        piece_values<TS>(w[l], x);
#pragma unroll
        for (int k4 = 0; k4 < EPL; k4 += 4) {
          const float4 qe = *reinterpret_cast<const float4 *>(&qbar[l * EPL + k4]);
          a = fmaf(qe.x, x[k4 + 0], a);
          a = fmaf(qe.y, x[k4 + 1], a);
          a = fmaf(qe.z, x[k4 + 2], a);
          a = fmaf(qe.w, x[k4 + 3], a);
        }
      }
      if ((valid >> v) & 1u) {
        sv[v] = a / p.sqrt_d;
        out[j0 + v] = sv[v];
      }
    }
  }
  // the chunk's share of the normaliser
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < V; ++v) mx = fmaxf(mx, sv[v]);
  mx = block_max<NWV>(mx, red);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      if ((valid >> v) & 1u) sum += expf(sv[v] - mx);
  }
  sum = block_sum<NWV>(sum, red);
  // the chunk's Top-K: by ranks for one block per thread, else by a radix
  // select; the candidates go out in block order
  const int k = min(kh, n);
  const bool keep_all = k == n;
  int2 *cand = sp.cand + ((long)row * sp.nchunk + c) * kh;
  if constexpr (V == 1) {
    if (k > 0) {
      const bool keep = keep_all ? (valid & 1u) != 0 : rank_keep<NT>(sv[0], valid & 1u, k, runs);
      int total;
      const int pos = block_scan_flag<NWV>(keep, total, cnt);
      if (keep) cand[pos] = make_int2(j0, __float_as_int(sv[0]));
    }
  } else {
    Threshold th{0u, 0u, k};
    if (!keep_all && k > 0)
      th = radix_threshold<NT>(k, sel, [&](auto &&f) {
#pragma unroll
        for (int v = 0; v < V; ++v)
          if ((valid >> v) & 1u) f(order_key(sv[v]));
      });
    if (k > 0) {
      int pos, total;
      const uint32_t takem = kept_mask<V, NWV>(sv, valid, keep_all, th, cnt, pos, total);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if ((takem >> v) & 1u) {
          cand[pos] = make_int2(j0 + v, __float_as_int(sv[v]));
          ++pos;
        }
    }
  }
  for (int x = k + tid; x < kh; x += NT) cand[x] = make_int2(-1, __float_as_int(-INFINITY));
  if (tid == 0) sp.part[(long)row * sp.nchunk + c] = make_float2(mx, sum);

}

// Decode selection, phase 2: one workgroup of NT threads per row merges the
// chunks' candidates (merge_row), R per thread.
template <int R, int NT>
__global__ __launch_bounds__(NT) void select_merge_kernel(DecodeParams p, SelectParams sp) {
  __shared__ float red[NT / kWave];
  __shared__ int cnt[NT / kWave];
  __shared__ SelectScratch sel;
  __shared__ uint64_t runs[R == 1 ? NT : 1];
  merge_row<R, NT>(p, sp, blockIdx.x, red, cnt, sel, runs);
}

// Hierarchical selection, fine pass (review 7-2): one workgroup per row.
// The candidates are every block of the row's kept super-blocks (the coarse
// pass's Top-C, ascending) followed by the trailing history blocks that
// form no complete super-block -- all in block order, R consecutive
// candidates per thread (each candidate's summary requested as a whole).  Each candidate's pooled score is the same fixed
// fp32 order as in select_kernel; the gate normaliser runs over the
// candidates, and the kept set is their exact Top-K (radix select, earlier
// block on ties).  Writes the candidates' scores, the kept blocks ascending
// with log g = s - lse, the current block (log g 0), then -1 padding.
template <int D, int G, typename TS>
__global__ __launch_bounds__(512) void select_fine_kernel(DecodeParams p, HierParams h) {
#pragma clang fp contract(off)
  constexpr int NT = 512, NWV = NT / kWave, R = 2;
  constexpr int BB = D * (int)sizeof(TS), NL = BB / 16, EPL = 16 / (int)sizeof(TS);
  __shared__ __attribute__((aligned(16))) float qbar[D];
  __shared__ float red[NWV];
  __shared__ int cnt[NWV];
  __shared__ SelectScratch sel;
  __shared__ int ksup[NT * R / kCoarseBlocks];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int b = row / p.hkv, g = row % p.hkv;
  const int nhist = (p.seqlens[b] - 1) / kBlock;
  const int nsup = nhist / kCoarseBlocks;
  const int kc = min(h.C, nsup);
  const int ncand = kCoarseBlocks * kc + (nhist - kCoarseBlocks * nsup);
  if (tid < kc) ksup[tid] = h.kept[(long)row * (h.C + 1) + tid];
  if (tid < D) {
    const __bf16 *q = static_cast<const __bf16 *>(p.q);
    float qv[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) qv[hh] = (float)q[((long)b * p.hq + g * G + hh) * D + tid];
    float acc = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) acc = acc + qv[hh];
    qbar[tid] = acc / (float)G;
  }
  __syncthreads();
  const char *rbase =
      static_cast<const char *>(p.ksum) + (long)row * p.nblk_stride * (long)BB;
  float *out = p.scores + (long)row * p.nblk_stride;
  float sv[R];
  int jv[R];
  uint32_t valid = 0u;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int x = R * tid + c;
    sv[c] = -INFINITY;
    jv[c] = -1;
    if (x >= ncand) continue;
    const int j = x < kCoarseBlocks * kc
                      ? kCoarseBlocks * ksup[x / kCoarseBlocks] + x % kCoarseBlocks
                      : kCoarseBlocks * nsup + (x - kCoarseBlocks * kc);
    jv[c] = j;
    valid |= 1u << c;
    const unsigned off = (unsigned)(j / 64) * (unsigned)(NL * 1024) + 16u * (unsigned)(j % 64);
    u32x4 w[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l)
      w[l] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(rbase + (off + 1024u * (unsigned)l)));
    float a = 0.f;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      float x[EPL];
      piece_values<TS>(w[l], x);
#pragma unroll
      for (int k4 = 0; k4 < EPL; k4 += 4) {
        const float4 qe = *reinterpret_cast<const float4 *>(&qbar[l * EPL + k4]);
        a = fmaf(qe.x, x[k4 + 0], a);
        a = fmaf(qe.y, x[k4 + 1], a);
        a = fmaf(qe.z, x[k4 + 2], a);
        a = fmaf(qe.w, x[k4 + 3], a);
      }
    }
    sv[c] = a / p.sqrt_d;
    out[j] = sv[c];
  }
  // the normaliser over the candidates
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < R; ++c) mx = fmaxf(mx, sv[c]);
  mx = block_max<NWV>(mx, red);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int c = 0; c < R; ++c)
      if ((valid >> c) & 1u) sum += expf(sv[c] - mx);
  }
  sum = block_sum<NWV>(sum, red);
  const float lse = (ncand == 0 || mx == -INFINITY) ? -INFINITY : mx + logf(sum);
  const int k = min(p.Kb - 1, ncand);
  const bool keep_all = k == ncand;
  Threshold th{0u, 0u, k};
  if (!keep_all && k > 0)
    th = radix_threshold<NT>(k, sel, [&](auto &&f) {
#pragma unroll
      for (int c = 0; c < R; ++c)
        if ((valid >> c) & 1u) f(order_key(sv[c]));
    });
  int32_t *oidx = h.sel_idx + (long)row * p.Kb;
  float *olg = h.sel_lg + (long)row * p.Kb;
  if (k > 0) {
    int pos, total;
    const uint32_t takem = kept_mask<R, NWV>(sv, valid, keep_all, th, cnt, pos, total);
#pragma unroll
    for (int c = 0; c < R; ++c)
      if ((takem >> c) & 1u) {
        oidx[pos] = jv[c];
        olg[pos] = lse == -INFINITY ? -INFINITY : sv[c] - lse;
        ++pos;
      }
  }
  if (tid == 0) {
    oidx[k] = nhist;  // the current block
    olg[k] = 0.f;
    h.gate_lse[row] = lse;
  }
  for (int x = k + 1 + tid; x < p.Kb; x += NT) {
    oidx[x] = -1;
    olg[x] = -INFINITY;
  }
}

template <int D, typename TS>
static void launch_fine_g(const DecodeParams &p, const HierParams &h, hipStream_t stream) {
  const dim3 grid(p.batch * p.hkv);
  switch (p.hq / p.hkv) {
    case 1: hipLaunchKernelGGL((select_fine_kernel<D, 1, TS>), grid, dim3(512), 0, stream, p, h); break;
    case 2: hipLaunchKernelGGL((select_fine_kernel<D, 2, TS>), grid, dim3(512), 0, stream, p, h); break;
    case 4: hipLaunchKernelGGL((select_fine_kernel<D, 4, TS>), grid, dim3(512), 0, stream, p, h); break;
    default: hipLaunchKernelGGL((select_fine_kernel<D, 8, TS>), grid, dim3(512), 0, stream, p, h); break;
  }
}

hipError_t launch_decode_select_fine(const DecodeParams &p, const HierParams &h,
                                     hipStream_t stream) {
  if (p.D == 128) {
    if (p.sum_kind == kSumBf16) launch_fine_g<128, __bf16>(p, h, stream);
    else if (p.sum_kind == kSumFp8) launch_fine_g<128, uint8_t>(p, h, stream);
    else launch_fine_g<128, float>(p, h, stream);
  } else {
    if (p.sum_kind == kSumBf16) launch_fine_g<64, __bf16>(p, h, stream);
    else if (p.sum_kind == kSumFp8) launch_fine_g<64, uint8_t>(p, h, stream);
    else launch_fine_g<64, float>(p, h, stream);
  }
  return hipGetLastError();
}

hipError_t launch_pool_coarse(const DecodeParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(pool_coarse_kernel, dim3(p.cstride, p.batch * p.hkv), dim3(128), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D, int G, int V, typename TS, int NT>
static void launch_select(const DecodeParams &p, const SelectParams &sp, hipStream_t stream) {
  const dim3 grid(sp.nchunk, p.batch * p.hkv);
  hipLaunchKernelGGL((select_kernel<D, G, V, TS, NT>), grid, dim3(NT), 0, stream, p, sp);
}

template <int D, int G, typename TS>
static void launch_select_v(const DecodeParams &p, const SelectParams &sp, hipStream_t stream) {
  // 512-thread chunks only for one block per thread and 1- or 2-byte
  // summaries (fp32 ones hold too many registers for 8 waves of a workgroup
  // beside other workgroups)
  if (sizeof(TS) < 4 && sp.chunk_threads == 512 && sp.chunk_v == 1) {
    launch_select<D, G, 1, TS, 512>(p, sp, stream);
    return;
  }
  switch (sp.chunk_v) {
    case 1: launch_select<D, G, 1, TS, 256>(p, sp, stream); break;
    case 2: launch_select<D, G, 2, TS, 256>(p, sp, stream); break;
    case 4: launch_select<D, G, 4, TS, 256>(p, sp, stream); break;
    default: launch_select<D, G, 8, TS, 256>(p, sp, stream); break;
  }
}

template <int D, typename TS>
static void launch_select_g(const DecodeParams &p, const SelectParams &sp, hipStream_t stream) {
  switch (p.hq / p.hkv) {
    case 1: launch_select_v<D, 1, TS>(p, sp, stream); break;
    case 2: launch_select_v<D, 2, TS>(p, sp, stream); break;
    case 4: launch_select_v<D, 4, TS>(p, sp, stream); break;
    default: launch_select_v<D, 8, TS>(p, sp, stream); break;
  }
}

hipError_t launch_decode_select(const DecodeParams &p, const SelectParams &sp,
                                hipStream_t stream) {
  if (p.D == 128) {
    if (p.sum_kind == kSumBf16) launch_select_g<128, __bf16>(p, sp, stream);
    else if (p.sum_kind == kSumFp8) launch_select_g<128, uint8_t>(p, sp, stream);
    else launch_select_g<128, float>(p, sp, stream);
  } else {
    if (p.sum_kind == kSumBf16) launch_select_g<64, __bf16>(p, sp, stream);
    else if (p.sum_kind == kSumFp8) launch_select_g<64, uint8_t>(p, sp, stream);
    else launch_select_g<64, float>(p, sp, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ncand = sp.nchunk * (p.Kb - 1);
  const dim3 grid(p.batch * p.hkv);
  // up to 256 candidates: one per thread, Top-K by ranks; more: R per thread
  // of 256, radix select (one candidate per thread of 1024 with the ranks'
  // 16 runs measured slower than the radix select with 4 per thread)
  if (ncand <= 256)
    hipLaunchKernelGGL((select_merge_kernel<1, 256>), grid, dim3(256), 0, stream, p, sp);
  else if (ncand <= 512)
    hipLaunchKernelGGL((select_merge_kernel<2, 256>), grid, dim3(256), 0, stream, p, sp);
  else if (ncand <= 1024)
    hipLaunchKernelGGL((select_merge_kernel<4, 256>), grid, dim3(256), 0, stream, p, sp);
  else if (ncand <= 2048)
    hipLaunchKernelGGL((select_merge_kernel<8, 256>), grid, dim3(256), 0, stream, p, sp);
  else
    hipLaunchKernelGGL((select_merge_kernel<16, 256>), grid, dim3(256), 0, stream, p, sp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attend
// A workgroup takes one split of the kept blocks of one (sequence, kv head)
// row; each of its 4 waves streams every 4th of those blocks on its own
// (own online softmax, no barrier until the end).  Per 64-token block a
// wave runs both products on 16x16x32 bf16 MFMAs with the G query heads as
// the 16 columns (unused columns see zero queries):
//   S^T[key][head] = K Q^T  -- K rows read from the tile in the key order
//                              that makes each lane's S^T registers the 8
//                              consecutive keys the next product contracts
//                              over;
//   O^T[d][head]  += V^T P^T -- V read transposed from its tile.
// K and V pass through wave-private swizzled LDS tiles.  The next block's
// K and V are requested into staging registers (1 KB contiguous per load,
// 32-bit offsets from a uniform base) before the current block is
// computed, and written to the tiles once the current block's reads are
// done.  All requests land in registers, so the compiler's wait counts
// stay exact.  The running max
// per head moves only when a score passes it by more than kDecRescale
// (log2 units).  At the end the waves are merged through LDS into the
// split's unnormalised partial.
constexpr float kDecRescale = 8.f;
constexpr int kDecStepKeys = 32;  // keys per step: 32 or 64

template <int D, int G>
__global__ __launch_bounds__(256, kDecodeWgPerCu) void decode_attend_kernel(DecodeParams p) {
  static_assert(G <= 16, "query heads of a group are the 16 MFMA columns");
  constexpr int SK = kDecStepKeys;         // keys per step (a block is 64 / SK steps)
  constexpr int SPB = kBlock / SK;         // steps per block
  constexpr int NSL = SK / 32;             // 32-key slices per step
  constexpr int NKS = D / 32;              // contraction slices of S^T
  constexpr int NDT = D / 16;              // 16-row tiles of O^T
  constexpr int TILE = SK * D;             // tile elements
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPS = kWave / CPR;         // rows per 1 KB request
  constexpr int NREQ = SK / RPS;           // requests per tile
  static_assert(kMaxBudget / 4 <= kWave, "a wave's blocks fit one per lane");
  __shared__ __attribute__((aligned(16))) __bf16 ktile[4][TILE];  // one per wave
  __shared__ __attribute__((aligned(16))) __bf16 vtile[4][TILE];
  __shared__ float s_m[4][G], s_l[4][G];
  static_assert(G * D * 4 <= TILE * 2, "a wave's merged output fits in its K tile");

  const int row = blockIdx.y;  // b * hkv + g
  const int split = blockIdx.x;
  const int b = row / p.hkv, g = row % p.hkv;
  const int L = p.seqlens[b];
  const int cur = (L - 1) / kBlock;
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int q16 = lane / 16, c16 = lane % 16;
  const int32_t *sel = p.sel_idx + (long)row * p.Kb;
  const float *slg = p.sel_lg ? p.sel_lg + (long)row * p.Kb : nullptr;
  const int s0 = split * p.per_split + wave, s1 = min(p.Kb, split * p.per_split + p.per_split);
  const int nb = s0 < s1 ? (s1 - s0 + 3) / 4 : 0;  // this wave's blocks: s0, s0 + 4, ...
  const __bf16 *kc = static_cast<const __bf16 *>(p.k);
  const __bf16 *vc = static_cast<const __bf16 *>(p.v);
  const __bf16 *q = static_cast<const __bf16 *>(p.q);

  // Q^T as B operands: column c16 = query head c16 of the group (zero past G)
  // (columns past G load head 0 and are zeroed afterwards: no branch, the
  // loads issue back to back)
  bf16x8 qreg[NKS];
  {
    const __bf16 *qp = q + ((long)b * p.hq + g * G + (c16 < G ? c16 : 0)) * D + 8 * q16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8 *>(qp + 32 * ks);
    if (G < 16) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qreg[ks] = c16 < G ? qreg[ks] : bf16x8{};
    }
  }
  // Blocks of this wave, looked up once: lane k holds block k's first-row
  // offset (K and V alike), valid keys and log gate, read back with
  // readlane (a memory lookup inside the loop would wait for every request
  // in flight).  A slot that keeps no block (index -1 or past the current
  // block) reads the current block with every key masked.
  long b_off = 0;
  int b_nv = 0;
  float b_lg2 = 0.f;
  if (lane < nb) {
    const int c = s0 + 4 * lane;
    // the log gate is requested with the index (an ungated call reads the
    // index array in its place and discards it), so only the page lookup
    // waits for the index
    const float lgv = *(slg ? slg + c : reinterpret_cast<const float *>(sel + c));
    const int j = sel[c];
    const bool ok = j >= 0 && j <= cur;
    const int jj = ok ? j : cur;
    b_nv = !ok ? 0 : (jj == cur ? L - cur * kBlock : kBlock);
    b_off = kv_row(p, kc, b, g, jj * kBlock) - kc;  // a block never crosses a page
    b_lg2 = slg ? lgv * kLog2e : 0.f;
  }
  wait_vmem_all();

  // Staging, two register sets: lane l takes 16-byte chunk l % CPR of rows
  // i * RPS + l / CPR of the step (each load is RPS whole rows,
  // contiguous), K and V alike.
  u32x4 kst[2][NREQ], vst[2][NREQ];
  const int r_in = lane / CPR, pc = lane % CPR;
  // Addresses: a uniform base (the step's first row) plus a 32-bit byte
  // offset per lane, so the loads take the scalar-base form and need no
  // 64-bit address registers.
  auto issue_step = [&](auto SET, int st) {
    constexpr int x = decltype(SET)::value;
    const int k = st / SPB, ko = (st % SPB) * SK;
    const long off = lane_value(b_off, k);
    const int last = max(lane_value(b_nv, k), 1) - 1;  // rows past the end are never read
    const char *kb = reinterpret_cast<const char *>(kc + off);
    const char *vb = reinterpret_cast<const char *>(vc + off);
#pragma unroll
    for (int i = 0; i < NREQ; ++i) {
      const unsigned ob = (unsigned)(min(ko + i * RPS + r_in, last) * (D * 2) + pc * 16);
      // streaming, non-temporal: a kept block is read once per decode
      kst[x][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + ob));
      vst[x][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vb + ob));
    }
  };
  // staged K, V -> the wave's tiles, chunks permuted by the swizzle
  auto store_step = [&](auto SET) {
    constexpr int x = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < NREQ; ++i) {
      const int o = Swz<__bf16, D>::off(i * RPS + r_in, pc * 8);
      *reinterpret_cast<u32x4 *>(ktile[wave] + o) = kst[x][i];
      *reinterpret_cast<u32x4 *>(vtile[wave] + o) = vst[x][i];
    }
  };
  using X0 = std::integral_constant<int, 0>;
  using X1 = std::integral_constant<int, 1>;
  // key (within the step) of row r (0..15) of S^T tile t of 32-key slice
  // sl: output register i of lane group q16 then holds key 32 sl + 8 q16 +
  // 4 t + i, the order the next product contracts over
  const int krow = 8 * (c16 / 4) + (c16 % 4);

  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{};
  float m = -INFINITY, l = 0.f;  // per column (head c16); l is this lane's share

  auto compute_step = [&](int st) {
    const int k = st / SPB, ko = (st % SPB) * SK;
    const int nv = lane_value(b_nv, k) - ko;  // valid keys of this step (may be <= 0)
    const float lg2 = lane_value(b_lg2, k);
    const __bf16 *kt = ktile[wave], *vt = vtile[wave];
    f32x4 sacc[NSL][2];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[sl][t] = f32x4{};
        const int key = 32 * sl + 4 * t + krow;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          sacc[sl][t] = mfma16(tile_op<__bf16, D>(kt, key, 32 * ks + 8 * q16), qreg[ks],
                               sacc[sl][t]);
      }
    float z[NSL][2][4];
    bool need = false;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 32 * sl + 8 * q16 + 4 * t + i;
          z[sl][t][i] = key < nv ? sacc[sl][t][i] * p.scale_log2 + lg2 : -INFINITY;
          need |= z[sl][t][i] > m + kDecRescale;
        }
    if (__any(need)) {  // rare: move the running max of each column, rescale
      float mx = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[sl][t][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      if (mn > m) {
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        m = mn;
      }
    }
    // P^T as B operands (8 consecutive keys per lane), then O^T += V^T P^T
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = z[sl][t][i] == -INFINITY ? 0.f : fast_exp2(z[sl][t][i] - m);
          l += pr;
          pb[4 * t + i] = (__bf16)pr;
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        oacc[dt] = mfma16(tile_op_rows16<D>(vt, 32 * sl, 16 * dt), pb, oacc[dt]);
    }
  };

  // Step st + 2 is requested (into the register set step st freed) before
  // step st is computed; step st + 1, requested one step earlier, is then
  // written to the tiles.  Past the end the last step is re-requested
  // (cache hits), so the count of requests in flight is the same on every
  // path.  The tiles are rewritten only after this wave's reads of them
  // have completed, and read again only after the writes completed
  // (transposed reads issued while the wave's own LDS writes are pending
  // have returned wrong data on gfx950).
  constexpr int PER_STEP = 2 * NREQ;  // requests per step
  const int nst = nb * SPB;
  auto step = [&](auto CUR, auto NXT, int st) {
    issue_step(CUR, min(st + 2, nst - 1));  // set CUR held step st, now stored
    compute_step(st);
    wait_lds_all();
    wait_vmem<PER_STEP>();  // step st + 1 (set NXT) has landed
    store_step(NXT);
    wait_lds_all();
  };
  if (nst > 0) {
    issue_step(X0{}, 0);
    issue_step(X1{}, min(1, nst - 1));
    wait_vmem<PER_STEP>();
    store_step(X0{});
    wait_vmem_all();  // nothing in flight at the loop entry
    wait_lds_all();
    if constexpr (SPB % 2 == 0) {
      // an even number of steps: no path leaves the loop between the two
      // halves, so the requests of the first half are never counted as
      // pending when the next iteration reuses its registers
      for (int st = 0; st < nst; st += 2) {
        step(X0{}, X1{}, st);
        step(X1{}, X0{}, st + 1);
      }
    } else {
      for (int st = 0; st < nst; st += 2) {
        step(X0{}, X1{}, st);
        if (st + 1 >= nst) break;
        step(X1{}, X0{}, st + 1);
      }
    }
    wait_vmem<0>();
  }

  // Merge the 4 lane groups of each column, then the 4 waves, into this
  // split's unnormalised partial.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // each wave's output goes to its own K tile, which it no longer reads
  auto obuf = [&](int w, int hh, int d) -> float & {
    return reinterpret_cast<float *>(ktile[w])[hh * D + d];
  };
  wait_lds_all();
  if (c16 < G) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) obuf(wave, c16, 16 * dt + 4 * q16 + i) = oacc[dt][i];
    if (q16 == 0) {
      s_m[wave][c16] = m;
      s_l[wave][c16] = l;
    }
  }
  __syncthreads();
  if (p.nsplit == 1) {
    // the workgroup holds the whole row: normalise and write o and lse here
    // (the same arithmetic as the combine over one split)
    __shared__ float s_M[G], s_L[G];
    if (threadIdx.x < G) {
      const int hh = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][hh]);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = s_m[w][hh] == -INFINITY ? 0.f : fast_exp2(s_m[w][hh] - M);
        sum += sc * s_l[w][hh];
      }
      const float wgt = M == -INFINITY ? 0.f : 1.f;  // exp2(M - M) of the one split
      s_M[hh] = M;
      s_L[hh] = sum * wgt;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < G * D; x += 256) {
      const int hh = x / D, d = x % D;
      const float M = s_M[hh];
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = s_m[w][hh] == -INFINITY ? 0.f : fast_exp2(s_m[w][hh] - M);
        sum += sc * obuf(w, hh, d);
      }
      const float acc = sum * (M == -INFINITY ? 0.f : 1.f);
      const long at = ((long)b * p.hq + g * G + hh) * D + d;
      const float val = acc / s_L[hh];
      if (p.out_bf16)
        static_cast<__bf16 *>(p.o)[at] = from_f32<__bf16>(val);
      else
        static_cast<float *>(p.o)[at] = val;
      if (d == 0 && p.lse)
        p.lse[(long)b * p.hq + g * G + hh] = (M + fast_log2(s_L[hh])) * kLn2;
    }
    return;
  }
  float *out = p.partial + ((long)row * p.nsplit + split) * G * (D + 2);
  for (int x = threadIdx.x; x < G * (D + 1); x += 256) {
    const int hh = x / (D + 1), d = x % (D + 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][hh]);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = s_m[w][hh] == -INFINITY ? 0.f : fast_exp2(s_m[w][hh] - M);
      sum += sc * (d < D ? obuf(w, hh, d) : s_l[w][hh]);
    }
    if (d < D) {
      out[hh * (D + 2) + d] = sum;
    } else {
      out[hh * (D + 2) + D] = M;
      out[hh * (D + 2) + D + 1] = sum;
    }
  }
}

// Merge the splits of every (sequence, kv head) in split order.
template <int D, int G, typename TO>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int row = blockIdx.x;
  const int b = row / p.hkv, g = row % p.hkv;
  const float *part = p.partial + (long)row * p.nsplit * G * (D + 2);
  TO *o = static_cast<TO *>(p.o);
  constexpr int U = 8;  // splits whose partials are loaded together
  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int hh = x / D, d = x % D;
    float M = -INFINITY;
    for (int s0 = 0; s0 < p.nsplit; s0 += U) {
      float mv[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        mv[u] = (s0 + u < p.nsplit) ? part[((s0 + u) * G + hh) * (D + 2) + D] : -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) M = fmaxf(M, mv[u]);
    }
    float Lsum = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < p.nsplit; s0 += U) {
      float mv[U], lv[U], av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float *ps = part + ((s0 + u) * G + hh) * (D + 2);
        const bool in = s0 + u < p.nsplit;
        mv[u] = in ? ps[D] : -INFINITY;
        lv[u] = in ? ps[D + 1] : 0.f;
        av[u] = in ? ps[d] : 0.f;
      }
      // splits in order; a split past the end adds exact zeros
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = (mv[u] == -INFINITY) ? 0.f : fast_exp2(mv[u] - M);
        Lsum += lv[u] * w;
        acc += av[u] * w;
      }
    }
    const int h = g * G + hh;
    o[((long)b * p.hq + h) * D + d] = from_f32<TO>(acc / Lsum);
    if (d == 0 && p.lse) p.lse[(long)b * p.hq + h] = (M + fast_log2(Lsum)) * kLn2;
  }
}

// ------------------------------------------------------------------ launch
hipError_t launch_pool_keys(const DecodeParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(pool_keys_kernel, dim3(p.nblk_stride, p.batch * p.hkv), dim3(128), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_append(const DecodeParams &p, const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(p.batch * p.hkv), dim3(128), 0, stream, p,
                     static_cast<const __bf16 *>(k_new), static_cast<const __bf16 *>(v_new),
                     static_cast<__bf16 *>(k_cache), static_cast<__bf16 *>(v_cache));
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_attend_t(const DecodeParams &p, hipStream_t stream) {
  const int rows = p.batch * p.hkv;
  hipLaunchKernelGGL((decode_attend_kernel<D, G>), dim3(p.nsplit, rows), dim3(256), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;  // one split: already final
  if (p.out_bf16)
    hipLaunchKernelGGL((decode_combine_kernel<D, G, __bf16>), dim3(rows), dim3(256), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, G, float>), dim3(rows), dim3(256), 0, stream,
                       p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attend_d(const DecodeParams &p, hipStream_t stream) {
  switch (p.hq / p.hkv) {
    case 1: return launch_attend_t<D, 1>(p, stream);
    case 2: return launch_attend_t<D, 2>(p, stream);
    case 4: return launch_attend_t<D, 4>(p, stream);
    case 8: return launch_attend_t<D, 8>(p, stream);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_decode_attend(const DecodeParams &p, hipStream_t stream) {
  return p.D == 128 ? launch_attend_d<128>(p, stream) : launch_attend_d<64>(p, stream);
}

// ------------------------------------------------------------------ scratch
// Split partials of sas_decode_noalloc: a fixed array in device memory, one
// copy per device (each device that runs the library holds it until the
// process ends).  In host code `decode_scratch` names a host-side stand-in,
// not the device array: its device address is asked for once per device
// (with that device current) and kept; kernels get that address.  Calls on
// one device share the array and find the previous call's contents in it;
// the partials of a call are all written before its combine reads them.
static __device__ __align__(256) float decode_scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch_address(float **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float *per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(decode_scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<float *>(addr);
  }
  *out = per_device[dev];
  return hipSuccess;
}

}  // namespace sas

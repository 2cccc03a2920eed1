// Decode path for gfx950 (dimensionstp.github.io review, section 3-7:
// score cached block summaries, keep the Top-K per query group, read the
// kept blocks of the paged KV cache, run the block-sparse decode kernel;
// GQA groups share one selection).
//
//   pool:    summary of block j = mean of its 64 keys, summed in token order
//            in fp32 (one thread per (block, channel), reads coalesced
//            along the channel).
//   scores:  s_j = (fmaf chain over channels of qbar * summary) / sqrt(d),
//            qbar = sum of the group's query heads in head order / G, all
//            in fp32 in exactly this order, so the Top-K decision is taken
//            on values the oracle reproduces bit for bit.  Summaries are
//            channel-major, so lanes (blocks) read consecutive addresses.
//   attend:  split-K over the kept blocks of every (sequence, kv head):
//            each wave of a workgroup streams its own share of 64-token
//            K/V blocks (16-byte coalesced loads, several passes in flight
//            in registers), keeps an fp32 online softmax per query head
//            with the block's log gate added; the waves merge into an
//            unnormalised partial per split, and a second kernel merges
//            the partials with a log-sum-exp combine in a fixed order.
#include <type_traits>

#include "sas_device.h"
#include "sas_launch.h"
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

// A block summary (the fp32 mean) stored as fp32, or rounded to the nearest
// bf16 (ties to even) when summaries are bf16.
__device__ inline void store_summary(const DecodeParams &p, long idx, float v) {
  if (p.sum_bf16)
    static_cast<__bf16 *>(p.ksum)[idx] = (__bf16)v;
  else
    static_cast<float *>(p.ksum)[idx] = v;
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
  store_summary(p, (((long)b * p.hkv + g) * p.D + e) * p.nblk_stride + j, acc / (float)kBlock);
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
    store_summary(p, (((long)b * p.hkv + g) * p.D + e) * p.nblk_stride + j,
                  acc / (float)kBlock);
  }
}

// ------------------------------------------------------------------ scores
template <typename TS>
__global__ __launch_bounds__(256) void pooled_scores_kernel(DecodeParams p) {
#pragma clang fp contract(off)
  __shared__ float qbar[256];
  const int bg = blockIdx.y;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int G = p.hq / p.hkv;
  const __bf16 *q = static_cast<const __bf16 *>(p.q);
  for (int e = threadIdx.x; e < p.D; e += blockDim.x) {
    float acc = 0.f;
    for (int hh = 0; hh < G; ++hh) acc = acc + (float)q[((long)b * p.hq + g * G + hh) * p.D + e];
    qbar[e] = acc / (float)G;
  }
  __syncthreads();
  const int nhist = (p.seqlens[b] - 1) / kBlock;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nhist) return;
  const TS *ks =
      static_cast<const TS *>(p.ksum) + ((long)b * p.hkv + g) * p.D * p.nblk_stride + j;
  float acc = 0.f;
  for (int e = 0; e < p.D; ++e) acc = fmaf(qbar[e], (float)ks[(long)e * p.nblk_stride], acc);
  p.scores[((long)b * p.hkv + g) * p.nblk_stride + j] = acc / p.sqrt_d;
}

// V consecutive blocks per thread (4: 16-byte fp32 / 8-byte bf16 loads; 1 for short grids, so
// that a single long sequence still spreads over every compute unit), V
// independent chains each in channel order, so every score is bit-identical
// to the one-block form; channels in batches of 64 / V loads in flight.  For
// summary strides that are multiples of 4.
template <int D, int V, typename TS>
__global__ __launch_bounds__(256) void pooled_scores_vec_kernel(DecodeParams p) {
#pragma clang fp contract(off)
  using vec = TS __attribute__((ext_vector_type(V)));
  __shared__ float qbar[D];
  const int bg = blockIdx.y;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int G = p.hq / p.hkv;
  const __bf16 *q = static_cast<const __bf16 *>(p.q);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float acc = 0.f;
    for (int hh = 0; hh < G; ++hh) acc = acc + (float)q[((long)b * p.hq + g * G + hh) * D + e];
    qbar[e] = acc / (float)G;
  }
  __syncthreads();
  const int nhist = (p.seqlens[b] - 1) / kBlock;
  const int j0 = V * (blockIdx.x * blockDim.x + threadIdx.x);
  if (j0 >= nhist) return;
  const TS *ks =
      static_cast<const TS *>(p.ksum) + ((long)b * p.hkv + g) * D * p.nblk_stride + j0;
  float a[V];
#pragma unroll
  for (int c = 0; c < V; ++c) a[c] = 0.f;
  constexpr int BATCH = 64 / V;
#pragma unroll 1
  for (int e0 = 0; e0 < D; e0 += BATCH) {
    vec v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      v[u] = *reinterpret_cast<const vec *>(ks + (long)(e0 + u) * p.nblk_stride);
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float w = qbar[e0 + u];
#pragma unroll
      for (int c = 0; c < V; ++c) a[c] = fmaf(w, (float)v[u][c], a[c]);
    }
  }
  float *out = p.scores + ((long)b * p.hkv + g) * p.nblk_stride + j0;
#pragma unroll
  for (int c = 0; c < V; ++c)
    if (j0 + c < nhist) out[c] = a[c] / p.sqrt_d;
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
      kst[x][i] = *reinterpret_cast<const u32x4 *>(kb + ob);
      vst[x][i] = *reinterpret_cast<const u32x4 *>(vb + ob);
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

template <typename TS>
static hipError_t launch_pooled_scores_t(const DecodeParams &p, hipStream_t stream) {
  if (p.nblk_stride % 4 == 0 && (p.D == 128 || p.D == 64)) {
    const dim3 grid4((p.nblk_stride / 4 + 255) / 256, p.batch * p.hkv);
    const dim3 grid1((p.nblk_stride + 255) / 256, p.batch * p.hkv);
    const bool narrow = (long)grid4.x * grid4.y < 256;  // fewer workgroups than CUs
    if (p.D == 128) {
      if (narrow)
        hipLaunchKernelGGL((pooled_scores_vec_kernel<128, 1, TS>), grid1, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((pooled_scores_vec_kernel<128, 4, TS>), grid4, dim3(256), 0, stream, p);
    } else {
      if (narrow)
        hipLaunchKernelGGL((pooled_scores_vec_kernel<64, 1, TS>), grid1, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((pooled_scores_vec_kernel<64, 4, TS>), grid4, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(pooled_scores_kernel<TS>, dim3((p.nblk_stride + 255) / 256, p.batch * p.hkv),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pooled_scores(const DecodeParams &p, hipStream_t stream) {
  return p.sum_bf16 ? launch_pooled_scores_t<__bf16>(p, stream)
                    : launch_pooled_scores_t<float>(p, stream);
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

}  // namespace sas

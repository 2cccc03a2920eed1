// Exact Top-K over fp32 scores held in registers, one workgroup per row of
// candidates: the order-preserving key map, workgroup reductions and scans,
// the radix select of the k-th largest key, and the kept set in candidate
// order.  Shared by the training gate (gate.hip) and the decode selection
// (decode.hip).
//
// Order: larger score first, the earlier candidate on ties, -0 == +0.
// Candidates are entries R * tid + c (c = 0..R-1) of the workgroup's row,
// so entry order is thread order; the kept set is emitted in that order.
#pragma once
#include "sas_device.h"

namespace sas {

// A 32-bit key whose unsigned order is the order of the floats (-0 mapped
// to +0 first, so the two compare equal).
__device__ inline uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup reductions and scans through a small LDS scratch (NWV waves).
template <int NWV>
__device__ inline float block_max(float x, float *red) {
  x = wave_max(x);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < NWV; ++k) r = fmaxf(r, red[k]);
  return r;
}

template <int NWV>
__device__ inline float block_sum(float x, float *red) {
  x = wave_sum(x);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < NWV; ++k) r += red[k];  // fixed order: deterministic
  return r;
}

// Exclusive prefix sum of a non-negative count over the workgroup in
// thread order, and the total.
template <int NWV>
__device__ inline int block_scan_int(int x, int &total, int *cnt) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int incl = x;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == kWave - 1) cnt[w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NWV; ++k) {
    if (k < w) off += cnt[k];
    total += cnt[k];
  }
  return off + incl - x;
}

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the total.
template <int NWV>
__device__ inline int block_scan_flag(bool flag, int &total, int *cnt) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) cnt[w] = __popcll(m);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NWV; ++k) {
    if (k < w) off += cnt[k];
    total += cnt[k];
  }
  return off + below;
}

// LDS a radix select needs.
struct SelectScratch {
  int hist[256];
  int bin, rem, cnt;
};

// The k-th largest key among a workgroup's candidates, as (prefix, pmask,
// remaining): a candidate is kept when its key masked by pmask is above
// prefix, or equal to it and among the first `remaining` such candidates in
// entry order.  4 passes of 8 bits (LDS histograms); the select stops early
// once the threshold bin is kept whole.  for_each(f) must call
// f(candidate_key) for this thread's valid candidates.  Requires 0 < k <
// number of valid candidates.
struct Threshold {
  uint32_t prefix, pmask;
  int remaining;
};

template <int NT, typename ForEach>
__device__ inline Threshold radix_threshold(int k, SelectScratch &s, ForEach &&for_each) {
  const int tid = threadIdx.x;
  Threshold t{0u, 0u, k};
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += NT) s.hist[b] = 0;
    __syncthreads();
    for_each([&](uint32_t key) {
      if ((key & t.pmask) == t.prefix) atomicAdd(&s.hist[(key >> shift) & 255u], 1);
    });
    __syncthreads();
    if (tid < kWave) {
      const int lane = tid;
      // lane owns bins 4 lane .. 4 lane + 3; suffix sums run from the top bin
      const int c0 = s.hist[4 * lane], c1 = s.hist[4 * lane + 1], c2 = s.hist[4 * lane + 2],
                c3 = s.hist[4 * lane + 3];
      const int local = c0 + c1 + c2 + c3;
      int incl = local;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_down(incl, o);
        if (lane + o < kWave) incl += y;
      }
      int cum = incl - local;  // keys in bins above this lane's four
      const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int x = 3; x >= 0; --x) {
        if (cum < t.remaining && cum + cs[x] >= t.remaining) {
          s.bin = 4 * lane + x;
          s.rem = t.remaining - cum;
          s.cnt = cs[x];
        }
        cum += cs[x];
      }
    }
    __syncthreads();
    t.prefix |= (uint32_t)s.bin << shift;
    t.pmask |= 255u << shift;
    t.remaining = s.rem;
    const bool whole_bin = s.rem == s.cnt;
    __syncthreads();
    // every key of the threshold bin is kept: the bits below it cannot
    // change the kept set
    if (whole_bin) break;
  }
  return t;
}

// This thread's kept candidates (bit c = entry R tid + c) given the
// threshold, for candidates whose bit is set in `valid`; keep_all keeps
// every valid candidate.  Also returns, through pos, the number of kept
// candidates in earlier threads (the output position of this thread's
// first) and through total the number kept in all.
template <int R, int NWV>
__device__ inline uint32_t kept_mask(const float (&sv)[R], uint32_t valid, bool keep_all,
                                     const Threshold &t, int *cnt, int &pos, int &total) {
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    if (!((valid >> c) & 1u)) continue;
    const uint32_t key = order_key(sv[c]) & t.pmask;
    if (keep_all || key > t.prefix) gtm |= 1u << c;
    else if (key == t.prefix) eqm |= 1u << c;
  }
  int eq_tot;
  int eq_rank = block_scan_int<NWV>(__popc(eqm), eq_tot, cnt);
  uint32_t takem = gtm;
#pragma unroll
  for (int c = 0; c < R; ++c)
    if ((eqm >> c) & 1u) {
      if (eq_rank < t.remaining) takem |= 1u << c;
      ++eq_rank;
    }
  pos = block_scan_int<NWV>(__popc(takem), total, cnt);
  return takem;
}

// Exact Top-K of one candidate per thread (entry order = thread order), by
// ranks instead of a radix select: a candidate's 64-bit key is its order key
// above the complement of its thread index, so all keys differ and, of two
// candidates, the one with the larger key is kept first (larger score, the
// earlier one on ties).  Each wave sorts its 64 keys in descending order
// (a bitonic network over lane shuffles, no LDS), the sorted runs go to LDS
// (runs[NT]), and a candidate is kept when fewer than k keys of all runs
// exceed its own (a binary search per run, the runs searched side by side).
// Invalid candidates take key 0, below every valid key.  One workgroup
// barrier; requires NT threads, a multiple of the wave size.
template <int NT>
__device__ inline bool rank_keep(float s, bool valid, int k, uint64_t *runs) {
  constexpr int NR = NT / kWave;
  const int lane = threadIdx.x % kWave;
  const uint64_t key =
      valid ? ((uint64_t)order_key(s) << 32) | (uint64_t)(~(uint32_t)threadIdx.x) : 0ull;
  uint64_t x = key;
#pragma unroll
  for (int kk = 2; kk <= kWave; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const uint64_t o = __shfl_xor(x, j);
      // pairs in a descending block keep the larger key in the lower lane
      const bool keep_max = ((lane & j) == 0) == ((lane & kk) == 0);
      x = keep_max ? (x > o ? x : o) : (x < o ? x : o);
    }
  }
  runs[threadIdx.x] = x;
  __syncthreads();
  // keys above this one in each run: 6 halving steps, then the last entry
  int pos[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) pos[r] = 0;
#pragma unroll
  for (int b = kWave / 2; b >= 1; b >>= 1) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (runs[kWave * r + pos[r] + b - 1] > key) pos[r] += b;
  }
  int rank = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) rank += pos[r] + (runs[kWave * r + kWave - 1] > key ? 1 : 0);
  return valid && rank < k;
}

}  // namespace sas

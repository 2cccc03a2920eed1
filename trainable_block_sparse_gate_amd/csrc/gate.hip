// Gate + hard Top-K (forward) and the gate backward, one workgroup per row.
//
// Forward (review, sections 1-2, 2-1 and 3-3; paper text, section 4): per
// row with current block i,
//   lse      = log sum_{j in N} exp(s_j),  N = {j < i} (or {j <= i})
//   log g_j  = s_j - lse,  the current block keeps log g = 0 in the first mode
//   kept     = the min(Kb-1, i) largest s_j over j < i, lower j on ties.
// The activation ablations (paper text section 4; review 3-3) replace the
// normalised log gate of the kept history blocks by log sigmoid(s_j)
// (mode 2) or s_j itself (mode 3); they have no normaliser.  The
// ranking-preservation ablation (mode 4, straight-through) keeps the
// history normaliser but gives every kept block the hard gate 1 (log 0).
// The Top-K threshold is found with an exact radix select over 32-bit
// order-preserving keys of the fp32 scores (4 passes of 8 bits, LDS
// histograms); the kept blocks are then emitted in index order with a
// workgroup-wide ballot scan, so the result is unique and deterministic.
//
// Backward (review section 2-1; paper text, ablation results, where the
// normaliser is shared by every history block):
//   d s_m = [m kept] dlg_m - exp(s_m - lse) * sum over kept j of dlg_j;
// with independent gates d s_m = [m kept] dlg_m * (d log g_m / d s_m);
// straight-through (mode 4): dL/dg_j = dlg_j (the hard gate is 1) passed
// through the soft gate's Jacobian: d s_m = g_m ([m kept] dlg_m - sum over
// kept j of g_j dlg_j), g = exp(s - lse).
// Pages cited by title: "review" is the page "SAS: Simple Attention
// Sparsification via End-to-End Optimization of Context Ranking Review";
// "paper text" is the page "SAS: Simple Attention Sparsification via
// End-to-End Optimization of Context Ranking" that holds the paper's text.

constexpr int kGateSigmoid = 2, kGateRaw = 3, kGateSte = 4;  // the ablations
#include "sas_device.h"
#include "sas_launch.h"
#include "select.h"

namespace sas {

constexpr int kGateThreads = 256;
constexpr int kGateWaves = kGateThreads / kWave;

__device__ inline void row_geometry(const GateParams &p, int r, int &i) {
  const int Q = r % p.QB;
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, Q);
  i = Q - p.cu_qblocks[s];
}

// R > 0: the row's scores (at most NT * R) are read once into registers,
// thread t holding the R consecutive entries R t .. R t + R - 1;
// every pass below then works on registers instead of re-reading the row
// (long sequences have thousands of candidate blocks), and the kept blocks are
// placed with two workgroup scans in all (entries are in index order across
// the threads).  R = 0 reads the row in each pass and places the kept
// blocks chunk by chunk.
template <int R, int NT>
__global__ __launch_bounds__(NT) void gate_topk_kernel(GateParams p) {
  constexpr int NWV = NT / kWave;
  __shared__ float red[NWV];
  __shared__ int cnt[NWV];
  __shared__ SelectScratch sel;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int i;
  row_geometry(p, r, i);
  const float *srow = p.scores + (long)r * p.ld;
  const bool independent = p.mode == kGateSigmoid || p.mode == kGateRaw;
  const int nn = (p.mode == 1) ? i + 1 : i;
  const int k = min(p.Kb - 1, i);

  float sv[R > 0 ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = R * tid + c;
      sv[c] = j < nn ? srow[j] : -INFINITY;
    }
  }
  // f(j, s_j) for this thread's entries j < lim, in ascending order
  auto each = [&](int lim, auto &&f) {
    if constexpr (R > 0) {
#pragma unroll
      for (int c = 0; c < R; ++c) {
        const int j = R * tid + c;
        if (j < lim) f(j, sv[c]);
      }
    } else {
      for (int j = tid; j < lim; j += NT) f(j, srow[j]);
    }
  };

  // Normaliser (independent gates have none; the uniform test skips it).
  float lse = 0.f;
  if (!independent) {
    float mx = -INFINITY;
    each(nn, [&](int, float x) { mx = fmaxf(mx, x); });
    mx = block_max<NWV>(mx, red);
    float sum = 0.f;
    if (mx != -INFINITY) each(nn, [&](int, float x) { sum += expf(x - mx); });
    sum = block_sum<NWV>(sum, red);
    lse = (nn == 0 || mx == -INFINITY) ? -INFINITY : mx + logf(sum);
  }

  // Exact k-th largest key (radix select), unless every candidate is kept.
  const bool keep_all = (k == i);
  Threshold th{0u, 0u, k};
  if (!keep_all && k > 0)
    th = radix_threshold<NT>(k, sel, [&](auto &&f) {
      each(i, [&](int, float x) { f(order_key(x)); });
    });
  const uint32_t prefix = th.prefix, pmask = th.pmask;
  const int remaining = th.remaining;

  // Emit kept blocks in index order: keys above the threshold, plus the
  // first `remaining` keys equal to it.
  int32_t *oidx = p.sel_idx + (long)r * p.Kb;
  float *olg = p.sel_lg + (long)r * p.Kb;
  auto gate_of = [&](float sj) -> float {
    if (p.mode == kGateSigmoid)  // log sigmoid(s) = min(s, 0) - log(1 + exp(-|s|))
      return fminf(sj, 0.f) - log1pf(expf(-fabsf(sj)));
    if (p.mode == kGateRaw) return sj;
    if (p.mode == kGateSte) return 0.f;  // hard gate
    return (lse == -INFINITY) ? -INFINITY : sj - lse;
  };
  int base = 0, eq_base = 0;
  auto emit = [&](int j, float sj) {  // j: this thread's entry of the chunk
    const bool valid = j < i;
    const uint32_t key = order_key(valid ? sj : 0.f) & pmask;
    const bool eq = valid && !keep_all && key == prefix;
    int eq_tot;
    const int eq_rank = eq_base + block_scan_flag<NWV>(eq, eq_tot, cnt);
    const bool take = valid && (keep_all || key > prefix || (eq && eq_rank < remaining));
    int take_tot;
    const int pos = base + block_scan_flag<NWV>(take, take_tot, cnt);
    if (take) {
      oidx[pos] = j;
      olg[pos] = gate_of(sj);
    }
    base += take_tot;
    eq_base += eq_tot;
  };
  if (k > 0) {
    if constexpr (R > 0) {
      // this thread's kept entries (the first `remaining` keys equal to the
      // threshold in index order are kept), placed by two workgroup scans
      uint32_t valid = 0u;
#pragma unroll
      for (int c = 0; c < R; ++c)
        if (R * tid + c < i) valid |= 1u << c;
      int pos, take_tot;
      const uint32_t takem = kept_mask<R, NWV>(sv, valid, keep_all, th, cnt, pos, take_tot);
#pragma unroll
      for (int c = 0; c < R; ++c)
        if ((takem >> c) & 1u) {
          oidx[pos] = R * tid + c;
          olg[pos] = gate_of(sv[c]);
          ++pos;
        }
    } else {
      for (int c0 = 0; c0 < i; c0 += NT) {
        const int j = c0 + tid;
        emit(j, j < i ? srow[j] : 0.f);
      }
    }
  }
  if (tid == 0) {
    oidx[k] = i;
    olg[k] = (p.mode == 1) ? ((lse == -INFINITY) ? -INFINITY : srow[i] - lse) : 0.f;
    p.gate_lse[r] = lse;
  }
  for (int x = k + 1 + tid; x < p.Kb; x += NT) {
    oidx[x] = -1;
    olg[x] = -INFINITY;
  }
}

hipError_t launch_gate_topk(const GateParams &p, hipStream_t stream) {
  if (p.nrows == 0) return hipSuccess;
  // rows hold at most ld scores (one more than the history in SAS_GATE_ALL
  // is still within ld): registers when they fit, else re-reads
  // (long rows take 1024 threads: 4x the threads on each pass of the few
  // rows a long sequence has)
  const dim3 grid(p.nrows);
  if (p.ld <= 256) hipLaunchKernelGGL((gate_topk_kernel<1, 256>), grid, dim3(256), 0, stream, p);
  else if (p.ld <= 1024)
    hipLaunchKernelGGL((gate_topk_kernel<4, 256>), grid, dim3(256), 0, stream, p);
  else if (p.ld <= 4096)
    hipLaunchKernelGGL((gate_topk_kernel<4, 1024>), grid, dim3(1024), 0, stream, p);
  else if (p.ld <= 8192)
    hipLaunchKernelGGL((gate_topk_kernel<8, 1024>), grid, dim3(1024), 0, stream, p);
  else if (p.ld <= 16384)
    hipLaunchKernelGGL((gate_topk_kernel<16, 1024>), grid, dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL((gate_topk_kernel<0, 256>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(kGateThreads) void gate_bwd_kernel(GateBwdParams p) {
  __shared__ int s_j[kMaxBudget];
  __shared__ float s_d[kMaxBudget];
  __shared__ int s_n;
  __shared__ float s_tot;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int Q = r % p.QB;
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, Q);
  const int i = Q - p.cu_qblocks[s];
  const bool independent = p.mode == kGateSigmoid || p.mode == kGateRaw;
  const int nn = (p.mode == 1) ? i + 1 : i;
  const float lse = independent ? 0.f : p.gate_lse[r];
  const int32_t *sel = p.sel_idx + (long)r * p.Kb;
  const float *dlg = p.dlg + (long)r * p.Kb;
  if (tid == 0) {
    // kept entries that carry a gradient, ascending by block index
    int n = 0;
    float tot = 0.f;
    for (int sl = 0; sl < p.Kb; ++sl) {
      const int j = sel[sl];
      if (j < 0 || j > i || (j == i && p.mode != 1)) continue;
      s_j[n] = j;
      // straight-through: the kept gradient enters weighted by the soft gate
      const float d = p.mode == kGateSte ? expf(p.logits[(long)r * p.ld + j] - lse) * dlg[sl]
                                         : dlg[sl];
      s_d[n] = d;
      tot += d;
      ++n;
    }
    s_n = n;
    s_tot = tot;
  }
  __syncthreads();
  const int n = s_n;
  const float tot = s_tot;
  const float *srow = p.logits + (long)r * p.ld;
  float *out = p.dlogits + (long)r * p.ld;
  for (long c = tid; c < p.ld; c += kGateThreads) {
    float val = 0.f;
    if (independent) {
      // kept history blocks only; d log sigmoid(s) / ds = sigmoid(-s)
      if (c < i) {
        int lo = 0, hi = n - 1;
        while (lo <= hi) {
          const int mid = (lo + hi) >> 1;
          if (s_j[mid] == c) {
            val = p.mode == kGateRaw ? s_d[mid] : s_d[mid] / (1.f + expf(srow[c]));
            break;
          }
          if (s_j[mid] < c) lo = mid + 1; else hi = mid - 1;
        }
      }
    } else if (c < nn && lse != -INFINITY) {
      // (straight-through: s_d and tot already carry the soft gates)
      val = -expf(srow[c] - lse) * tot;
      int lo = 0, hi = n - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        if (s_j[mid] == c) {
          val += s_d[mid];
          break;
        }
        if (s_j[mid] < c) lo = mid + 1; else hi = mid - 1;
      }
    }
    out[c] = val;
  }
}

hipError_t launch_gate_bwd(const GateBwdParams &p, hipStream_t stream) {
  if (p.nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_bwd_kernel, dim3(p.nrows), dim3(kGateThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sas

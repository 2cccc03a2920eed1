// Gated block-sparse attention forward for gfx950.
//
// What it computes (review, section 2-2, and the fused-kernel description
// in section 3-6): for each query token t of block
// i and head h, o_t = softmax_u(scale * q_t.k_u + log g(blk(u))) v_u over the
// keys of the kept history blocks and the keys u <= t of block i, plus the
// row log-sum-exp.  The gate is added to every logit of its block inside
// the tile, and the attention matrix is never materialised.
//
// Design (MI355X):
//   - one workgroup per (query block, kv head): its waves are the G query
//     heads that share the kv head (GQA), 64 query rows each, so every K/V
//     tile staged in LDS feeds G*64 rows;
//   - K/V tiles are gathered by kept-block index into double-buffered LDS,
//     row-major with padded rows; the product that contracts over keys reads
//     V transposed with ds_read_b64_tr_b16;
//   - S^T = K Q^T on 32x32 MFMA tiles with Q held in registers, so each
//     lane owns one query column and the softmax row statistics need a
//     single cross-half exchange; the key order inside each tile is chosen
//     so that the probabilities chain straight into O^T += V^T P^T;
//   - fp32 online softmax in the log2 domain; the log gate of the tile is one
//     scalar; the current (diagonal) block goes first so the running max is
//     finite before any gated history tile; the output is rescaled only when
//     a tile's max jumps well above the running reference;
//   - two tiles ahead are in flight: one in LDS, one in registers.
// Pages cited by title: "review" is the page "SAS: Simple Attention
// Sparsification via End-to-End Optimization of Context Ranking Review";
// "paper text" is the page "SAS: Simple Attention Sparsification via
// End-to-End Optimization of Context Ranking" that holds the paper's text.
#include "sas_device.h"
#include "sas_launch.h"
#include "tile_stage.h"

namespace sas {

// Lazy rescaling: the running reference max of a query row moves only when
// a tile's max exceeds it by more than this (log2 units), so most tiles skip
// the O *= alpha pass; probabilities stay <= 2^kRescale, exact in fp32 sums
// and well inside bf16 range.
constexpr float kRescale = 8.f;

// Query tiles (of 32 rows) per wave: 1 = two waves per head, 32 query rows
// each, which keeps a wave within 256 registers so two waves share a SIMD
// (one's softmax overlaps the other's MFMAs).
constexpr int kFwdQT = 1;

// OUTER: the gate-position ablation (review 3-2; paper text section 4):
// the softmax runs over the ungated logits and each tile's probabilities
// are scaled by the tile's gate only where they weight the values.
template <typename T, typename TO, int D, int NW, bool OUTER>
__global__ __launch_bounds__(NW * (2 / kFwdQT) * 64) void fwd_kernel(FwdParams p) {
  using M = Mfma<T>;
  constexpr int QT = kFwdQT;           // 32-query tiles per wave
  constexpr int WPH = 2 / QT;          // waves per head
  constexpr int NT = NW * WPH * kWave;
  using RT = RowTile<T, D, NT>;
  constexpr int KS = M::K, E = M::E;
  constexpr int NKS = D / KS;          // k-steps over head_dim
  constexpr int NDT = D / 32;          // 32-row d tiles of O^T
  constexpr int NKC = kBlock / KS;     // k-steps over a 64-key tile
  constexpr int SPT = 32 / KS;         // k-steps per 32-key half tile
  constexpr int TILE = RT::ELEMS;

  __shared__ __attribute__((aligned(16))) T tiles[2 * 2 * TILE];  // [buf][K | V]
  __shared__ int s_j[kMaxBudget];
  __shared__ float s_lg[kMaxBudget];
  __shared__ int s_n;

  const T *q = static_cast<const T *>(p.q);
  const T *kk = static_cast<const T *>(p.k);
  const T *vv = static_cast<const T *>(p.v);

  const int Q = blockIdx.x;
  const int nhc = (p.G + NW - 1) / NW;
  const int g = blockIdx.y / nhc, hc = blockIdx.y % nhc;
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int hf = lane / 32, l32 = lane % 32;
  const int hh = hc * NW + wave / WPH;
  const int nt0 = (wave % WPH) * QT;  // this wave's first 32-query tile
  const bool head_ok = hh < p.G;
  const int h = g * p.G + (head_ok ? hh : 0);

  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, Q);
  const int i = Q - p.cu_qblocks[s];
  const int seq_start = p.cu_seqlens[s];
  const int seq_len = p.cu_seqlens[s + 1] - seq_start;
  const int nq = min(kBlock, seq_len - i * kBlock);
  const long row = (long)g * p.QB + Q;

  // tile order: the current (diagonal) block first, so the running max is
  // finite before any gated history tile, then the kept history blocks
  // (built by wave 0, all slots read at once)
  if (wave == 0) {
    const int n = wave_kept_blocks(p.sel_idx + row * p.Kb, p.sel_lg + row * p.Kb, p.Kb, i, true,
                                   s_j, nullptr, s_lg);
    if (lane == 0) s_n = n;
  }

  // Q as the B operand of S^T = K Q^T: lane -> query column.
  typename M::Op qreg[QT][NKS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    // rows past the block's end read its last row (their outputs are never
    // written), so the loads need no branch and issue back to back
    const int ql = min(32 * (nt0 + t) + l32, nq - 1);
    const T *qp = q + ((long)(seq_start + i * kBlock + ql) * p.hq + h) * D + hf * E;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[t][ks] = lds_op<T>(qp + ks * KS);
  }

  f32x16 oacc[NDT][QT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int t = 0; t < QT; ++t) oacc[dt][t] = f32x16{};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }

  // the tile list is visible; Q may still be in flight, so its latency
  // overlaps the first tile's (storing that tile waits for both)
  barrier_keep_requests();
  const int ntiles = s_n;
  const int kstride = p.hkv * D;
  RT kst, vst;
  auto load_tile = [&](int it) {
    const int j = __builtin_amdgcn_readfirstlane(s_j[it]);
    const long tok = seq_start + (long)j * kBlock;
    const int nv = min(kBlock, seq_len - j * kBlock);
    rowtile_load<T, T, D, NT>(kst, kk + (tok * p.hkv + g) * D, kstride, nv);
    rowtile_load<T, T, D, NT>(vst, vv + (tok * p.hkv + g) * D, kstride, nv);
  };
  auto store_tile = [&](int b) {
    rowtile_store<T, D, NT>(kst, tiles + (2 * b + 0) * TILE);
    rowtile_store<T, D, NT>(vst, tiles + (2 * b + 1) * TILE);
  };
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
    if (ntiles > 1) load_tile(1);
  }
  __syncthreads();

  // Per tile: compute from one buffer, then store the next tile into the
  // other, issue the loads of the one after, and barrier (no LDS write of a
  // wave in flight while its transposed reads issue).
  for (int it = 0; it < ntiles; ++it) {
    const int b = it & 1;
    const float lg2 = s_lg[it];
    const bool diag = (s_j[it] == i);
    const T *Ks = tiles + (2 * b + 0) * TILE;
    const T *Vs = tiles + (2 * b + 1) * TILE;

    // S^T[key][query] for two 32-key halves x this wave's 32-query tiles.
    f32x16 sacc[2][QT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int krow = 32 * mt + chain_key_of_row<T>(l32);
#pragma unroll
      for (int t = 0; t < QT; ++t) sacc[mt][t] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename M::Op a = tile_op<T, D>(Ks, krow, hf * E + ks * KS);
#pragma unroll
        for (int t = 0; t < QT; ++t) sacc[mt][t] = M::run(a, qreg[t][ks], sacc[mt][t]);
      }
    }
    if constexpr (E == 8) {
      // K reads run ahead of the products that use them
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 2 * NKS * QT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first d tile's V operands are requested before the softmax, whose
    // arithmetic then covers their latency
    typename M::Op vop[2][NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) vop[0][kc] = tile_op_rows<T, D>(Vs, kc * KS, 0);
    if constexpr (E == 8) __builtin_amdgcn_sched_barrier(0);

    // Online softmax per query column (log2 domain, gate folded in).  The
    // max is taken over the raw scores (the scale is positive and the gate
    // term is the same for the whole tile); the causal mask is only
    // evaluated on the diagonal tile; the row sum is a pairwise tree.
    typename M::Op pop[QT][NKC];  // probabilities as B operands of O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int ql = 32 * (nt0 + t) + l32;
      if (diag) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mt + chain_slot<T>(r, hf) > ql) sacc[mt][t][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float lz = OUTER ? 0.f : lg2;  // the gate's term in the logits
      const float zmax = mx * p.scale_log2 + lz;
      // move the reference only on a large increase (first tile: from -inf)
      const bool move = zmax > m_run[t] + kRescale;
      const float m_new = move ? zmax : m_run[t];
      const float alpha = move ? fast_exp2(m_run[t] - m_new) : 1.f;
      // a tile whose gate is zero adds nothing (and no 0 * inf)
      const float c = lz == -INFINITY ? -INFINITY : lz - m_new;
      float ps[16];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(sacc[mt][t][r], p.scale_log2, c));
          sacc[mt][t][r] = pr;
          ps[r] = mt == 0 ? pr : ps[r] + pr;
        }
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int r = 0; r < w; ++r) ps[r] += ps[r + w];
      float sum = ps[0];
      sum += __shfl_xor(sum, 32);
      l_run[t] = l_run[t] * alpha + sum;
      m_run[t] = m_new;
      if (__builtin_amdgcn_read_exec() & __ballot(move)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][t][r] *= alpha;
      }
      if constexpr (OUTER) {
        // the values see the gated probabilities, the row sum the ungated
        const float gate = fast_exp2(lg2);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[mt][t][r] *= gate;
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) pop[t][kc] = regs_op<T>(sacc[kc / SPT][t], (kc % SPT) * E);
    }

    // O^T[d][query] += V^T[d][key] P^T[key][query], V read transposed (the
    // operands of the next d tile are requested a tile ahead)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt + 1 < NDT) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          vop[(dt + 1) & 1][kc] = tile_op_rows<T, D>(Vs, kc * KS, 32 * (dt + 1));
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
        for (int t = 0; t < QT; ++t) oacc[dt][t] = M::run(vop[dt & 1][kc], pop[t][kc], oacc[dt][t]);
      }
    }
    if constexpr (E == 8) {
#pragma unroll
      for (int k = 0; k < NDT * NKC * QT - NKC * QT; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NKC * QT, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (it + 1 < ntiles) store_tile(b ^ 1);
    if (it + 2 < ntiles) load_tile(it + 2);
    __syncthreads();
  }

  if (!head_ok) return;
  TO *o = static_cast<TO *>(p.o);
  if constexpr (sizeof(TO) == 2 && sizeof(T) == 2) {
    // bf16 output goes through the (now idle) tile buffers: each wave puts
    // its 32 QT rows into a private swizzled region, then stores whole
    // 16-byte chunks, 16 lanes per row, so every row is written in full
    // lines rather than in 8-byte pieces spread over many instructions.
    using SW = Swz<__bf16, D>;
    constexpr int ROWS = 32 * QT, CPR = D / 8;
    static_assert((NT / kWave) * ROWS * D <= 2 * 2 * TILE, "all waves' rows fit the tiles");
    __bf16 *ob = reinterpret_cast<__bf16 *>(tiles) + wave * (ROWS * D);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const float inv = 1.f / l_run[t];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = 32 * dt + d_row(4 * rg, hf);
          bf16x4 w;
#pragma unroll
          for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[dt][t][4 * rg + x] * inv);
          *reinterpret_cast<bf16x4 *>(ob + SW::off(32 * t + l32, d0)) = w;
        }
      const int ql = 32 * (nt0 + t) + l32;
      if (hf == 0 && ql < nq) {
        const long tq = seq_start + i * kBlock + ql;
        p.lse[(long)h * p.T + tq] = (m_run[t] + fast_log2(l_run[t])) * kLn2;
      }
    }
    wait_lds_all();
#pragma unroll
    for (int c0 = 0; c0 < ROWS * CPR; c0 += kWave) {
      const int c = c0 + lane, r = c / CPR, cc = c % CPR;
      const int ql = 32 * nt0 + r;
      if (ql < nq) {
        const long tq = seq_start + i * kBlock + ql;
        *reinterpret_cast<u32x4 *>(o + (tq * p.hq + h) * D + 8 * cc) =
            *reinterpret_cast<const u32x4 *>(ob + SW::off(r, 8 * cc));
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int ql = 32 * (nt0 + t) + l32;
    if (ql >= nq) continue;
    const long tq = seq_start + i * kBlock + ql;
    const float inv = 1.f / l_run[t];
    TO *op = o + (tq * p.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * dt + d_row(4 * rg, hf);
        if constexpr (sizeof(TO) == 2) {
          bf16x4 w;
#pragma unroll
          for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[dt][t][4 * rg + x] * inv);
          *reinterpret_cast<bf16x4 *>(op + d0) = w;
        } else {
          float4 w = make_float4(oacc[dt][t][4 * rg] * inv, oacc[dt][t][4 * rg + 1] * inv,
                                 oacc[dt][t][4 * rg + 2] * inv, oacc[dt][t][4 * rg + 3] * inv);
          *reinterpret_cast<float4 *>(op + d0) = w;
        }
      }
    if (hf == 0) p.lse[(long)h * p.T + tq] = (m_run[t] + fast_log2(l_run[t])) * kLn2;
  }
}

template <typename T, typename TO, int D, int NW>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  dim3 grid(p.QB, p.hkv * ((p.G + NW - 1) / NW));
  if (p.outer)
    hipLaunchKernelGGL((fwd_kernel<T, TO, D, NW, true>), grid, dim3(NW * (2 / kFwdQT) * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, TO, D, NW, false>), grid, dim3(NW * (2 / kFwdQT) * 64), 0,
                       stream, p);
  return hipGetLastError();
}

template <typename T, typename TO, int D>
static hipError_t launch_fwd_d(const FwdParams &p, hipStream_t stream) {
  if (p.G >= 4) return launch_fwd_t<T, TO, D, 4>(p, stream);
  if (p.G == 2 || p.G == 3) return launch_fwd_t<T, TO, D, 2>(p, stream);
  return launch_fwd_t<T, TO, D, 1>(p, stream);
}

hipError_t launch_fwd(const FwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                      hipStream_t stream) {
  if (dtype_bf16) {
    if (out_bf16)
      return head_dim == 128 ? launch_fwd_d<__bf16, __bf16, 128>(p, stream)
                             : launch_fwd_d<__bf16, __bf16, 64>(p, stream);
    return head_dim == 128 ? launch_fwd_d<__bf16, float, 128>(p, stream)
                           : launch_fwd_d<__bf16, float, 64>(p, stream);
  }
  return head_dim == 128 ? launch_fwd_d<float, float, 128>(p, stream)
                         : launch_fwd_d<float, float, 64>(p, stream);
}

}  // namespace sas

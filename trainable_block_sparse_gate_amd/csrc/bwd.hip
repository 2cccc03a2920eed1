// Gated block-sparse attention backward for gfx950.
//
// Gradients of o_t = sum_u P_tu v_u, P_t = softmax_u(scale q_t.k_u + log g),
// which the pages say the fused kernel keeps through to the selector
// (review, section 3-6; paper text, ablation results: the inner gate's
// gradient carries P_gated (dP - D)):
//   D_t   = sum_e dO_te o_te            dP_tu = dO_t . v_u
//   dS_tu = P_tu (dP_tu - D_t)          dq_t  = scale sum_u dS_tu k_u
//   dk_u  = scale sum_t dS_tu q_t       dv_u  = sum_t P_tu dO_t
//   dlg[row][slot] = sum over the row's tokens, its G heads and the slot's
//                    keys of dS_tu       (the per-block log-gate gradient)
//
// Work split (all deterministic, no atomics on results):
//   1. csr:    for every (kv head, key block), the (query block, slot) pairs
//              that keep it, in query-block order (one wave per key block).
//   2. scan:   segments of at most `seg` pairs per key block, prefix-summed.
//   3. dq:     one workgroup per (query block, kv head) -- the forward's
//              geometry; recomputes P from the saved lse, forms dS, and
//              produces dq and the per-tile sums of dS (dlg).  D is first
//              taken from the stored o (rounded to the output dtype) for dq;
//              the exact D_t = sum_u P_tu dP_tu is accumulated over the tiles
//              and used for dlg and, through the workspace, for dk.  dlg of a
//              tile is sum P dP - sum_t D_t (sum over the tile of P_tu), so
//              the rounding of o never enters the selector gradient.
//   4. dkdv:   (bwd_dkdv.hip) one workgroup per segment of a key block:
//              K and V stay in registers, Q/dO tiles of the keeping rows
//              stream through LDS, dK^T and dV^T accumulate in registers;
//              the partials of split key blocks are summed in segment order
//              by a second, small kernel.
// Pages cited by title: "review" is the page "SAS: Simple Attention
// Sparsification via End-to-End Optimization of Context Ranking Review";
// "paper text" is the page "SAS: Simple Attention Sparsification via
// End-to-End Optimization of Context Ranking" that holds the paper's text.
#include "sas_device.h"
#include "sas_launch.h"
#include "tile_stage.h"

namespace sas {

// ------------------------------------------------------------------ csr
// One wave per x = kb * hkv + g (key-block major: the segments of early key
// blocks, which the most rows keep, come first in the dk/dv grid, so the
// longest workgroups start first and the short ones fill the tail).  Rows
// that can keep key block j of sequence s are its query blocks i >= j.
__global__ __launch_bounds__(256) void bwd_csr_kernel(BwdParams p) {
  // waves walk the key blocks head by head (neighbouring waves read the same
  // selection rows); results are stored at the key-block-major index x
  const int wv = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (wv >= p.hkv * p.QB) return;
  const int g = wv / p.QB, kb = wv % p.QB;
  const int x = kb * p.hkv + g;
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, kb);
  const int q0 = p.cu_qblocks[s], nb = p.cu_qblocks[s + 1] - q0;
  const int j = kb - q0;
  int32_t *out = p.list + (long)x * p.max_nb;
  int n = 0;
  for (int i0 = j; i0 < nb; i0 += kWave) {
    const int i = i0 + lane;
    int slot = -1;
    if (i < nb) {
      // a block appears at most once in a row's kept list; the slots are
      // read with no early exit, so their loads issue back to back
      const int32_t *sel = p.sel_idx + ((long)g * p.QB + q0 + i) * p.Kb;
#pragma unroll 16
      for (int sl = 0; sl < p.Kb; ++sl) slot = sel[sl] == j ? sl : slot;
    }
    const uint64_t m = __ballot(slot >= 0);
    if (slot >= 0) {
      const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
      out[pos] = ((q0 + i) << 8) | slot;
    }
    n += __popcll(m);
  }
  if (lane == 0) p.count[x] = n;
}

// ------------------------------------------------------------------ scan
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void bwd_seg_scan_kernel(BwdParams p) {
  __shared__ int part[kScanThreads];
  const int n = p.hkv * p.QB;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int b0 = threadIdx.x * per, b1 = min(n, b0 + per);
  // every key block gets at least one segment (a block no row keeps then
  // simply writes zeros)
  int local = 0;
  for (int x = b0; x < b1; ++x) {
    local += max(1, (p.count[x] + p.seg - 1) / p.seg);
  }
  part[threadIdx.x] = local;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int y = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += y;
    __syncthreads();
  }
  int run = part[threadIdx.x] - local;  // exclusive
  for (int x = b0; x < b1; ++x) {
    p.seg_off[x] = run;
    run += max(1, (p.count[x] + p.seg - 1) / p.seg);
  }
  if (threadIdx.x == kScanThreads - 1) p.seg_off[n] = part[kScanThreads - 1];
}

// ------------------------------------------------------------------ dq
// The forward's geometry: WPH waves per query head of one kv head, QT 32-row
// query tiles per wave, Q and dO held in registers as B operands.  K and V
// tiles of the kept blocks go straight from global memory into two LDS
// arrays (row-major, swizzled); dQ^T = K^T dS^T reads K transposed with
// ds_read_b64_tr_b16.  The tile loop alternates MFMA and VALU steps with a
// workgroup barrier after each (see the loop).  Transposed reads issued
// while LDS stores of the same wave are in flight have returned wrong data
// on gfx950: this wave's LDS stores in the loop (the row sums of a VALU
// step) complete at that step's barrier, before the next MFMA step issues
// any transposed read.  The global-to-LDS requests into the other tile
// array may be in flight during an MFMA step, as in the dK/dV kernel; the
// full-size parity tests cover that overlap.
constexpr int kDqQT = 1;  // 32-query tiles per wave (1: two waves per head)
// floats per (wave, tile) record of per-row sums: 32 QT rows and one of
// padding, so the lanes reading one row of consecutive tiles hit distinct
// LDS banks (an unpadded stride of 32 floats put every other lane on the
// same bank)
constexpr int kDqRec = 32 * kDqQT + 1;

// OUTER: the gate-position ablation.  P comes from the ungated logits,
// dP is scaled by the tile's gate, and the tile's d log g is the sum of
// P dP alone (P does not depend on the gate).
template <typename T, typename TO, int D, int NW, bool OUTER>
__global__ __launch_bounds__(NW * (2 / kDqQT) * 64) void bwd_dq_kernel(BwdParams p) {
  using M = Mfma<T>;
  constexpr int QT = kDqQT;
  constexpr int WPH = 2 / QT;  // waves per head
  constexpr int NWV = NW * WPH;
  constexpr int NT = NWV * kWave;
  using RT = RowTile<T, D, NT>;
  constexpr int KS = M::K, E = M::E;
  constexpr int NKS = D / KS, NDT = D / 32, SPT = 32 / KS;
  constexpr int TILE = RT::ELEMS;

  // K and V of the kept tiles, double buffered as two arrays ([K | V] each)
  // so that the compiler can tell a read of one from a request in flight
  // into the other
  __shared__ __attribute__((aligned(16))) T tiles0[2 * TILE];
  __shared__ __attribute__((aligned(16))) T tiles1[2 * TILE];
  __shared__ float s_F[NWV][kMaxBudget];  // per tile: the wave's share of dlg
  __shared__ int s_slot[kMaxBudget];     // tiles in processing order
  __shared__ int s_j[kMaxBudget];
  __shared__ float s_lg[kMaxBudget];     // log gate * log2(e)
  __shared__ int s_n;
  // [2][NWV][Kb][kDqRec]: per tile and query row, the sums over the tile's
  // keys of P (s_G) and of P dP (s_Fq)
  extern __shared__ float s_G[];
  float *s_Fq = s_G + NWV * p.Kb * kDqRec;

  const T *q = static_cast<const T *>(p.q);
  const T *kk = static_cast<const T *>(p.k);
  const T *vv = static_cast<const T *>(p.v);
  const TO *oo = static_cast<const TO *>(p.o);
  const TO *dO = static_cast<const TO *>(p.dO);

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

  // the kept blocks in slot order (wave 0, all slots read at once)
  if (wave == 0) {
    const int n = wave_kept_blocks(p.sel_idx + row * p.Kb, p.sel_lg + row * p.Kb, p.Kb, i, false,
                                   s_j, s_slot, s_lg);
    if (lane == 0) s_n = n;
  }

  // Q and dO as B operands (lane -> query column), D and lse per column.
  // Every load is issued before any is used, and the first K/V tile is
  // requested before the Q/dO/O data is consumed, so the prologue costs one
  // memory latency.
  typename M::Op qreg[QT][NKS], doreg[QT][NKS];
  float Dv[QT], lse2[QT];
  OutChunk<TO, E> dch[QT][NKS], och[QT][NKS];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int ql = 32 * (nt0 + nt) + l32;
    const long t = seq_start + (long)i * kBlock + ql;
    // rows past the block's end read its last row: their P is zero (lse
    // +inf), so neither their values nor their D reach any result, and the
    // loads need no branch and issue back to back
    const long base = ((t - max(0, ql - (nq - 1))) * p.hq + h) * D + hf * E;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qreg[nt][ks] = lds_op<T>(q + base + ks * KS);
      dch[nt][ks].load(dO + base + ks * KS);
      och[nt][ks].load(oo + base + ks * KS);
    }
    lse2[nt] = INFINITY;  // padding rows: P = 0
    if (ql < nq) lse2[nt] = p.lse[(long)h * p.T + t] * kLog2e;
  }
  float Eacc[QT];  // exact D: sum_u P dP (lane-partial)
  f32x16 dqacc[NDT][QT];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    Eacc[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqacc[dt][nt] = f32x16{};
  }

  barrier_keep_requests();  // the tile list is visible; the loads above may be in flight
  const int ntiles = s_n;
  // Tile u of the list goes straight from global memory into LDS
  // (global_load_lds, 16 bytes per lane, one request per 1 KB of rows),
  // each 16-byte chunk at its swizzled position; rows past the block's end
  // repeat its last row.  Each wave issues its share; completion is counted
  // by vmcnt.
  auto issue_tile = [&](T *buf, int u) {
    constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
    constexpr int RPI = kWave / CPR;              // rows per request
    constexpr int NREQ = kBlock / RPI;            // requests per K (or V) tile
    static_assert(NREQ % NWV == 0, "requests split evenly over the waves");
    const int j = __builtin_amdgcn_readfirstlane(s_j[u]);
    const long tok = seq_start + (long)j * kBlock;
    const int nv = min(kBlock, seq_len - j * kBlock);
    const char *kb = reinterpret_cast<const char *>(kk + (tok * p.hkv + g) * D);
    const char *vb = reinterpret_cast<const char *>(vv + (tok * p.hkv + g) * D);
    const unsigned rstride = (unsigned)(p.hkv * D * (int)sizeof(T));
#pragma unroll
    for (int q = 0; q < NREQ / NWV; ++q) {
      const int req = q * NWV + wave;
      const int row = req * RPI + lane / CPR;
      const int rr = row < nv ? row : nv - 1;
      const unsigned off =
          (unsigned)rr * rstride + (unsigned)(((lane % CPR) ^ Swz<T, D>::f(row)) * 16);
      load_lds16(kb + off, buf + req * RPI * D);
      load_lds16(vb + off, buf + TILE + req * RPI * D);
    }
  };
  if (ntiles > 0) issue_tile(tiles0, 0);

#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int ql = 32 * (nt0 + nt) + l32;
    const long base = ((seq_start + (long)i * kBlock + ql) * p.hq + h) * D + hf * E;
    float dacc = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int e = 0; e < E; ++e) dacc += dch[nt][ks].get(e) * och[nt][ks].get(e);
      doreg[nt][ks] = dch[nt][ks].template as_op<T>();
    }
    // a wider dO is handed to the dk/dv phase rounded to the input dtype
    if constexpr (sizeof(TO) != sizeof(T)) {
      if (ql < nq && head_ok) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          *reinterpret_cast<typename M::Op *>(p.dO16 + base + ks * KS) = doreg[nt][ks];
      }
    }
    dacc += __shfl_xor(dacc, 32);
    Dv[nt] = dacc;
  }

  // the first tile (and the Q / dO / O loads before it) has landed
  wait_vmem<0>();
  __syncthreads();

  // The tile loop as a sequence of steps, two per 32-key half h of the
  // kept tiles (h = 0 .. 2 ntiles - 1, tile h / 2, key half h % 2):
  //   step 2h      MFMA:  dQ^T += K^T dS^T of half h - 1, then S^T and
  //                       dP^T of half h;
  //   step 2h + 1  VALU:  P^T and dS^T of half h (the exponentials, the
  //                       row sums for d log g), kept as MFMA operands;
  // and a last MFMA step 4 ntiles for the dQ of the last half.  Every step
  // ends with a workgroup barrier.  The second half of the waves (`lag`)
  // passes one extra barrier before its first step and the first half one
  // after its last, so the lagging waves run each step one barrier interval
  // later: the two waves that share a SIMD are always in different kinds of
  // step, one keeping the matrix core busy while the other computes
  // exponentials.
  //
  // LDS buffers: tile u lives in tiles0 / tiles1 for u even / odd.  Its
  // last reader is step 4u + 4 (the dQ of its second half), which the
  // lagging waves run in interval 4u + 5; tile u + 2 is first read by the
  // leading waves' step 4u + 8.  So each wave requests its share of tile
  // u + 2 in interval 4u + 6 (leading: step 4u + 6; lagging: step 4u + 5)
  // and waits for it at the end of interval 4u + 7 (leading: step 4u + 7;
  // lagging: step 4u + 6), before that interval's barrier.  Two tiles per
  // loop iteration keep each step's buffers known at compile time, and no
  // request is in flight across an iteration's end.
  const int lag = wave >= NWV / 2 ? 1 : 0;
  f32x16 sacc[QT], pacc[QT];      // S^T, dP^T of the half in flight
  typename M::Op dsop[QT][SPT];    // dS^T of the previous half (B operands)
  float Fp[QT], Gp[QT];            // lane partials over a tile: sum P dP, sum P
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) Fp[nt] = Gp[nt] = 0.f;

  // dQ^T[d][query] += K^T[d][key] dS^T[key][query] over key half mt of the
  // tile in Kp.
  // bf16: per-lane base offsets of the operand reads; each step makes them
  // opaque, so that the slices' addresses (one XOR each) are formed where
  // they are used instead of being held in registers across the loop.
  unsigned ob_s = 0, ob_ta = 0, ob_tb = 0;
  if constexpr (sizeof(T) == 2) {
    ob_s = op_base_bytes<D>(chain_key_of_row<T>(l32), hf);
    rows_base_bytes<D>(ob_ta, ob_tb);
  }
  auto dq_half = [&](const T *Kp, int mt) {
    if constexpr (sizeof(T) == 2) {
      // every operand read first (they complete in order; each MFMA waits
      // for its own), then the products
      __asm__ volatile("" : "+v"(ob_ta), "+v"(ob_tb));
      bf16x8 ops[NDT][SPT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc)
          ops[dt][kc] = tile_op_rows_x<D>(Kp, ob_ta, ob_tb, 32 * mt + kc * KS, dt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc)
#pragma unroll
          for (int nt = 0; nt < QT; ++nt)
            dqacc[dt][nt] = M::run(ops[dt][kc], dsop[nt][kc], dqacc[dt][nt]);
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int kc = 0; kc < SPT; ++kc) {
          const typename M::Op a = tile_op_rows<T, D>(Kp, 32 * mt + kc * KS, 32 * dt);
#pragma unroll
          for (int nt = 0; nt < QT; ++nt) dqacc[dt][nt] = M::run(a, dsop[nt][kc], dqacc[dt][nt]);
        }
      }
    }
  };
  // S^T and dP^T of key half mt of the tile in Ks (K, then V).  bf16: the
  // K and V operands run LA slices ahead of the products.
  auto sdp_half = [&](const T *Ks, int mt) {
    const T *Vs = Ks + TILE;
    if constexpr (sizeof(T) == 2) {
      constexpr int LA = 3;
      __asm__ volatile("" : "+v"(ob_s));
      bf16x8 ka[LA + 1], va[LA + 1];
#pragma unroll
      for (int ks = 0; ks < LA; ++ks) {
        ka[ks] = tile_op_x<D>(Ks, ob_s, mt, ks);
        va[ks] = tile_op_x<D>(Vs, ob_s, mt, ks);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks + LA < NKS) {
          ka[(ks + LA) % (LA + 1)] = tile_op_x<D>(Ks, ob_s, mt, ks + LA);
          va[(ks + LA) % (LA + 1)] = tile_op_x<D>(Vs, ob_s, mt, ks + LA);
        }
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
          sacc[nt] = M::run(ka[ks % (LA + 1)], qreg[nt][ks], ks == 0 ? f32x16{} : sacc[nt]);
          pacc[nt] = M::run(va[ks % (LA + 1)], doreg[nt][ks], ks == 0 ? f32x16{} : pacc[nt]);
        }
      }
    } else {
      const int krow = 32 * mt + chain_key_of_row<T>(l32);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename M::Op a = tile_op<T, D>(Ks, krow, hf * E + ks * KS);
        const typename M::Op bb = tile_op<T, D>(Vs, krow, hf * E + ks * KS);
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
          sacc[nt] = M::run(a, qreg[nt][ks], ks == 0 ? f32x16{} : sacc[nt]);
          pacc[nt] = M::run(bb, doreg[nt][ks], ks == 0 ? f32x16{} : pacc[nt]);
        }
      }
    }
  };
  // dS^T = P^T (dP^T - D) of key half mt of tile it, P^T recomputed from
  // the saved lse, packed as the next MFMA step's operands as it is
  // produced; the sums of P dP and of P over the 16 values of a lane run in
  // two chains (even and odd registers), so no value outlives its own
  // register.  The causal mask is only evaluated on the diagonal tile.
  auto ds_half = [&](int it, int mt) {
    const float lg2 = s_lg[it];
    const bool diag = (s_j[it] == i);
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
      const int ql = 32 * (nt0 + nt) + l32;
      const float c = (OUTER ? 0.f : lg2) - lse2[nt];
      const float gate = OUTER ? fast_exp2(lg2) : 1.f;
      float f[2] = {0.f, 0.f}, gs[2] = {0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        float ds[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int r = kc * E + e;
          float pr = fast_exp2(fmaf(sacc[nt][r], p.scale_log2, c));
          if (diag && 32 * mt + chain_slot<T>(r, hf) > ql) pr = 0.f;
          const float pd = pr * (OUTER ? gate * pacc[nt][r] : pacc[nt][r]);
          ds[e] = fmaf(-pr, Dv[nt], pd);
          f[r & 1] += pd;
          gs[r & 1] += pr;
        }
        if constexpr (sizeof(T) == 2) {
          bf16x8 b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)ds[e];
          dsop[nt][kc] = b;
        } else {
          dsop[nt][kc] = ds[0];
        }
      }
      const float fl = f[0] + f[1];
      Fp[nt] += fl;
      Eacc[nt] += fl;
      if constexpr (!OUTER) Gp[nt] += gs[0] + gs[1];  // outer: no D term in d log g
    }
    if (mt == 1) {
      // per query row (the two lane halves added); the sums over rows wait
      // until after the loop
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) {
        const float fsum = Fp[nt] + __shfl_xor(Fp[nt], 32);
        const float gsum = Gp[nt] + __shfl_xor(Gp[nt], 32);
        if (hf == 0) {
          s_Fq[(wave * p.Kb + it) * kDqRec + 32 * nt + l32] = fsum;
          s_G[(wave * p.Kb + it) * kDqRec + 32 * nt + l32] = gsum;
        }
        Fp[nt] = Gp[nt] = 0.f;
      }
    }
  };
  // The four steps of tile u (in `cur`; tile u - 1 in `prev`, which then
  // receives tile u + 1).
  auto tile_steps = [&](T *cur, T *prev, int u) {
    const bool next = u + 1 < ntiles;
    // step 4u: dQ of tile u - 1's second half, S / dP of tile u's first
    __builtin_amdgcn_s_setprio(1);
    if (u > 0) dq_half(prev, 1);
    sdp_half(cur, 0);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
    // step 4u + 1
    ds_half(u, 0);
    if (lag && next) issue_tile(prev, u + 1);
    phase_barrier();
    // step 4u + 2
    __builtin_amdgcn_s_setprio(1);
    dq_half(cur, 0);
    sdp_half(cur, 1);
    __builtin_amdgcn_s_setprio(0);
    if (!lag && next) issue_tile(prev, u + 1);
    if (lag) wait_vmem<0>();
    phase_barrier();
    // step 4u + 3
    ds_half(u, 1);
    if (!lag) wait_vmem<0>();
    phase_barrier();
  };
  if (lag) phase_barrier();
  for (int u = 0; u < ntiles; u += 2) {
    tile_steps(tiles0, tiles1, u);
    if (u + 1 < ntiles) tile_steps(tiles1, tiles0, u + 1);
  }
  // step 4 ntiles: the dQ of the last half (nothing is in flight)
  if (ntiles > 0) dq_half((ntiles & 1) ? tiles0 : tiles1, 1);
  phase_barrier();
  if (!lag) phase_barrier();
  // Exact D per query row, then dlg of each tile = sum P dP - sum_t D_t G_t.
  // Both row statistics are stored for all 64 rows of the block (rows past
  // its end: lse +inf, D 0) so the dk/dv phase can fetch them as a whole,
  // in the form that phase seeds its products with: -lse / scale and -D,
  // for bf16 inputs as 16-byte records [hi, mid, lo, 0 x 5] of three bf16
  // parts that add up to the value (an MFMA A operand).
  float Ex[QT];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    Ex[nt] = Eacc[nt] + __shfl_xor(Eacc[nt], 32);
    const int ql = 32 * (nt0 + nt) + l32;
    if (hf == 0 && head_ok) {
      const long at = ((long)h * p.QB + Q) * kBlock + ql;
      const float Ln = -lse2[nt] / p.scale_log2, Dn = ql < nq ? -Ex[nt] : 0.f;
      if constexpr (sizeof(T) == 2) {
        reinterpret_cast<bf16x8 *>(p.Lbuf)[at] = split3_bf16(Ln);
        reinterpret_cast<bf16x8 *>(p.Dbuf)[at] = split3_bf16(Dn);
      } else {
        p.Lbuf[at] = Ln;
        p.Dbuf[at] = Dn;
      }
    }
  }
  // this wave's share of dlg per tile, one tile per lane, rows in order:
  // sum over the wave's rows of (sum P dP - D_t sum P); D_t of row q comes
  // from lane q (read across lanes, no memory)
  for (int t0 = 0; t0 < ntiles; t0 += kWave) {
    const int t = t0 + lane;
    float val = 0.f;
#pragma unroll
    for (int nt = 0; nt < QT; ++nt)
      for (int q = 0; q < 32; ++q) {
        const float e = lane_value(Ex[nt], q);
        if (t < ntiles) {
          const int at = (wave * p.Kb + t) * kDqRec + 32 * nt + q;
          val += s_Fq[at] - e * s_G[at];
        }
      }
    if (t < ntiles) s_F[wave][t] = head_ok ? val : 0.f;
  }

  // dQ goes out through the (now idle) tile buffers, one half of the
  // columns at a time: each wave puts its rows' half into a private
  // swizzled region, then stores whole 16-byte chunks, 16 lanes per half
  // row, so rows are written in full lines.
  if (head_ok) {
    using SW = Swz<float, D / 2>;
    constexpr int ROWS = 32 * QT, HC = D / 8;  // rows, 16-byte chunks per half row
    constexpr int WPA = (NWV + 1) / 2;  // waves per tile array
    static_assert(WPA * ROWS * (D / 2) * 4 <= 2 * TILE * (int)sizeof(T),
                  "the waves' half rows fit the tile arrays");
    float *ob = reinterpret_cast<float *>(wave < WPA ? tiles0 : tiles1) +
                (wave % WPA) * (ROWS * (D / 2));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int nt = 0; nt < QT; ++nt)
#pragma unroll
        for (int dt = half * NDT / 2; dt < (half + 1) * NDT / 2; ++dt)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int d0 = 32 * dt + d_row(4 * rg, hf) - half * (D / 2);
            *reinterpret_cast<float4 *>(ob + SW::off(32 * nt + l32, d0)) = make_float4(
                dqacc[dt][nt][4 * rg] * p.scale, dqacc[dt][nt][4 * rg + 1] * p.scale,
                dqacc[dt][nt][4 * rg + 2] * p.scale, dqacc[dt][nt][4 * rg + 3] * p.scale);
          }
      wait_lds_all();
#pragma unroll
      for (int c0 = 0; c0 < ROWS * HC; c0 += kWave) {
        const int c = c0 + lane, r = c / HC, cc = c % HC;
        const int ql = 32 * nt0 + r;
        if (ql < nq) {
          const long t = seq_start + (long)i * kBlock + ql;
          *reinterpret_cast<float4 *>(p.dq + (t * p.hq + h) * D + half * (D / 2) + 4 * cc) =
              *reinterpret_cast<const float4 *>(ob + SW::off(r, 4 * cc));
        }
      }
      wait_lds_all();  // the region is rewritten by the next half
    }
  }
  __syncthreads();
  // Per-slot log-gate gradient: heads of this workgroup summed in order.
  float *dst = nhc == 1 ? p.dlg + row * p.Kb : p.dlg_part + ((long)hc * p.hkv * p.QB + row) * p.Kb;
  for (int sl = threadIdx.x; sl < p.Kb; sl += NT) {
    float val = 0.f;
    for (int it = 0; it < ntiles; ++it)
      if (s_slot[it] == sl) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) val += s_F[w][it];
      }
    dst[sl] = val;
  }
}

__global__ void bwd_dlg_sum_kernel(BwdParams p, int nhc) {
  const long n = (long)p.hkv * p.QB * p.Kb;
  const long x = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= n) return;
  float v = 0.f;
  for (int hc = 0; hc < nhc; ++hc) v += p.dlg_part[hc * n + x];
  p.dlg[x] = v;
}


// ------------------------------------------------------------------ launch
constexpr int kLdsBytes = 160 * 1024;

template <typename T, int D, int NW>
constexpr int dq_static_lds() {
  return (int)sizeof(T) * 4 * kBlock * D + (NW * (2 / kDqQT) + 3) * kMaxBudget * 4 + 64;
}

template <typename T, int D, int NW>
static size_t dq_dynamic_lds(const BwdParams &p) {
  return 2 * sizeof(float) * NW * (2 / kDqQT) * p.Kb * kDqRec;  // s_G, s_Fq
}

template <typename T, typename TO, int D, int NW>
static hipError_t launch_dq_t(const BwdParams &p, hipStream_t stream) {
  const int nhc = (p.G + NW - 1) / NW;
  const size_t dyn = dq_dynamic_lds<T, D, NW>(p);
  if (p.outer)
    hipLaunchKernelGGL((bwd_dq_kernel<T, TO, D, NW, true>), dim3(p.QB, p.hkv * nhc),
                       dim3(NW * (2 / kDqQT) * 64), dyn, stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, TO, D, NW, false>), dim3(p.QB, p.hkv * nhc),
                       dim3(NW * (2 / kDqQT) * 64), dyn, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nhc == 1) return e;
  const long n = (long)p.hkv * p.QB * p.Kb;
  hipLaunchKernelGGL(bwd_dlg_sum_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, nhc);
  return hipGetLastError();
}

template <typename T, int D>
static bool dq_fits(const BwdParams &p) {
  if (p.G >= 4) return dq_static_lds<T, D, 4>() + dq_dynamic_lds<T, D, 4>(p) <= kLdsBytes;
  if (p.G >= 2) return dq_static_lds<T, D, 2>() + dq_dynamic_lds<T, D, 2>(p) <= kLdsBytes;
  return dq_static_lds<T, D, 1>() + dq_dynamic_lds<T, D, 1>(p) <= kLdsBytes;
}

hipError_t launch_bwd_prepare(const BwdParams &p, hipStream_t stream) {
  const int nx = p.hkv * p.QB;
  hipLaunchKernelGGL(bwd_csr_kernel, dim3((nx + 3) / 4), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_seg_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, typename TO, int D>
static hipError_t launch_dq_d(const BwdParams &p, hipStream_t stream) {
  if (!dq_fits<T, D>(p)) return hipErrorNotSupported;  // nothing launched
  if (p.G >= 4) return launch_dq_t<T, TO, D, 4>(p, stream);
  if (p.G >= 2) return launch_dq_t<T, TO, D, 2>(p, stream);
  return launch_dq_t<T, TO, D, 1>(p, stream);
}

hipError_t launch_bwd_dq(const BwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                         hipStream_t stream) {
  if (dtype_bf16) {
    if (out_bf16)
      return head_dim == 128 ? launch_dq_d<__bf16, __bf16, 128>(p, stream)
                             : launch_dq_d<__bf16, __bf16, 64>(p, stream);
    return head_dim == 128 ? launch_dq_d<__bf16, float, 128>(p, stream)
                           : launch_dq_d<__bf16, float, 64>(p, stream);
  }
  return head_dim == 128 ? launch_dq_d<float, float, 128>(p, stream)
                         : launch_dq_d<float, float, 64>(p, stream);
}

bool bwd_dq_supported(const BwdParams &p, int dtype_bf16, int head_dim) {
  if (dtype_bf16) return head_dim == 128 ? dq_fits<__bf16, 128>(p) : dq_fits<__bf16, 64>(p);
  return head_dim == 128 ? dq_fits<float, 128>(p) : dq_fits<float, 64>(p);
}


}  // namespace sas

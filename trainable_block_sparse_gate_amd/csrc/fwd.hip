// Gated block-sparse attention forward for gfx950.
//
// What it computes (dimensionstp.github.io review, section 2-2, and the
// fused-kernel description in section 3-6): for each query token t of block
// i and head h, o_t = softmax_u(scale * q_t.k_u + log g(blk(u))) v_u over the
// keys of the kept history blocks and the keys u <= t of block i, plus the
// row log-sum-exp.  The gate is added to every logit of its block inside
// the tile, and the attention matrix is never materialised.
//
// Design (MI355X):
//   - one workgroup per (query block, kv head): its waves are the G query
//     heads that share the kv head (GQA), 64 query rows each, so every K/V
//     tile staged in LDS feeds G*64 rows;
//   - K/V tiles are gathered by kept-block index; K is stored row-major and
//     V transposed in LDS, both padded by 16 bytes per row;
//   - S^T = K Q^T on 32x32 MFMA tiles with Q held in registers, so each
//     lane owns one query column and the softmax row statistics need a
//     single cross-half exchange; the key order inside each tile is chosen
//     so that the probabilities chain straight into O^T += V^T P^T;
//   - fp32 online softmax in the log2 domain; the log gate of the tile is one
//     scalar; the current (diagonal) block goes first so the running max is
//     finite before any gated history tile;
//   - the next tile's global loads are issued before the current tile's
//     MFMAs (register staging, one LDS buffer).
#include "sas_device.h"
#include "sas_launch.h"

namespace sas {

template <typename T, int D, int NW>
struct FwdTile {
  static constexpr int NT = NW * kWave;               // threads
  static constexpr int VEC = 16 / sizeof(T);          // elements per 16 bytes
  static constexpr int KROW = D + VEC;                // K row stride (elements)
  static constexpr int VROW = kBlock + VEC;           // V^T row stride (elements)
  static constexpr int KTOT = kBlock * D / VEC;         // 16-byte K chunks per tile
  static constexpr int VTOT = (kBlock / 4) * (D / VEC);  // 4-key x 16-byte V chunks
  static constexpr int KCH = (KTOT + NT - 1) / NT;       // per thread
  static constexpr int VCH = (VTOT + NT - 1) / NT;
};

template <typename T, int D, int NW>
struct TileStage {
  uint4 k[FwdTile<T, D, NW>::KCH];
  uint4 v[FwdTile<T, D, NW>::VCH][4];
};

// Global -> registers for one 64-key tile (zero past the sequence end).
template <typename T, int D, int NW>
__device__ inline void stage_load(TileStage<T, D, NW> &st, const T *kbase, const T *vbase,
                                  int nvalid, int kstride) {
  using F = FwdTile<T, D, NW>;
  constexpr int DC = D / F::VEC;
#pragma unroll
  for (int it = 0; it < F::KCH; ++it) {
    int c = threadIdx.x + it * F::NT;
    int key = c / DC, dc = c % DC;
    st.k[it] = (c < F::KTOT && key < nvalid)
                   ? *reinterpret_cast<const uint4 *>(kbase + (long)key * kstride + dc * F::VEC)
                   : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < F::VCH; ++it) {
    int c = threadIdx.x + it * F::NT;
    int kg = c / DC, dc = c % DC;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      int key = 4 * kg + x;
      st.v[it][x] = (c < F::VTOT && key < nvalid) ? *reinterpret_cast<const uint4 *>(vbase + (long)key * kstride +
                                                                    dc * F::VEC)
                                 : make_uint4(0, 0, 0, 0);
    }
  }
}

// Registers -> LDS: K row-major, V transposed ([d][key]).
template <typename T, int D, int NW>
__device__ inline void stage_store(const TileStage<T, D, NW> &st, T *Ks, T *Vt) {
  using F = FwdTile<T, D, NW>;
  constexpr int DC = D / F::VEC;
#pragma unroll
  for (int it = 0; it < F::KCH; ++it) {
    int c = threadIdx.x + it * F::NT;
    int key = c / DC, dc = c % DC;
    if (F::KTOT % F::NT != 0 && c >= F::KTOT) continue;
    *reinterpret_cast<uint4 *>(Ks + key * F::KROW + dc * F::VEC) = st.k[it];
  }
#pragma unroll
  for (int it = 0; it < F::VCH; ++it) {
    int c = threadIdx.x + it * F::NT;
    int kg = c / DC, dc = c % DC;
    if (F::VTOT % F::NT != 0 && c >= F::VTOT) continue;
    const T *r0 = reinterpret_cast<const T *>(&st.v[it][0]);
    const T *r1 = reinterpret_cast<const T *>(&st.v[it][1]);
    const T *r2 = reinterpret_cast<const T *>(&st.v[it][2]);
    const T *r3 = reinterpret_cast<const T *>(&st.v[it][3]);
#pragma unroll
    for (int e = 0; e < F::VEC; ++e) {
      T *dst = Vt + (dc * F::VEC + e) * F::VROW + 4 * kg;
      if constexpr (sizeof(T) == 2) {
        bf16x4 w = {r0[e], r1[e], r2[e], r3[e]};
        *reinterpret_cast<bf16x4 *>(dst) = w;
      } else {
        float4 w = make_float4(r0[e], r1[e], r2[e], r3[e]);
        *reinterpret_cast<float4 *>(dst) = w;
      }
    }
  }
}

template <typename T>
__device__ inline typename Mfma<T>::Op load_op(const T *p) {
  if constexpr (sizeof(T) == 2)
    return *reinterpret_cast<const bf16x8 *>(p);
  else
    return *p;
}

template <typename T, typename TO, int D, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdParams p) {
  using M = Mfma<T>;
  using F = FwdTile<T, D, NW>;
  constexpr int KS = M::K, E = M::E;
  constexpr int NKS = D / KS;          // k-steps over head_dim
  constexpr int NDT = D / 32;          // 32-row d tiles of O^T
  constexpr int NKC = kBlock / KS;     // k-steps over a 64-key tile
  constexpr int SPT = 32 / KS;         // k-steps per 32-key half tile

  __shared__ __attribute__((aligned(16))) T Ks[kBlock * F::KROW];
  __shared__ __attribute__((aligned(16))) T Vt[D * F::VROW];
  __shared__ int s_order[kMaxBudget];
  __shared__ int s_n;

  const T *q = static_cast<const T *>(p.q);
  const T *kk = static_cast<const T *>(p.k);
  const T *vv = static_cast<const T *>(p.v);

  const int Q = blockIdx.x;
  const int nhc = (p.G + NW - 1) / NW;
  const int g = blockIdx.y / nhc, hc = blockIdx.y % nhc;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int hf = lane / 32, l32 = lane % 32;
  const int hh = hc * NW + wave;
  const bool head_ok = hh < p.G;
  const int h = g * p.G + (head_ok ? hh : 0);

  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, Q);
  const int i = Q - p.cu_qblocks[s];
  const int seq_start = p.cu_seqlens[s];
  const int seq_len = p.cu_seqlens[s + 1] - seq_start;
  const int nq = min(kBlock, seq_len - i * kBlock);
  const long row = (long)g * p.QB + Q;
  const int32_t *sel = p.sel_idx + row * p.Kb;
  const float *slg = p.sel_lg + row * p.Kb;

  if (threadIdx.x == 0) {
    int n = 0;
    for (int sl = 0; sl < p.Kb; ++sl)
      if (sel[sl] == i) s_order[n++] = sl;
    for (int sl = 0; sl < p.Kb; ++sl) {
      int j = sel[sl];
      if (j >= 0 && j < i) s_order[n++] = sl;
    }
    s_n = n;
  }

  // Q as the B operand of S^T = K Q^T: lane -> query column, 2 tiles of 32.
  typename M::Op qreg[2][NKS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    int ql = 32 * nt + l32;
    const T *qp = q + ((long)(seq_start + i * kBlock + ql) * p.hq + h) * D + hf * E;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ql < nq)
        qreg[nt][ks] = load_op<T>(qp + ks * KS);
      else
        qreg[nt][ks] = typename M::Op{};
    }
  }

  f32x16 oacc[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  __syncthreads();
  const int ntiles = s_n;
  const int kstride = p.hkv * D;

  TileStage<T, D, NW> st;
  auto tile_ptrs = [&](int it, const T *&kb, const T *&vb, int &nvalid, int &j) {
    j = sel[s_order[it]];
    long tok = seq_start + (long)j * kBlock;
    kb = kk + (tok * p.hkv + g) * D;
    vb = vv + (tok * p.hkv + g) * D;
    nvalid = min(kBlock, seq_len - j * kBlock);
  };
  if (ntiles > 0) {
    const T *kb, *vb;
    int nv, j;
    tile_ptrs(0, kb, vb, nv, j);
    stage_load<T, D, NW>(st, kb, vb, nv, kstride);
  }

  for (int it = 0; it < ntiles; ++it) {
    const int slot = s_order[it];
    const int j = sel[slot];
    const float lg2 = slg[slot] * kLog2e;
    const bool diag = (j == i);
    __syncthreads();
    stage_store<T, D, NW>(st, Ks, Vt);
    __syncthreads();
    if (it + 1 < ntiles) {
      const T *kb, *vb;
      int nv, jn;
      tile_ptrs(it + 1, kb, vb, nv, jn);
      stage_load<T, D, NW>(st, kb, vb, nv, kstride);
    }

    // S^T[key][query] for two 32-key halves x two 32-query tiles.
    f32x16 sacc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const T *arow = Ks + (32 * mt + chain_key_of_row<T>(l32)) * F::KROW + hf * E;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        typename M::Op a = load_op<T>(arow + ks * KS);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = M::run(a, qreg[nt][ks], sacc[mt][nt]);
      }
    }

    // Online softmax per query column (log2 domain, gate folded in).
    typename M::Op pop[2][NKC];  // probabilities as B operands of O^T += V^T P^T
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int ql = 32 * nt + l32;
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = sacc[mt][nt][r] * p.scale_log2 + lg2;
          if (diag) {
            int key = 32 * mt + chain_slot<T>(r, hf);
            if (key > ql) z = -INFINITY;
          }
          sacc[mt][nt][r] = z;
          mx = fmaxf(mx, z);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float alpha = fast_exp2(m_run[nt] - m_new);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(sacc[mt][nt][r] - m_new);
          sacc[mt][nt][r] = pr;
          sum += pr;
        }
      sum += __shfl_xor(sum, 32);
      l_run[nt] = l_run[nt] * alpha + sum;
      m_run[nt] = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][nt][r] *= alpha;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int mt = kc / SPT, r0 = (kc % SPT) * E;
        if constexpr (E == 8) {
          bf16x8 b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)sacc[mt][nt][r0 + e];
          pop[nt][kc] = b;
        } else {
          pop[nt][kc] = sacc[mt][nt][r0];
        }
      }
    }

    // O^T[d][query] += V^T[d][key] P^T[key][query]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const T *arow = Vt + (32 * dt + l32) * F::VROW + hf * E;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        typename M::Op a = load_op<T>(arow + kc * KS);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = M::run(a, pop[nt][kc], oacc[dt][nt]);
      }
    }
  }

  if (!head_ok) return;
  TO *o = static_cast<TO *>(p.o);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ql = 32 * nt + l32;
    if (ql >= nq) continue;
    const long t = seq_start + i * kBlock + ql;
    const float inv = 1.f / l_run[nt];
    TO *op = o + (t * p.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * dt + d_row(4 * rg, hf);
        if constexpr (sizeof(TO) == 2) {
          bf16x4 w;
#pragma unroll
          for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[dt][nt][4 * rg + x] * inv);
          *reinterpret_cast<bf16x4 *>(op + d0) = w;
        } else {
          float4 w = make_float4(oacc[dt][nt][4 * rg] * inv, oacc[dt][nt][4 * rg + 1] * inv,
                                 oacc[dt][nt][4 * rg + 2] * inv, oacc[dt][nt][4 * rg + 3] * inv);
          *reinterpret_cast<float4 *>(op + d0) = w;
        }
      }
    if (hf == 0) p.lse[(long)h * p.T + t] = (m_run[nt] + fast_log2(l_run[nt])) * kLn2;
  }
}

template <typename T, typename TO, int D, int NW>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  dim3 grid(p.QB, p.hkv * ((p.G + NW - 1) / NW));
  hipLaunchKernelGGL((fwd_kernel<T, TO, D, NW>), grid, dim3(NW * 64), 0, stream, p);
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

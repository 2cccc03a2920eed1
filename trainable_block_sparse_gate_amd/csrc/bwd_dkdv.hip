// Gated block-sparse attention backward for gfx950: dK and dV.
//
// dk_u = scale sum_t dS_tu q_t and dv_u = sum_t P_tu dO_t over the query
// rows whose selection keeps u's block (dimensionstp.github.io review,
// sections 3-6: gradients pass through the gated probabilities).  One
// workgroup per segment of a key block, from the per-key-block lists that
// the preparation kernels build: K and V stay in registers, Q/dO tiles of
// the keeping rows stream through LDS, dK^T and dV^T accumulate in
// registers.  Key blocks kept by many rows are split over several segments;
// each writes a partial sum and the last one to finish adds all of them in
// segment order, so the result does not depend on which workgroup finishes
// last.
#include "sas_device.h"
#include "sas_launch.h"
#include "tile_stage.h"

namespace sas {
// ------------------------------------------------------------------ dk/dv
// Workgroup of 4 waves: wave = (query half qh, key half kh).  Each wave
// owns 32 keys (K, V as B operands in registers) and, per step, 32 of the
// 64 query rows of one head of one keeping row.  Q and dO tiles are double
// buffered in LDS (row-major only) with the step after next in flight from
// memory; the products that contract over query rows read their operands
// transposed straight from the row-major tiles.
constexpr int kSegMax = 64;  // entries per segment the kernel can hold

template <typename T, typename TO, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  using M = Mfma<T>;
  constexpr int NT = 256;
  using RT = RowTile<T, D, NT>;
  constexpr int KS = M::K, E = M::E;
  constexpr int NKS = D / KS, NDT = D / 32, SPT = 32 / KS;
  constexpr int TILE = RT::ELEMS;                 // elements per tile
  constexpr int LDS_T = 2 * 2 * TILE;             // {Q, dO} x 2 buffers
  constexpr int LDS_RED = 2 * 2 * NDT * 16 * kWave;  // floats: 2 waves x (dk, dv)
  constexpr int LDS_BYTES =
      (LDS_T * (int)sizeof(T) > LDS_RED * 4) ? LDS_T * (int)sizeof(T) : LDS_RED * 4;

  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float s_lse[2][kBlock];
  __shared__ __attribute__((aligned(16))) float s_D[2][kBlock];
  __shared__ int s_ent[kSegMax];
  __shared__ float s_lg[kSegMax];
  __shared__ int s_last;

  const int w = blockIdx.x;
  const int nx = p.hkv * p.QB;
  if (w >= p.seg_off[nx]) return;
  int lo = 0, hi = nx - 1;  // largest x with seg_off[x] <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.seg_off[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int x = lo;
  const int g = x / p.QB, kb = x % p.QB;
  const int s = seq_of_qblock(p.cu_qblocks, p.num_seqs, kb);
  const int q0 = p.cu_qblocks[s];
  const int j = kb - q0;
  const int seq_start = p.cu_seqlens[s];
  const int seq_len = p.cu_seqlens[s + 1] - seq_start;
  const int nvalid = min(kBlock, seq_len - j * kBlock);
  const long ktok0 = seq_start + (long)j * kBlock;
  const int nseg = p.seg_off[x + 1] - p.seg_off[x];
  const int seg = w - p.seg_off[x];
  const int cnt = p.count[x];
  const int e0 = seg * p.seg, e1 = min(cnt, e0 + p.seg);
  const int nent = max(0, e1 - e0);

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int hf = lane / 32, l32 = lane % 32;
  const int kh = wave % 2, qh = wave / 2;
  const int key = 32 * kh + l32;  // this lane's key (column of S)

  if (threadIdx.x < nent) {
    const int ent = p.list[(long)x * p.max_nb + e0 + threadIdx.x];
    s_ent[threadIdx.x] = ent;
    s_lg[threadIdx.x] = p.sel_lg[((long)g * p.QB + (ent >> 8)) * p.Kb + (ent & 255)] * kLog2e;
  }

  const T *q = static_cast<const T *>(p.q);
  const T *kk = static_cast<const T *>(p.k);
  const T *vv = static_cast<const T *>(p.v);
  const TO *dO = static_cast<const TO *>(p.dO);
  T *tiles = reinterpret_cast<T *>(smem);  // [buf][Q | dO][64][ROW]

  typename M::Op kreg[NKS], vreg[NKS];
  {
    const long base = ((ktok0 + key) * p.hkv + g) * D + hf * E;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (key < nvalid) {
        kreg[ks] = lds_op<T>(kk + base + ks * KS);
        vreg[ks] = lds_op<T>(vv + base + ks * KS);
      } else {
        kreg[ks] = typename M::Op{};
        vreg[ks] = typename M::Op{};
      }
    }
    // K and V are complete before any step's loads are issued; the wait
    // counter tracking then never makes a step wait for its own prefetch
    wait_vmem_all();
  }
  f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dkacc[dt] = dvacc[dt] = f32x16{};

  const int G = p.G;
  const int nsteps = nent * G;
  const long qstride = (long)p.hq * D;
  RT qst, dst;
  // lse and D of the staged step, raw: nothing consumes them before the
  // step is stored, so the loads stay in flight for a whole step
  float st_lse = 0.f, st_D = 0.f;
  bool st_ok = false;
  __syncthreads();  // s_ent / s_lg visible

  auto load_step = [&](int st) {
    const int ent = s_ent[st / G];
    const int i = (ent >> 8) - q0;
    const int h = g * G + st % G;
    const long t0 = seq_start + (long)i * kBlock;
    const int nq = min(kBlock, seq_len - i * kBlock);
    rowtile_load<T, T, D, NT>(qst, q + (t0 * p.hq + h) * D, qstride, nq);
    rowtile_load<TO, T, D, NT>(dst, dO + (t0 * p.hq + h) * D, qstride, nq);
    if (threadIdx.x < kBlock) {
      st_ok = threadIdx.x < nq;
      const int r = st_ok ? threadIdx.x : nq - 1;
      st_lse = p.lse[(long)h * p.T + t0 + r];
      st_D = p.Dbuf[(long)h * p.T + t0 + r];
    }
  };
  auto store_step = [&](int b) {
    rowtile_store<T, D, NT>(qst, tiles + (2 * b + 0) * TILE);
    rowtile_store<T, D, NT>(dst, tiles + (2 * b + 1) * TILE);
    if (threadIdx.x < kBlock) {
      s_lse[b][threadIdx.x] = st_ok ? st_lse * kLog2e : INFINITY;
      s_D[b][threadIdx.x] = st_ok ? st_D : 0.f;
    }
  };
  if (nsteps > 0) {
    load_step(0);
    store_step(0);
    if (nsteps > 1) load_step(1);
  }
  __syncthreads();

  // Per step: compute from one buffer, then store the next step's tile
  // (loaded one step earlier) into the other buffer, issue the loads of the
  // step after that, and barrier.  No LDS write of a wave is in flight while
  // its transposed reads (ds_read_b64_tr_b16) issue: with writes pending,
  // those reads returned wrong data on gfx950.
  for (int st = 0; st < nsteps; ++st) {
    const int b = st & 1;

    const int e = st / G;
    const int i = (s_ent[e] >> 8) - q0;
    const int nq = min(kBlock, seq_len - i * kBlock);
    const float lg2 = s_lg[e];
    const bool diag = (i == j);
    const T *Qs = tiles + (2 * b + 0) * TILE;
    const T *Ds = tiles + (2 * b + 1) * TILE;

    // S[query][key] and dP[query][key] for 32 queries x this wave's 32 keys;
    // query rows loaded in chain order so P and dS feed the next products.
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    const int qrow = 32 * qh + chain_key_of_row<T>(l32);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sacc = M::run(tile_op<T, D>(Qs, qrow, hf * E + ks * KS), kreg[ks], sacc);
      pacc = M::run(tile_op<T, D>(Ds, qrow, hf * E + ks * KS), vreg[ks], pacc);
    }
    // this lane's 16 query rows, in register order, come in four runs of 4
    // consecutive rows: fetch their lse and D as float4s
    // (bf16 chain order; the fp32 order interleaves, so it reads one by one)
    float lse_r[16], D_r[16];
    if constexpr (E == 8) {
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) {
        const int q4 = 32 * qh + chain_slot<T>(r0, hf);
        const float4 a = *reinterpret_cast<const float4 *>(&s_lse[b][q4]);
        const float4 c = *reinterpret_cast<const float4 *>(&s_D[b][q4]);
        lse_r[r0] = a.x; lse_r[r0 + 1] = a.y; lse_r[r0 + 2] = a.z; lse_r[r0 + 3] = a.w;
        D_r[r0] = c.x; D_r[r0 + 1] = c.y; D_r[r0 + 2] = c.z; D_r[r0 + 3] = c.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        lse_r[r] = s_lse[b][32 * qh + chain_slot<T>(r, hf)];
        D_r[r] = s_D[b][32 * qh + chain_slot<T>(r, hf)];
      }
    }
    // full tiles (the common case) need no mask; the test is uniform
    if (!diag && nq == kBlock && nvalid == kBlock) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(sacc[r] * p.scale_log2 + lg2 - lse_r[r]);
        sacc[r] = pr;
        pacc[r] = pr * (pacc[r] - D_r[r]);
      }
    } else {
      const bool key_ok = key < nvalid;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qh + chain_slot<T>(r, hf);
        const bool ok = key_ok && ql < nq && !(diag && key > ql);
        const float z = ok ? sacc[r] * p.scale_log2 + lg2 - lse_r[r] : -INFINITY;
        const float pr = fast_exp2(z);
        sacc[r] = pr;
        pacc[r] = pr * (pacc[r] - D_r[r]);
      }
    }
    // dV^T[d][key] += dO^T[d][query] P[query][key];  dK^T += Q^T dS
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int kc = 0; kc < SPT; ++kc) {
        const int kq = 32 * qh + kc * KS;
        dvacc[dt] = M::run(tile_op_rows<T, D>(Ds, kq, 32 * dt), regs_op<T>(sacc, kc * E),
                           dvacc[dt]);
        dkacc[dt] = M::run(tile_op_rows<T, D>(Qs, kq, 32 * dt), regs_op<T>(pacc, kc * E),
                           dkacc[dt]);
      }
    }
    if (st + 1 < nsteps) store_step(b ^ 1);
    if (st + 2 < nsteps) load_step(st + 2);
    __syncthreads();
  }

  // Add the two query halves: waves qh = 1 hand their sums to qh = 0.
  float *red = reinterpret_cast<float *>(smem);
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((kh * 2 + 0) * NDT * 16 + dt * 16 + r) * kWave + lane] = dkacc[dt][r];
        red[((kh * 2 + 1) * NDT * 16 + dt * 16 + r) * kWave + lane] = dvacc[dt][r];
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[dt][r] += red[((kh * 2 + 0) * NDT * 16 + dt * 16 + r) * kWave + lane];
        dvacc[dt][r] += red[((kh * 2 + 1) * NDT * 16 + dt * 16 + r) * kWave + lane];
      }
    // lane holds key `key`, 4 consecutive d per register group
    float *dk_out, *dv_out;
    bool write = true;
    if (nseg == 1) {
      write = key < nvalid;
      dk_out = p.dk + ((ktok0 + key) * p.hkv + g) * D;
      dv_out = p.dv + ((ktok0 + key) * p.hkv + g) * D;
    } else {
      float *part = p.partial + (long)w * 2 * kBlock * D;
      dk_out = part + (long)key * D;
      dv_out = part + (long)(kBlock + key) * D;
    }
    if (write) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = 32 * dt + d_row(4 * rg, hf);
          *reinterpret_cast<float4 *>(dk_out + d0) =
              make_float4(dkacc[dt][4 * rg] * p.scale, dkacc[dt][4 * rg + 1] * p.scale,
                          dkacc[dt][4 * rg + 2] * p.scale, dkacc[dt][4 * rg + 3] * p.scale);
          *reinterpret_cast<float4 *>(dv_out + d0) =
              make_float4(dvacc[dt][4 * rg], dvacc[dt][4 * rg + 1], dvacc[dt][4 * rg + 2],
                          dvacc[dt][4 * rg + 3]);
        }
    }
  }
  if (nseg == 1) return;

  // Split key block: the last segment to finish adds the partials in order.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&p.done[x], 1) == nseg - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int n = kBlock * D;
  const float *part0 = p.partial + (long)p.seg_off[x] * 2 * n;
  for (int e = threadIdx.x * 4; e < 2 * n; e += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sg = 0; sg < nseg; ++sg) {
      const float4 v = *reinterpret_cast<const float4 *>(part0 + (long)sg * 2 * n + e);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const int which = e / n, kk2 = (e % n) / D, d = e % D;
    if (kk2 >= nvalid) continue;
    float *out = (which == 0 ? p.dk : p.dv) + ((ktok0 + kk2) * p.hkv + g) * D + d;
    *reinterpret_cast<float4 *>(out) = acc;
  }
}

// ------------------------------------------------------------------ launch
template <typename T, typename TO, int D>
static hipError_t launch_dkdv_t(const BwdParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, TO, D>), dim3(p.U), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdParams &p, int dtype_bf16, int out_bf16, int head_dim,
                           hipStream_t stream) {
  if (dtype_bf16) {
    if (out_bf16)
      return head_dim == 128 ? launch_dkdv_t<__bf16, __bf16, 128>(p, stream)
                             : launch_dkdv_t<__bf16, __bf16, 64>(p, stream);
    return head_dim == 128 ? launch_dkdv_t<__bf16, float, 128>(p, stream)
                           : launch_dkdv_t<__bf16, float, 64>(p, stream);
  }
  return head_dim == 128 ? launch_dkdv_t<float, float, 128>(p, stream)
                         : launch_dkdv_t<float, float, 64>(p, stream);
}

}  // namespace sas

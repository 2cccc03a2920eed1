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
//            each workgroup streams a few 64-token K/V blocks (16-byte
//            coalesced loads, next block prefetched into registers), keeps
//            an fp32 online softmax per query head with the block's log
//            gate added, and writes an unnormalised partial; a second
//            kernel merges the partials with a log-sum-exp combine in a
//            fixed order.
#include "sas_device.h"
#include "sas_launch.h"

namespace sas {

__device__ inline const __bf16 *kv_row(const DecodeParams &p, const __bf16 *cache, int b, int g,
                                       int tok) {
  if (p.paged) {
    const int page = p.page_table[(long)b * p.max_pages + tok / kBlock];
    return cache + (((long)page * p.hkv + g) * kBlock + (tok % kBlock)) * p.D;
  }
  return cache + (((long)b * p.hkv + g) * p.max_seqlen + tok) * p.D;
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
  p.ksum[(((long)b * p.hkv + g) * p.D + e) * p.nblk_stride + j] = acc / (float)kBlock;
}

// ------------------------------------------------------------------ scores
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
  const float *ks = p.ksum + ((long)b * p.hkv + g) * p.D * p.nblk_stride + j;
  float acc = 0.f;
  for (int e = 0; e < p.D; ++e) acc = fmaf(qbar[e], ks[(long)e * p.nblk_stride], acc);
  p.scores[((long)b * p.hkv + g) * p.nblk_stride + j] = acc / p.sqrt_d;
}

// ------------------------------------------------------------------ attend
// Thread layout per 64-token block: thread = (key group kr, channel chunk
// dc); a chunk is 8 channels (16 bytes), KR = 256 / (D / 8) key groups,
// each thread owns keys kr, kr + KR, ... (KPT of them).  Running max and
// sum of every query head live in LDS; one wave per head updates them.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_attend_kernel(DecodeParams p) {
  constexpr int DC = D / 8;
  constexpr int KR = 256 / DC;
  constexpr int KPT = kBlock / KR;
  __shared__ float part[kBlock][G][DC + 1];  // per-chunk partial dot products
  __shared__ float prob[G][kBlock];
  __shared__ float s_m[G], s_l[G], s_alpha[G];
  __shared__ float obuf[KR][G][D];

  const int row = blockIdx.y;  // b * hkv + g
  const int split = blockIdx.x;
  const int b = row / p.hkv, g = row % p.hkv;
  const int L = p.seqlens[b];
  const int cur = (L - 1) / kBlock;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int kr = tid / DC, dc = tid % DC;
  const int32_t *sel = p.sel_idx + (long)row * p.Kb;
  const float *slg = p.sel_lg ? p.sel_lg + (long)row * p.Kb : nullptr;
  const int s0 = split * p.per_split, s1 = min(p.Kb, s0 + p.per_split);
  const __bf16 *kc = static_cast<const __bf16 *>(p.k);
  const __bf16 *vc = static_cast<const __bf16 *>(p.v);
  const __bf16 *q = static_cast<const __bf16 *>(p.q);

  // this thread's 8 channels of every query head of the group, pre-scaled
  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint4 raw =
        *reinterpret_cast<const uint4 *>(q + ((long)b * p.hq + g * G + hh) * D + dc * 8);
    const __bf16 *qq = reinterpret_cast<const __bf16 *>(&raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hh][e] = (float)qq[e] * p.scale_log2;
  }
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }

  auto valid_block = [&](int sl, int &j, int &nv) {
    j = sel[sl];
    if (j < 0 || j > cur) return false;
    nv = (j == cur) ? L - cur * kBlock : kBlock;
    return true;
  };
  uint4 kst[KPT], vst[KPT];
  auto load_block = [&](int j, int nv) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int key = kr + m * KR;
      if (key < nv) {
        kst[m] = *reinterpret_cast<const uint4 *>(kv_row(p, kc, b, g, j * kBlock + key) + dc * 8);
        vst[m] = *reinterpret_cast<const uint4 *>(kv_row(p, vc, b, g, j * kBlock + key) + dc * 8);
      } else {
        kst[m] = make_uint4(0, 0, 0, 0);
        vst[m] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  int sl = s0, j = 0, nv = 0;
  while (sl < s1 && !valid_block(sl, j, nv)) ++sl;
  if (sl < s1) load_block(j, nv);

  while (sl < s1) {
    const int nvc = nv;
    const float lg2 = slg ? slg[sl] * kLog2e : 0.f;
    float vf[KPT][8];
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const __bf16 *kk = reinterpret_cast<const __bf16 *>(&kst[m]);
      const __bf16 *vv = reinterpret_cast<const __bf16 *>(&vst[m]);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d_ = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d_ = fmaf(qv[hh][e], (float)kk[e], d_);
        part[kr + m * KR][hh][dc] = d_;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[m][e] = (float)vv[e];
    }
    // prefetch the next valid block of this split
    int sn = sl + 1, jn = 0, nvn = 0;
    while (sn < s1 && !valid_block(sn, jn, nvn)) ++sn;
    if (sn < s1) load_block(jn, nvn);
    __syncthreads();
    // one wave per head: finish the dot products, gate, mask, update stats
    for (int hh = wave; hh < G; hh += 4) {
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) z += part[lane][hh][c];
      z = lane < nvc ? z + lg2 : -INFINITY;
      const float m_old = s_m[hh];
      const float m_new = fmaxf(m_old, wave_max(z));
      const float pz = (m_new == -INFINITY) ? 0.f : fast_exp2(z - m_new);
      const float sum = wave_sum(pz);
      prob[hh][lane] = pz;
      if (lane == 0) {
        const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
        s_alpha[hh] = alpha;
        s_l[hh] = s_l[hh] * alpha + sum;
        s_m[hh] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float alpha = s_alpha[hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const float pr = prob[hh][kr + m * KR];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[m][e], acc[hh][e]);
      }
    }
    __syncthreads();
    sl = sn;
    j = jn;
    nv = nvn;
  }

  // sum the key groups, then write this split's unnormalised partial
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) obuf[kr][hh][dc * 8 + e] = acc[hh][e];
  __syncthreads();
  float *out = p.partial + ((long)row * p.nsplit + split) * G * (D + 2);
  for (int x = tid; x < G * D; x += 256) {
    const int hh = x / D, d = x % D;
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < KR; ++r) o += obuf[r][hh][d];
    out[hh * (D + 2) + d] = o;
  }
  if (tid < G) {
    out[tid * (D + 2) + D] = s_m[tid];
    out[tid * (D + 2) + D + 1] = s_l[tid];
  }
}

// Merge the splits of every (sequence, kv head) in split order.
template <int D, int G, typename TO>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int row = blockIdx.x;
  const int b = row / p.hkv, g = row % p.hkv;
  const float *part = p.partial + (long)row * p.nsplit * G * (D + 2);
  TO *o = static_cast<TO *>(p.o);
  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int hh = x / D, d = x % D;
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) M = fmaxf(M, part[(sp * G + hh) * (D + 2) + D]);
    float Lsum = 0.f, acc = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      const float *ps = part + (sp * G + hh) * (D + 2);
      const float w = (ps[D] == -INFINITY) ? 0.f : fast_exp2(ps[D] - M);
      Lsum += ps[D + 1] * w;
      acc += ps[d] * w;
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

hipError_t launch_pooled_scores(const DecodeParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(pooled_scores_kernel, dim3((p.nblk_stride + 255) / 256, p.batch * p.hkv),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_attend_t(const DecodeParams &p, hipStream_t stream) {
  const int rows = p.batch * p.hkv;
  hipLaunchKernelGGL((decode_attend_kernel<D, G>), dim3(p.nsplit, rows), dim3(256), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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

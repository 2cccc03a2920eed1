// Device helpers shared by the gfx950 kernels: MFMA wrappers with their
// operand layouts, bf16 conversion and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kBlock = 64;   // tokens per block
constexpr int kWave = 64;    // lanes per wavefront
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// 32x32 MFMA tiles.  One instruction computes D[32][32] += A[32][K] B[K][32]
// with K = 16 (bf16, v_mfma_f32_32x32x16_bf16) or K = 2 (fp32,
// v_mfma_f32_32x32x2f32).  Operand layout, lane l = 0..63, h = l / 32:
//   A: lane holds A[l % 32][h*E .. h*E + E-1]     (E = K / 2 elements)
//   B: lane holds B[h*E .. h*E + E-1][l % 32]
//   D: lane holds 16 values, register r -> D[8*(r/4) + 4*h + r%4][l % 32]
// ---------------------------------------------------------------------------
template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  static constexpr int K = 16;  // contraction per instruction
  static constexpr int E = 8;   // operand elements per lane
  typedef bf16x8 Op;
  __device__ static inline f32x16 run(const Op &a, const Op &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int K = 2;
  static constexpr int E = 1;
  typedef float Op;
  __device__ static inline f32x16 run(const Op &a, const Op &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// 16x16x32 bf16 MFMA: lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16], e = 0..7; D register r is D[4 (l / 16) + r][l % 16].
__device__ inline f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row of the D tile held by register r of a lane in half h.
__device__ __host__ constexpr inline int d_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// When a D tile (rows = keys) is fed back as the B operand of a second MFMA
// that contracts over those keys, register r of half h lands on contraction
// position slot(r, h).  Loading the first product's A rows in the order
// key(m) = slot(r(m), h(m)) makes every lane's registers hold consecutive
// keys, so the result chains into the next product with no data movement.
template <typename T>
__device__ __host__ constexpr inline int chain_slot(int r, int h) {
  return Mfma<T>::E == 8 ? 16 * (r / 8) + 8 * h + (r % 8) : 2 * r + h;
}
template <typename T>
__device__ __host__ constexpr inline int chain_key_of_row(int m) {
  return chain_slot<T>(4 * (m / 8) + (m % 4), (m / 4) % 2);
}

// ---------------------------------------------------------------------------
// MFMA operand that contracts over the ROWS of a row-major LDS tile X[k][m]
// (row stride ld elements): lane l receives X[kb + h*E + e][mb + l % 32],
// e = 0..E-1, h = l / 32 -- the k-contiguous layout both A and B operands
// use.  For bf16 this is two ds_read_b64_tr_b16: within each 16-lane group,
// output lane j, element e comes from source lane 4e + j/4, element j % 4,
// so a source lane s that points at row kb + s/4, columns 4(s%4)..+3 of its
// group's 16 columns hands every output lane four consecutive rows of one
// column.  Groups: lanes 16g..16g+15 cover columns 16(g%2)..+15 and rows
// 8(g/2)..+7 (two reads of four rows).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) short lds_short;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <typename T>
__device__ inline typename Mfma<T>::Op lds_op_rows(const T *X, int ld, int kb, int mb) {
  const int lane = threadIdx.x % kWave;
  if constexpr (sizeof(T) == 2) {
    const int g = lane / 16, s = lane % 16;
    const int row = kb + 8 * (g / 2) + s / 4;
    const int col = mb + 16 * (g % 2) + 4 * (s % 4);
    const lds_short *base = (const lds_short *)((const T *)X + row * ld + col);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)base);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + 4 * ld));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  } else {
    return X[(kb + lane / 32) * ld + mb + lane % 32];
  }
}

// Wait until every vector-memory load this wave issued has returned
// (s_waitcnt vmcnt(0); the expcnt and lgkmcnt fields are left at their
// maxima, i.e. not waited on).  Resets the compiler's pending-load tracking
// at a point where that is cheap.
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N) alone (N < 64; vmcnt sits in bits 3:0 and 15:14).
// The scheduler moves no instruction across it, so whatever follows in the
// source really runs after the wait.
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier without the workgroup-scope fence that __syncthreads()
// adds (that fence also waits for every global->LDS request in flight):
// this wave's LDS accesses are complete, the compiler moves no memory
// access across it, and outstanding global->LDS requests stay in flight.
__device__ inline void barrier_keep_requests() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier between two steps of a software-pipelined loop: this
// wave's LDS accesses are complete, and no instruction, arithmetic
// included, is moved across it, so each step's work stays inside its step.
__device__ inline void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// x as three bf16 parts [hi, mid, lo, 0, 0, 0, 0, 0] with hi + mid + lo = x
// to within 2^-24 relative (each part is the rounding of what the previous
// ones leave; the differences are exact in fp32).  Infinite x gives
// [x, 0, ...].
__device__ inline bf16x8 split3_bf16(float x) {
  bf16x8 r = {};
  const __bf16 hi = (__bf16)x;
  const float r1 = __builtin_isfinite(x) ? x - (float)hi : 0.f;
  const __bf16 mid = (__bf16)r1;
  r[0] = hi;
  r[1] = mid;
  r[2] = (__bf16)(r1 - (float)mid);
  return r;
}

// Index of the calling wave in its workgroup, as a wave-uniform value:
// threadIdx.x / 64 is the same in every lane, but only readfirstlane lets
// the compiler know, so that what depends on it (head indices, loop
// bounds, addresses) stays in scalar registers and loops over it stay
// uniform branches rather than exec-masked ones.  Call with all lanes active.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// The kept blocks of one selection row as seen by query block i, built by
// one whole wave: the slots' block indices j (-1 = empty) with j <= i, in
// slot order -- with the current block i moved to the front when
// current_first -- are written to out_j (and their slots to out_slot when it
// is given, their log gates times log2 e to out_lg2).  All of the row's
// slots are read at once (one per lane, Kb <= 4 * 64).  Returns the count.
__device__ inline int wave_kept_blocks(const int32_t *sel, const float *slg, int Kb, int i,
                                       bool current_first, int *out_j, int *out_slot,
                                       float *out_lg2) {
  const int lane = threadIdx.x % kWave;
  int jv[4];
  float lgv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int sl = 64 * c + lane;
    jv[c] = -1;
    lgv[c] = 0.f;
    if (sl < Kb) {
      jv[c] = sel[sl];
      lgv[c] = slg[sl];
    }
  }
  int nd = 0;  // the current block (at most once), when it goes first
  if (current_first) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool cur = jv[c] == i;
      if (cur) {
        out_j[0] = i;
        if (out_slot) out_slot[0] = 64 * c + lane;
        out_lg2[0] = lgv[c] * kLog2e;
      }
      nd += __popcll(__ballot(cur));
    }
  }
  int n = nd;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool ok = jv[c] >= 0 && (current_first ? jv[c] < i : jv[c] <= i);
    const uint64_t m = __ballot(ok);
    if (ok) {
      const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
      out_j[pos] = jv[c];
      if (out_slot) out_slot[pos] = 64 * c + lane;
      out_lg2[pos] = lgv[c] * kLog2e;
    }
    n += __popcll(m);
  }
  return n;
}

// Value of x in lane k (k uniform across the wave), without touching memory.
__device__ inline int lane_value(int x, int k) { return __builtin_amdgcn_readlane(x, k); }
__device__ inline float lane_value(float x, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}
__device__ inline long lane_value(long x, int k) {
  const unsigned lo = __builtin_amdgcn_readlane((int)(unsigned)((unsigned long)x), k);
  const unsigned hi = __builtin_amdgcn_readlane((int)(unsigned)((unsigned long)x >> 32), k);
  return (long)(((unsigned long)hi << 32) | lo);
}

// Wait until this wave's LDS reads and writes have completed (lgkmcnt(0));
// the scheduler moves no instruction across it.
__device__ inline void wait_lds_all() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte-per-lane global -> LDS request (global_load_lds_dwordx4):
// lane l's 16 bytes from gsrc land at lds_base + 16 l; lds_base must be the
// same for every lane of the wave.  Completion is counted by vmcnt.
__device__ inline void load_lds16(const void *gsrc, void *lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_base,
                                   16, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ inline float to_f32(__bf16 x) { return (float)x; }
__device__ inline float to_f32(float x) { return x; }

template <typename T>
__device__ inline T from_f32(float x);
template <>
__device__ inline float from_f32<float>(float x) { return x; }
template <>
__device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // round to nearest even

// ---------------------------------------------------------------------------
// Wavefront reductions (all 64 lanes)
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Sequence of a global query block: largest s with cu_qblocks[s] <= Q.
__device__ inline int seq_of_qblock(const int32_t *cu_qblocks, int num_seqs, int Q) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_qblocks[mid] <= Q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace sas

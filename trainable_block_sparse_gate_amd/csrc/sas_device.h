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

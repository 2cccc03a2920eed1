// Staging of one 64-row x D tile: global -> registers -> LDS.
//
// A thread owns 16-byte chunks (VEC elements of the LDS element type T);
// consecutive threads take consecutive chunks of a row, so the global loads
// are coalesced 16-byte (or 32-byte when an fp32 source is narrowed to bf16)
// accesses.  The chunks live in registers as native 4 x u32 vectors.
#pragma once
#include "sas_device.h"

namespace sas {

// Row-major tiles in LDS, 64 rows x D columns, no padding, with the 16-byte
// chunks of each row permuted by an XOR swizzle so that the access patterns
// the kernels use are free of bank conflicts.  The LDS serves 256 bytes (64
// banks of 4 bytes) per cycle, and a 16-chunk row (256 bytes) spans every
// bank once, so a chunk's banks are set by its stored position alone:
//   - 16-byte operand reads: 16 lanes per cycle read the same column chunk
//     of 16 different rows (an aligned group of 16), so the 16 rows must
//     store it at 16 different positions;
//   - transposed reads (ds_read_b64_tr_b16): 32 lanes per cycle read 4
//     consecutive rows (4a .. 4a + 3) x 4 aligned consecutive chunks (two
//     16-lane groups of two chunks each), so those 16 chunks must land at 16
//     different positions.
// With 16 chunks per row the chunk c of row r is stored at c ^ f(r),
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3): a bijection on each aligned group
// of 16 rows, and on rows 4a .. 4a + 3 it takes 4 values with distinct
// upper two bits, so XOR with the chunk's own lower two bits gives 16
// different positions.  (An earlier map, ((r & 7) << 1) | ((r >> 3) & 1),
// left the transposed reads 2-way conflicted: measured half of their LDS
// cycles.)  f(r + 16) = f(r), and XOR acts on the chunk bits only, so an
// offset can be moved by 16 rows or XORed with a chunk offset directly.
template <typename T, int D>
struct Swz {
  static constexpr int VEC = 16 / sizeof(T);  // elements per chunk
  static constexpr int CPR = D / VEC;         // chunks per row
  __device__ static inline int f(int r) {
    if constexpr (CPR >= 16)
      return ((r & 3) << 2) | ((r >> 2) & 3);
    else
      return (r >> 1) & (CPR - 1);
  }
  // element offset of (row, col) inside a tile
  __device__ static inline int off(int r, int col) {
    return r * D + (((col / VEC) ^ f(r)) * VEC) + (col % VEC);
  }
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of T from TS elements at src (TS == T: one load; fp32 -> bf16:
// two 16-byte loads, rounded to nearest even).
template <typename TS, typename T>
__device__ inline u32x4 load_chunk(const TS *src) {
  if constexpr (sizeof(TS) == sizeof(T)) {
    return *reinterpret_cast<const u32x4 *>(src);
  } else {
    const float4 a = reinterpret_cast<const float4 *>(src)[0];
    const float4 b = reinterpret_cast<const float4 *>(src)[1];
    const bf16x8 w = {(__bf16)a.x, (__bf16)a.y, (__bf16)a.z, (__bf16)a.w,
                      (__bf16)b.x, (__bf16)b.y, (__bf16)b.z, (__bf16)b.w};
    return __builtin_bit_cast(u32x4, w);
  }
}

// Register staging of one tile.
template <typename T, int D, int NT>
struct RowTile {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int DC = D / VEC;
  static constexpr int TOT = kBlock * DC;
  static constexpr int CH = (TOT + NT - 1) / NT;
  static constexpr int ELEMS = kBlock * D;  // LDS elements per tile
  u32x4 v[CH];
};

// Rows >= nvalid are loaded from row nvalid - 1 (finite values; the kernels
// mask those rows out of every product that could see them).  base should
// be wave-uniform: each lane then adds only a 32-bit byte offset to it
// (64 rows of `stride` elements must span less than 2^31 bytes).
template <typename TS, typename T, int D, int NT>
__device__ inline void rowtile_load(RowTile<T, D, NT> &st, const TS *base, int stride,
                                    int nvalid) {
  using F = RowTile<T, D, NT>;
  const char *b = reinterpret_cast<const char *>(base);
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    const int row = c / F::DC, dc = c % F::DC;
    if (F::TOT % NT == 0 || c < F::TOT) {
      const int r = row < nvalid ? row : nvalid - 1;
      const unsigned off = (unsigned)((r * stride + dc * F::VEC) * (int)sizeof(TS));
      st.v[it] = load_chunk<TS, T>(reinterpret_cast<const TS *>(b + off));
    }
  }
}

template <typename T, int D, int NT>
__device__ inline void rowtile_store(const RowTile<T, D, NT> &st, T *lds) {
  using F = RowTile<T, D, NT>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    if (F::TOT % NT != 0 && c >= F::TOT) continue;
    const int row = c / F::DC, dc = c % F::DC;
    *reinterpret_cast<u32x4 *>(lds + Swz<T, D>::off(row, dc * F::VEC)) = st.v[it];
  }
}

// E consecutive values of an output-dtype tensor (dO, o) held in registers
// with vector loads; get(e) is value e as a float, as_op<T>() the values as
// one MFMA operand of type T (rounded to nearest even when TO is wider).
template <typename TO, int E>
struct OutChunk;

template <>
struct OutChunk<__bf16, 8> {
  u32x4 w;
  __device__ void load(const __bf16 *p) { w = *reinterpret_cast<const u32x4 *>(p); }
  __device__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  __device__ float get(int e) const {
    const unsigned x = w[e / 2];
    return __uint_as_float((e % 2) ? (x & 0xffff0000u) : (x << 16));
  }
  template <typename T>
  __device__ bf16x8 as_op() const { return __builtin_bit_cast(bf16x8, w); }
};

template <>
struct OutChunk<float, 8> {
  float4 a, b;
  __device__ void load(const float *p) {
    a = reinterpret_cast<const float4 *>(p)[0];
    b = reinterpret_cast<const float4 *>(p)[1];
  }
  __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ float get(int e) const {
    const float4 &c = e < 4 ? a : b;
    switch (e % 4) {
      case 0: return c.x;
      case 1: return c.y;
      case 2: return c.z;
      default: return c.w;
    }
  }
  template <typename T>
  __device__ bf16x8 as_op() const {
    return bf16x8{(__bf16)a.x, (__bf16)a.y, (__bf16)a.z, (__bf16)a.w,
                  (__bf16)b.x, (__bf16)b.y, (__bf16)b.z, (__bf16)b.w};
  }
};

template <>
struct OutChunk<float, 1> {
  float v;
  __device__ void load(const float *p) { v = *p; }
  __device__ void zero() { v = 0.f; }
  __device__ float get(int) const { return v; }
  template <typename T>
  __device__ float as_op() const { return v; }
};

// MFMA operand from a swizzled tile, k-contiguous along a row:
// lane gets X[row][col .. col + E - 1].
template <typename T, int D>
__device__ inline typename Mfma<T>::Op tile_op(const T *X, int row, int col) {
  const T *p = X + Swz<T, D>::off(row, col);
  if constexpr (sizeof(T) == 2)
    return *reinterpret_cast<const bf16x8 *>(p);
  else
    return *p;
}

// MFMA operand contracting over the tile's ROWS (see lds_op_rows in
// sas_device.h for the lane mapping): lane l receives
// X[kb + h*E + e][mb + l % 32], e = 0..E-1.
template <typename T, int D>
__device__ inline typename Mfma<T>::Op tile_op_rows(const T *X, int kb, int mb) {
  const int lane = threadIdx.x % kWave;
  if constexpr (sizeof(T) == 2) {
    const int g = lane / 16, s = lane % 16;
    const int row = kb + 8 * (g / 2) + s / 4;
    const int col = mb + 16 * (g % 2) + 4 * (s % 4);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(const lds_short *)(X + Swz<T, D>::off(row, col)));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(const lds_short *)(X + Swz<T, D>::off(row + 4, col)));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  } else {
    return X[Swz<T, D>::off(kb + lane / 32, mb + lane % 32)];
  }
}

// Operand of a 16x16x32 bf16 MFMA that contracts over the ROWS of a
// swizzled tile: lane l (group q = l / 16, s = l % 16) receives
// X[kb + 8 q + e][mb + s], e = 0..7 (two ds_read_b64_tr_b16 of 4 rows each;
// within a 16-lane group output lane j, element e comes from source lane
// 4 e + j / 4, element j % 4, so source lane s points at row kb + 8 q + s / 4,
// columns mb + 4 (s % 4) .. + 3).
template <int D>
__device__ inline bf16x8 tile_op_rows16(const __bf16 *X, int kb, int mb) {
  const int lane = threadIdx.x % kWave;
  const int q = lane / 16, s = lane % 16;
  const int row = kb + 8 * q + s / 4;
  const int col = mb + 4 * (s % 4);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(const lds_short *)(X + Swz<__bf16, D>::off(row, col)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(const lds_short *)(X + Swz<__bf16, D>::off(row + 4, col)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

// bf16 tiles addressed from per-lane byte offsets.  Rows that differ by a
// multiple of 16 share f, and XOR acts on the chunk bits of an offset only
// (below the row bits, above the bytes within a chunk), so the offset of
// (row + 16 m, chunk ^ x) is 16 m * D * 2 + (offset of (row, chunk)) ^ 16 x:
// one base per lane serves every slice of a tile, the slice reached with a
// single XOR and the row block folded into the instruction's immediate.
//
// Base of the k-contiguous operand reads (tile_op at row `row`, column
// 8 hf): lane offset of (row, chunk hf).
template <int D>
__device__ inline unsigned op_base_bytes(int row, int hf) {
  return (unsigned)(row * D * 2 + ((hf ^ Swz<__bf16, D>::f(row)) * 16));
}
// tile_op<bf16, D>(X, row + 32 m, 8 hf + 16 ks) given base = op_base_bytes.
template <int D>
__device__ inline bf16x8 tile_op_x(const __bf16 *X, unsigned base, int m, int ks) {
  const char *p = reinterpret_cast<const char *>(X) + m * 32 * D * 2;
  return *reinterpret_cast<const bf16x8 *>(p + (base ^ (unsigned)(32 * ks)));
}
// Bases of the transposed reads of tile_op_rows (rows kb .. kb + 15 with
// kb a multiple of 16, columns from 0): the lane's first and second
// (4 rows further) read.
template <int D>
__device__ inline void rows_base_bytes(unsigned &a, unsigned &b) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, s = lane % 16;
  const int row = 8 * (g / 2) + s / 4;
  const int col = 16 * (g % 2) + 4 * (s % 4);
  a = (unsigned)(Swz<__bf16, D>::off(row, col) * 2);
  b = (unsigned)(Swz<__bf16, D>::off(row + 4, col) * 2);
}
// tile_op_rows<bf16, D>(X, kb, 32 dt) given the bases (kb a multiple of 16).
template <int D>
__device__ inline bf16x8 tile_op_rows_x(const __bf16 *X, unsigned a, unsigned b, int kb, int dt) {
  const char *p = reinterpret_cast<const char *>(X) + kb * D * 2;
  const unsigned x = (unsigned)(64 * dt);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(const lds_short *)(p + (a ^ x)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(const lds_short *)(p + (b ^ x)));
  const v8i16 ab = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

template <typename T>
__device__ inline typename Mfma<T>::Op lds_op(const T *p) {
  if constexpr (sizeof(T) == 2)
    return *reinterpret_cast<const bf16x8 *>(p);
  else
    return *p;
}

// E consecutive values of a D-tile register set, as one MFMA operand.
template <typename T>
__device__ inline typename Mfma<T>::Op regs_op(const f32x16 &acc, int r0) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)acc[r0 + e];
    return b;
  } else {
    return acc[r0];
  }
}

}  // namespace sas

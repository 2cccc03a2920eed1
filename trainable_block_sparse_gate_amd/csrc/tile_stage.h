// Staging of one 64-row x D tile: global -> registers -> LDS.
//
// A thread owns chunks of 4 consecutive rows x VEC consecutive columns
// (VEC = 16 bytes of the LDS element type T).  Loads are 16-byte (or 32-byte
// when an fp32 source is narrowed to bf16) and coalesced along the row; the
// chunk can then be written row-major (one 16-byte store per row) and/or
// transposed (VEC stores of 4 consecutive rows), which gives the
// column-contiguous operands the MFMA needs when a product contracts over
// the tile's rows.
#pragma once
#include "sas_device.h"

namespace sas {

template <typename T, int D, int NT>
struct Tile4 {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int DC = D / VEC;                 // column chunks per row group
  static constexpr int TOT = (kBlock / 4) * DC;      // chunks per tile
  static constexpr int CH = (TOT + NT - 1) / NT;     // chunks per thread
  static constexpr int ROW = D + VEC;                // row-major stride (elements)
  static constexpr int TROW = kBlock + VEC;          // transposed stride (elements)
  T v[CH][4][VEC];
};

template <typename TS, typename T>
__device__ inline void load_vec(T *dst, const TS *src, int n_elem) {
  if constexpr (sizeof(TS) == sizeof(T)) {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
  } else {  // fp32 source narrowed to bf16
    const float4 a = reinterpret_cast<const float4 *>(src)[0];
    const float4 b = reinterpret_cast<const float4 *>(src)[1];
    dst[0] = (T)a.x; dst[1] = (T)a.y; dst[2] = (T)a.z; dst[3] = (T)a.w;
    dst[4] = (T)b.x; dst[5] = (T)b.y; dst[6] = (T)b.z; dst[7] = (T)b.w;
  }
  (void)n_elem;
}

// rows >= nvalid are zero.  Row r of the tile starts at base + r * stride.
template <typename TS, typename T, int D, int NT>
__device__ inline void tile4_load(Tile4<T, D, NT> &st, const TS *base, long stride, int nvalid) {
  using F = Tile4<T, D, NT>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    const int kg = c / F::DC, dc = c % F::DC;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int row = 4 * kg + x;
      if ((F::TOT % NT == 0 || c < F::TOT) && row < nvalid) {
        load_vec<TS, T>(st.v[it][x], base + row * stride + dc * F::VEC, F::VEC);
      } else {
#pragma unroll
        for (int e = 0; e < F::VEC; ++e) st.v[it][x][e] = T(0.f);
      }
    }
  }
}

template <typename T, int D, int NT>
__device__ inline void tile4_store_rm(const Tile4<T, D, NT> &st, T *lds) {
  using F = Tile4<T, D, NT>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    if (F::TOT % NT != 0 && c >= F::TOT) continue;
    const int kg = c / F::DC, dc = c % F::DC;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      *reinterpret_cast<uint4 *>(lds + (4 * kg + x) * F::ROW + dc * F::VEC) =
          *reinterpret_cast<const uint4 *>(st.v[it][x]);
  }
}

template <typename T, int D, int NT>
__device__ inline void tile4_store_tr(const Tile4<T, D, NT> &st, T *lds) {
  using F = Tile4<T, D, NT>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    if (F::TOT % NT != 0 && c >= F::TOT) continue;
    const int kg = c / F::DC, dc = c % F::DC;
#pragma unroll
    for (int e = 0; e < F::VEC; ++e) {
      T *dst = lds + (dc * F::VEC + e) * F::TROW + 4 * kg;
      if constexpr (sizeof(T) == 2) {
        bf16x4 w = {st.v[it][0][e], st.v[it][1][e], st.v[it][2][e], st.v[it][3][e]};
        *reinterpret_cast<bf16x4 *>(dst) = w;
      } else {
        *reinterpret_cast<float4 *>(dst) =
            make_float4(st.v[it][0][e], st.v[it][1][e], st.v[it][2][e], st.v[it][3][e]);
      }
    }
  }
}

// Row-major staging only: 16-byte chunks (VEC elements of T), a row of D
// elements is D / VEC chunks, consecutive threads take consecutive chunks.
template <typename T, int D, int NT, int PAD>
struct RowTile {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int DC = D / VEC;
  static constexpr int TOT = kBlock * DC;
  static constexpr int CH = (TOT + NT - 1) / NT;
  static constexpr int ROW = D + PAD;  // LDS row stride (elements)
  T v[CH][VEC];
};

template <typename TS, typename T, int D, int NT, int PAD>
__device__ inline void rowtile_load(RowTile<T, D, NT, PAD> &st, const TS *base, long stride,
                                    int nvalid) {
  using F = RowTile<T, D, NT, PAD>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    const int row = c / F::DC, dc = c % F::DC;
    if ((F::TOT % NT == 0 || c < F::TOT) && row < nvalid) {
      load_vec<TS, T>(st.v[it], base + row * stride + dc * F::VEC, F::VEC);
    } else {
#pragma unroll
      for (int e = 0; e < F::VEC; ++e) st.v[it][e] = T(0.f);
    }
  }
}

template <typename T, int D, int NT, int PAD>
__device__ inline void rowtile_store(const RowTile<T, D, NT, PAD> &st, T *lds) {
  using F = RowTile<T, D, NT, PAD>;
#pragma unroll
  for (int it = 0; it < F::CH; ++it) {
    const int c = threadIdx.x + it * NT;
    if (F::TOT % NT != 0 && c >= F::TOT) continue;
    const int row = c / F::DC, dc = c % F::DC;
    *reinterpret_cast<uint4 *>(lds + row * F::ROW + dc * F::VEC) =
        *reinterpret_cast<const uint4 *>(st.v[it]);
  }
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

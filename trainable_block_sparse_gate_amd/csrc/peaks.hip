// Measured peaks of the device, for the roofline figures the benchmark
// reports beside the datasheet peaks.  Not part of the SAS library: this
// builds into its own small shared library that only the benchmark loads.
//
//   sas_peak_mfma_bf16   every wave of a full grid issues back-to-back
//                        32x32x16 bf16 MFMAs on register operands, with
//                        eight independent accumulators so the matrix core
//                        never waits on a result;
//   sas_peak_mfma_bf16_data  the same on operands taken from a buffer of
//                        random values that change from one instruction to
//                        the next (the rate under real data's power draw);
//   sas_peak_read        a streaming read of a device buffer (16-byte loads,
//                        grid-stride or one contiguous chunk per workgroup,
//                        4 to 16 loads in flight per thread), folded into
//                        one word per thread so no load is dropped.
// Each returns the hipError_t of its launch; the caller times the stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == 12345.f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // never true; keeps the work
}

// The same MFMA loop on data: eight A and eight B operands per lane from a
// buffer of (random) bf16 values, B rotating over the chains each
// iteration, so consecutive instructions see different operands.  The
// matrix cores then draw the power real data makes them draw, and the chip
// may lower its clock for it; the loop above on near-constant operands
// does not show that.
__global__ __launch_bounds__(256) void mfma_data_kernel(const u32x4 *src, int n16, int iters,
                                                        float *sink) {
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    a[c] = __builtin_bit_cast(bf16x8, src[(c * 256 + threadIdx.x) % n16]);
    b[c] = __builtin_bit_cast(bf16x8, src[(c * 256 + threadIdx.x + n16 / 2) % n16]);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; it += kChains) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + j) % kChains], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == 12345.f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // never true; keeps the work
}

// Each workgroup streams its own contiguous chunk of the buffer, U 16-byte
// loads in flight per thread (consecutive threads on consecutive 16 bytes).
template <int U>
__global__ __launch_bounds__(256) void read_chunk_kernel(const uint4 *src, long n16,
                                                         unsigned *sink) {
  const long per_wg = (n16 + gridDim.x - 1) / gridDim.x;
  const long lo = (long)blockIdx.x * per_wg;
  const long hi = lo + per_wg < n16 ? lo + per_wg : n16;
  unsigned acc = 0;
  long i = lo + threadIdx.x;
  const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(s4 + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(long)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void read_kernel(const uint4 *src, long n16, unsigned *sink) {
  const long stride = (long)gridDim.x * blockDim.x;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(long)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// flops = grid_wgs * 4 waves * iters * kChains * 32*32*16*2.
int sas_peak_mfma_bf16(int grid_wgs, int iters, float *sink, void *stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid_wgs), dim3(256), 0, (hipStream_t)stream, iters,
                     sink);
  return (int)hipGetLastError();
}

int sas_peak_mfma_chains(void) { return kChains; }

// flops as above; iters a multiple of the chain count; src holds n_bytes
// (a multiple of 16, at least 32) of bf16 operands.
int sas_peak_mfma_bf16_data(int grid_wgs, int iters, const void *src, long n_bytes, float *sink,
                            void *stream) {
  if (iters % kChains != 0 || n_bytes < 32 || n_bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_data_kernel, dim3(grid_wgs), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4 *>(src), (int)(n_bytes / 16), iters, sink);
  return (int)hipGetLastError();
}

// Reads n_bytes (a multiple of 16) from src; sink holds grid_wgs * 256 words.
// mode 0: grid-stride, four loads in flight per thread; mode 1 / 2: one
// contiguous chunk per workgroup, 8 / 16 nontemporal loads in flight.
int sas_peak_read(const void *src, long n_bytes, int grid_wgs, unsigned *sink, void *stream,
                  int mode) {
  const uint4 *s = static_cast<const uint4 *>(src);
  if (mode == 1)
    hipLaunchKernelGGL(read_chunk_kernel<8>, dim3(grid_wgs), dim3(256), 0, (hipStream_t)stream,
                       s, n_bytes / 16, sink);
  else if (mode == 2)
    hipLaunchKernelGGL(read_chunk_kernel<16>, dim3(grid_wgs), dim3(256), 0, (hipStream_t)stream,
                       s, n_bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_kernel, dim3(grid_wgs), dim3(256), 0, (hipStream_t)stream, s,
                       n_bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"

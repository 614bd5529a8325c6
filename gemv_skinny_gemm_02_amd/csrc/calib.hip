// calib.hip -- measurement kernels: the read and MFMA rates a kernel on this
// device can reach, against which the linear's kernels are reported.  They
// compute nothing of the linear.
//
//  * read_kernel: the grid reads a buffer once with 16-byte non-temporal
//    loads, 8 per thread in flight (256 threads), each workgroup one
//    contiguous slice or the whole grid in one sweep, and folds the words into
//    one value that is stored only if it equals a constant no ordinary data
//    hits (so the loads stay live).
//  * mfma_kernel: every wave runs `iters` rounds of 8 independent
//    v_mfma_f32_32x32x16_bf16 chains on register operands, then stores one
//    value per thread only if it equals the same constant.  (Measured on
//    MI355X: this form with 8 chains and 2048 workgroups issues at 98 % of the
//    nominal bf16 rate; the 16x16x32 form needs 16 chains to pass 90 %.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace skg {
namespace {

constexpr unsigned kNever = 0x7fc0dead;   // a NaN pattern no fold of the data is expected to give

// SWEEP false: workgroup b reads the b-th contiguous slice.  SWEEP true: the
// whole grid sweeps the buffer together (piece t + j*T for thread t of T), so
// the addresses in flight stay in one moving window.
template <bool SWEEP>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, unsigned long long n16,
                                                   unsigned* sink) {
  constexpr int U = 8;
  unsigned long long b0, b1, step;
  if constexpr (SWEEP) {
    b0 = (unsigned long long)blockIdx.x * 256;
    b1 = n16;
    step = (unsigned long long)gridDim.x * 256;
  } else {
    const unsigned long long per = (n16 + gridDim.x - 1) / gridDim.x;
    b0 = (unsigned long long)blockIdx.x * per;
    b1 = b0 + per < n16 ? b0 + per : n16;
    step = 256;
  }
  unsigned acc = 0;
  for (unsigned long long i = b0 + threadIdx.x; i < b1; i += step * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned long long j = i + (unsigned long long)u * step;
      v[u] = j < b1 ? load_nt(p + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == kNever) sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, unsigned* sink) {
  constexpr int C = 8;
  const unsigned t = threadIdx.x + 1u;
  u32x4 av = u32x4{t * 0x3f803f80u, t ^ 0x3f003f00u, t, t * 3u};
  u32x4 bv = u32x4{t ^ 0x3e803e80u, t * 5u, t + 7u, t * 0x00010001u};
  f32x16 acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  const bf16x8 A = __builtin_bit_cast(bf16x8, av), B = __builtin_bit_cast(bf16x8, bv);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) s += acc[c][0] + acc[c][5] + acc[c][15];
  if (__float_as_uint(s) == kNever) sink[threadIdx.x] = __float_as_uint(s);
}

}  // namespace

hipError_t launch_calib_read(const void* buf, unsigned long long n16, int grid, int sweep, unsigned* sink,
                             hipStream_t s) {
  if (sweep)
    hipLaunchKernelGGL(read_kernel<true>, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf), n16, sink);
  else
    hipLaunchKernelGGL(read_kernel<false>, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int grid, int iters, unsigned* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace skg



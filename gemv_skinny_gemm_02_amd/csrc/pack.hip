// pack.hip -- writes the fragment-packed weight layout, once per weight.
#include "kernels.hpp"

namespace skg {

namespace {

// One thread per 16 bytes of the packed weight.  Unit i is lane l = i % 64 of
// load h = (i / 64) % 2 of block (c*G + g)*N16 + b = i / 128: row 16b + l%16
// of group g, bytes 128c + off .. +15 of that row, where off is what the LDS
// tile kernel's MFMA operand takes for lane slot q = l/16 and load h:
// 32q + 16h for an fp8 weight used with bf16 x (tensor scale), 64h + 16q
// otherwise.  Rows past N and bytes past the row are zero.
template <bool FP8T>
__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ W, char* __restrict__ Wp, int N,
                                                   int rowb, int G, int N16, unsigned long long units) {
  const unsigned long long i = (unsigned long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= units) return;
  const int l = (int)(i & 63), h = (int)((i >> 6) & 1);
  const unsigned long long blk = i >> 7;
  const int b = (int)(blk % N16);
  const unsigned long long cg = blk / N16;
  const int g = (int)(cg % G), c = (int)(cg / G);
  const int row = b * 16 + (l & 15), q = l >> 4;
  const int byte = c * 128 + (FP8T ? q * 32 + h * 16 : h * 64 + q * 16);
  u32x4 v = u32x4{0, 0, 0, 0};
  if (row < N && byte < rowb) v = *reinterpret_cast<const u32x4*>(W + ((size_t)g * N + row) * rowb + byte);
  *reinterpret_cast<u32x4*>(Wp + i * 16) = v;
}

}  // namespace

hipError_t launch_pack(int op, const void* W, void* Wp, int N, int K, hipStream_t s) {
  const int G = op_groups(op), rowb = K * op_w_bytes(op), N16 = (N + 15) / 16;
  const unsigned long long units = packed_weight_bytes(op, N, K) / 16;
  const unsigned long long blocks = (units + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const char* w = static_cast<const char*>(W);
  char* p = static_cast<char*>(Wp);
  if (op_base(op) == OP_FP8T)
    hipLaunchKernelGGL(pack_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, w, p, N, rowb, G, N16, units);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, w, p, N, rowb, G, N16, units);
  return hipGetLastError();
}

}  // namespace skg

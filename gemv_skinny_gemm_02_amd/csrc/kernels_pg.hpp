// kernels_pg.hpp -- the weight stream over a fragment-packed bf16 weight
// (pg_kernel): the smallest weights and rows, where the packed tiles, which
// take whole 16-row blocks, leave most CUs idle.
//
// A workgroup owns RW (2, 4 or 8) weight rows of one 16-row block and KS
// waves split K.  In the packed layout the 16-byte pieces of one place (half
// h, lane slot q) of a 128-byte chunk sit row after row, 16 bytes apart, so
// the RW rows' pieces of a place are 16*RW contiguous bytes.  One wave load
// takes, for CPI = 8/RW chunks, all 8 places of each (lane l reads row l%RW,
// place (l/RW)%8 of chunk l/(8*RW) of its group of chunks): every byte of the
// segments it touches is used.  The rest of each 128-byte line belongs to the
// neighbouring row groups, which run on the same XCD so that the line is
// fetched into one L2 once.  Each lane multiplies its 8 bf16 with the matching
// 8 K of every x row (v_dot2c); the lanes of a row add their sums by a fixed
// butterfly, the waves in wave order through LDS, so the result is
// reproducible.
#pragma once

#include "kernels.hpp"

namespace skg {

template <int OP, int MT>
struct PgRound {
  u32x4 w[op_groups(OP)];
  u32x4 x[MT];
};

template <int OP, int MT, int RW, int KS, int P>
__global__ __launch_bounds__(64 * KS) void pg_kernel(const Args a) {
  constexpr int BO = op_base(OP);
  constexpr int G = op_groups(OP);
  static_assert(op_packed(OP) && (BO == OP_BF16 || BO == OP_GATED), "packed bf16 weights only");

  constexpr int CPI = 8 / RW;                  // chunks per wave load
  static_assert(RW == 2 || RW == 4 || RW == 8, "2, 4 or 8 rows per workgroup");

  __shared__ float red[KS][G][MT][RW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = a.M, N = a.N, K = a.K;
  // Row groups by XCD: workgroups are handed to the 8 XCDs in turn, so
  // workgroup b runs on XCD b % 8; give each XCD a contiguous run of row
  // groups, so that the two groups sharing a 128-byte line of a place are read
  // through the same L2.  Surplus workgroups of the rounded-up grid return.
  const int groups = (N + RW - 1) / RW, per_xcd = (groups + 7) >> 3;
  const int grp = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (grp >= groups) return;
  const int n0 = grp * RW;
  const int r = lane % RW, place = (lane / RW) & 7, cq = lane / (8 * RW);
  const int h = place >> 2, q = place & 3;
  const int n = min(n0 + r, N - 1);            // rows past N read row N-1; never stored
  const int N16 = (N + 15) >> 4;
  const size_t cstride = (size_t)G * N16 * 2048;
  const int NC = (K + 63) >> 6;                // 128-byte chunks of a row (64 K each)
  const int cgroups = (NC + CPI - 1) / CPI;   // groups of CPI chunks

  const char* wb[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    wb[g] = static_cast<const char*>(a.w) + ((size_t)g * N16 + (n >> 4)) * 2048 + h * 1024 + q * 256 + (n & 15) * 16;
  const char* xr[MT];                          // rows past M re-read row M-1: finite, never stored
#pragma unroll
  for (int m = 0; m < MT; ++m) xr[m] = static_cast<const char*>(a.x) + (size_t)min(m, M - 1) * K * 2;

  float acc[G][MT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[g][m] = 0.0f;

  // this lane's chunk in round j, and the first K of its piece there
  auto chunk_of = [&](int j) { return CPI * (j * KS + wave) + cq; };
  using Round = PgRound<OP, MT>;
  auto load = [&](Round& b, int j) {
    const int c = min(chunk_of(j), NC - 1);
    const int k0 = min(c * 64 + h * 32 + q * 8, K - 8);
#pragma unroll
    for (int g = 0; g < G; ++g) b.w[g] = *reinterpret_cast<const u32x4*>(wb[g] + (size_t)c * cstride);
#pragma unroll
    for (int m = 0; m < MT; ++m) b.x[m] = *reinterpret_cast<const u32x4*>(xr[m] + (size_t)k0 * 2);
  };
  auto compute = [&](const Round& b0, int j, auto tail) {
    Round b = b0;
    if constexpr (decltype(tail)::value) {     // pieces past K (or a missing second chunk) add nothing
      const int c = chunk_of(j);
      const bool dead = c >= NC || c * 64 + h * 32 + q * 8 >= K;
#pragma unroll
      for (int g = 0; g < G; ++g) b.w[g] = dead ? u32x4{0, 0, 0, 0} : b.w[g];
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float s = acc[g][m];
#pragma unroll
        for (int d = 0; d < 4; ++d) s = dot2(b.x[m][d], b.w[g][d], s);
        acc[g][m] = s;
      }
  };
  const int rounds = cgroups > wave ? (cgroups - wave + KS - 1) / KS : 0;
  Round buf[P];
  ring_pipeline<P>(buf, rounds, load, compute);

  // the 64/RW lanes of a row (lane bits above those of RW) add their sums in
  // a fixed order
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[g][m];
#pragma unroll
      for (int b = RW; b < 64; b <<= 1) v += __shfl_xor(v, b);
      acc[g][m] = v;
    }
  if (lane < RW) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave][g][m][lane] = acc[g][m];
  }
  __syncthreads();
  unsigned short* y = static_cast<unsigned short*>(a.y);
  for (int o = threadIdx.x; o < RW * MT; o += 64 * KS) {
    const int m = o / RW, rr = o % RW;
    if (m >= M || n0 + rr >= N) continue;
    float v = 0.0f, u = 0.0f;
#pragma unroll
    for (int w = 0; w < KS; ++w) {
      v += red[w][0][m][rr];
      if constexpr (G == 2) u += red[w][G - 1][m][rr];
    }
    if constexpr (BO == OP_GATED) v = silu_f32(v) * u;
    y[(size_t)m * N + n0 + rr] = f32_to_bf16(v);
  }
}

template <int OP, int MT, int RW, int KS, int P>
hipError_t launch_pg(const Args& a, hipStream_t s) {
  const unsigned grid = 8u * (unsigned)((((a.N + RW - 1) / RW) + 7) / 8);
  hipLaunchKernelGGL((pg_kernel<OP, MT, RW, KS, P>), dim3(grid), dim3(64 * KS), 0, s, a);
  return hipGetLastError();
}

template <int OP, int MT, int RW, int KS, int P>
constexpr LaunchFn pg_fn() {
  if constexpr (pg_valid(OP, MT, RW, KS, P)) return &launch_pg<OP, MT, RW, KS, P>;
  else return nullptr;
}

// Launch tables of the packed weight stream (ops_pg.hip): per SKG_PG variant,
// one entry per rows bucket of kGemvMT up to kPgMaxM.
template <int OP> const GemvRow* pg_table();
template <> const GemvRow* pg_table<OP_PACKED + OP_BF16>();
template <> const GemvRow* pg_table<OP_PACKED + OP_GATED>();

}  // namespace skg

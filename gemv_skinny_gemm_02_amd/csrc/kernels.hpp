// kernels.hpp -- gfx950 (CDNA4) kernels of the skinny decode linear
//   y[M, N] = x[M, K] . W[N, K]^T
// in its four forms (bf16; fused gate/up silu(x Wg^T) * (x Wu^T); fp8 weight
// with one per-tensor scale; A8W8 with per-row/128-K-group activation scales
// and 128 x 128 weight block scales).
//
// Two kernel families:
//  * gemv_kernel -- M <= 16.  The problem is a weight stream: every byte of W
//    is read once from HBM and used for only M multiply-adds, so the kernel is
//    built around 16-byte coalesced, non-temporal weight loads (one 1 KiB wave
//    load per row per round), bf16 pair dot products (v_dot2c_f32_bf16) on the
//    VALU, and N split across workgroups so that even M = 1 puts several
//    workgroups on each of the 256 CUs (N-split at small M: DeepSeek-V4-flash
//    decode round 3, "Retained change 1").  The K dimension is split across the
//    lanes of a wave and across KS waves of the workgroup; the partial sums are
//    combined in a fixed order (cross-lane reduce-scatter, then LDS), so a call
//    is bit-reproducible.  No split-K across workgroups and no atomics (the
//    pages' tuned decode rows use splitK=0: same section, "Retained change 2").
//  * tile_kernel -- M >= 16.  A dense contraction on the matrix cores:
//    v_mfma_f32_16x16x32_bf16 (bf16, gated, and fp8 weights converted to bf16
//    in registers) or v_mfma_f32_16x16x32_fp8_fp8 (A8W8), W fragments as the
//    A operand (16 rows of N) and x fragments as the B operand (16 rows of M).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "variants.hpp"

namespace skg {

struct Args {
  const void* x;
  const void* w;
  const float* s0;  // fp8 tensor: w_scale[1]; a8w8: x_scales[M, kb]
  const float* s1;  // a8w8 (both forms): w_scales[ceil(N/128), kb]
  void* y;
  int M, N, K;
  int kb;           // ceil(K / 128): scale groups along K
  float* ws;        // split-K partials [S][G][M][N] fp32 (tlds variants with S > 1)
  unsigned* cnt;    // split-K arrival counters, one per output tile, zero between calls
  float* xs_out;    // a8w8 with x quantised here: the x scales [M, kb] it computes, or NULL
  int split_wait;   // split-K tiles: 1 when a split's workgroup may wait (bounded) for the
                    // tile's other splits, i.e. the whole grid fits on the device at once;
                    // set by the launch from 0, kept at -1 (never wait) when waits are off
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two e4m3fn bytes (low pair if hi == false, high pair otherwise) of a dword
// -> two bf16 in one dword.  Every e4m3fn value is exactly a bf16 value; the
// scale operand is 1.0, so the conversion is exact.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned v) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<unsigned short>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

// Whether y takes 8-byte stores of four outputs: rows of a multiple of 4
// outputs and an 8-byte aligned base (y itself needs only 2-byte alignment).
__device__ __forceinline__ bool y_vec4(const void* y, int N) {
  return (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
}

// y[row, n .. n+3] = bf16(v[0 .. 3]) for n a multiple of 4, each value rounded
// once: a single 8-byte store when yvec and the row holds all four (a tile's
// output fragment gives each lane four consecutive outputs of one row), else
// one 2-byte store per output inside the row.
__device__ __forceinline__ void store_y4(unsigned short* y, size_t row, int n, int N, bool yvec, const float (&v)[4]) {
  if (yvec && n + 3 < N) {
    uint2 pk;
    pk.x = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
    pk.y = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(y + row * N + n) = pk;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) y[row * N + n + e] = f32_to_bf16(v[e]);
  }
}

__device__ __forceinline__ float silu_f32(float g) {
  // g * sigmoid(g) = g / (1 + e^-g); for very negative g, e^-g overflows to
  // +inf and the quotient is -0, the correctly signed limit.
  return g / (1.0f + __expf(-g));
}

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Split-K tile state (3 words of the workspace counters, laid out as
// kSplitLines describes).  Word 0 counts arrivals over all launches: each
// launch adds exactly 8 to it (its S arrivals, then 8 - S from the last to
// arrive), so it is a multiple of 8 between launches, a launch's epoch is the
// value over 8, and a workgroup's arrival rank is the value's low 3 bits.
// Words 1 and 2 hold the slice claims of even and odd epochs; the last to
// arrive clears the other one for the next launch.  Nothing needs a reset.
__device__ __forceinline__ unsigned* split_tile_state(unsigned* cnt, unsigned tile) {
  return cnt + (tile % kSplitLines) * 32 + (tile / kSplitLines) * 3;
}

// Arrive at a split-K tile (one thread of the workgroup, after its partials
// are stored and complete): returns the tile's arrival word before this
// arrival.  The last of the S arrivals also makes the launch's total 8 and
// clears the claim word of the next epoch.
template <int S>
__device__ __forceinline__ unsigned split_arrive(unsigned* st) {
  const unsigned old = __hip_atomic_fetch_add(st, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old & 7u) == (unsigned)(S - 1)) {
    if constexpr (S < 8) __hip_atomic_fetch_add(st, (unsigned)(8 - S), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st + 1 + (((old >> 3) + 1u) & 1u), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return old;
}

// The longest a split-K workgroup waits for the other splits of its tile, in
// ticks of the 100 MHz real-time counter (20 us): past it the last split to
// arrive adds the slice instead.
constexpr unsigned long long kSplitWaitTicks = 2000;

// Workgroups of `kernel` (block threads, smem bytes of dynamic LDS) that the
// current device holds at once: its occupancy per CU times the CUs, or 0 when
// the runtime cannot tell.  A host query, no stream work.
inline unsigned long long resident_workgroups(const void* kernel, int block, size_t smem) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, smem) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return (unsigned long long)cus * (unsigned long long)per_cu;
}

// Buffer resource over [p, p + bytes) for raw buffer loads/stores; cache
// policy bit 4 (sc1) makes an access device-coherent across the XCDs' L2s.
constexpr int kCoherent = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// ------------------------------------------- fixed-order cross-lane reduction
// Reduce-scatter of VC per-lane values over the 64 lanes of a wave.  While the
// count is even, each xor-exchange with mask S halves it: a lane keeps the
// half selected by its lane bit S and adds the partner's copy of that half.
// Once the count is odd, the remaining masks do full butterflies.  Every lane
// ends with VF totals; `off` is the index of its first one.  The order of the
// additions is fixed by the lane bits, so the result is reproducible.
template <int VC, int S>
struct ReduceScatter {
  static constexpr bool kHalve = (VC % 2 == 0) && VC > 1;
  static constexpr int kNext = kHalve ? VC / 2 : VC;
  using Rest = ReduceScatter<kNext, S / 2>;
  static constexpr int VF = Rest::VF;
  static constexpr int kBflyMask = (kHalve ? 0 : S) | Rest::kBflyMask;
  __device__ __forceinline__ static void run(float* v, int lane, int& off) {
    if constexpr (kHalve) {
      constexpr int H = VC / 2;
      const bool up = (lane & S) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, S);
      }
      off += up ? H : 0;
    } else {
#pragma unroll
      for (int i = 0; i < VC; ++i) v[i] += __shfl_xor(v[i], S);
    }
    Rest::run(v, lane, off);
  }
};
template <int VC>
struct ReduceScatter<VC, 0> {
  static constexpr int VF = VC;
  static constexpr int kBflyMask = 0;
  __device__ __forceinline__ static void run(float*, int, int&) {}
};

// ======================================================== load pipeline
// Both kernels stream their operands through a ring of P register buffers:
// buffer p holds the loads of round j0 + p.  Round j is consumed P rounds
// after its loads were issued, so P rounds of loads stay in flight while the
// oldest one is used (vector loads complete in issue order, so waiting for the
// oldest leaves the younger ones outstanding).  `rounds` is wave-uniform; the
// load functor clamps a round index past the wave's last to a valid address.
// The steady-state loop only sees rounds that are full for every lane
// (compute's second argument false); the drain handles the last P..2P-1
// rounds, where the final one may reach past K (true).
template <int P, class Buf, class LoadF, class ComputeF>
__device__ __forceinline__ void ring_pipeline(Buf (&buf)[P], int rounds, LoadF&& load, ComputeF&& compute) {
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  // unconditional prologue (load clamps its index): keeps the wait counts exact
#pragma unroll
  for (int p = 0; p < P; ++p) load(buf[p], p);
  int j0 = 0;
  for (; j0 + 2 * P <= rounds; j0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      compute(buf[p], j0 + p, Full{});
      // keep each round's loads right after the compute that frees its
      // buffer: the scheduler would otherwise sink them and shrink the ring
      __builtin_amdgcn_sched_barrier(0);
      load(buf[p], j0 + P + p);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = j0 + p;
    if (j < rounds) {
      compute(buf[p], j, Tail{});
      if (j + P < rounds) load(buf[p], j + P);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = j0 + P + p;
    if (j < rounds) compute(buf[p], j, Tail{});
  }
}

// =================================================================== GEMV
// One workgroup = 4 waves = (4/KS) row groups x KS K-slices.  Wave (rg, ks)
// owns rows n0 + rg*R + [0, R) (and the matching up rows N + ... for the gated
// form) and the K-chunks ((j*KS + ks)*64 + lane) for rounds j = 0, 1, ...; a
// chunk is one 16-byte load of a W row (8 bf16 or 16 fp8 K-elements).  P
// rounds are in flight per wave.
template <int OP, int MT, int R>
struct GemvRound {
  u32x4 w[op_groups(OP)][R];
  u32x4 x[MT][op_xd(OP) / 4];
};

template <int OP, int MT, int R, int KS, int P>
__global__ __launch_bounds__(256) void gemv_kernel(const Args a) {
  constexpr int G = op_groups(OP);
  constexpr int V = MT * R * G;
  constexpr int RG = 4 / KS;
  constexpr int RPW = RG * R;
  constexpr int KC = op_kc(OP);
  constexpr int XD = op_xd(OP);       // dwords of one x row per chunk
  constexpr int XV = XD / 4;          // 16-byte x loads per chunk per row
  constexpr int WB = op_w_bytes(OP);
  constexpr int XB = op_x_bytes(OP);

  __shared__ float red[4][V];
  extern __shared__ float sc[];      // A8W8: xs rows [MT][kb] then ws row [kb]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int rg = wave / KS, ks = wave - (wave / KS) * KS;
  const int M = a.M, N = a.N, K = a.K;
  const int wg_row0 = blockIdx.x * RPW;
  const int n0 = wg_row0 + rg * R;
  const int C = K / KC;               // chunks per row (K % KC == 0)

  const u32x4* wp[G][R];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(n0 + r, N - 1);   // rows past N load row N-1; never stored
      wp[g][r] = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.w) +
                                                (size_t)(n + g * N) * K * WB);
    }
  const u32x4* xp[MT];                // rows past M re-read row M-1: finite data, never stored
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xp[m] = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) +
                                           (size_t)(m < M ? m : M - 1) * K * XB);

  float* xs_l = sc;
  float* ws_l = sc + MT * a.kb;
  if constexpr (OP == OP_A8W8) {
    const int kb = a.kb;
    const int nblk = wg_row0 >> 7;    // RPW divides 128: one weight block row
    for (int i = threadIdx.x; i < MT * kb; i += 256) {
      const int m = i / kb;
      xs_l[i] = m < M ? a.s0[(size_t)m * kb + (i - m * kb)] : 0.0f;
    }
    for (int i = threadIdx.x; i < kb; i += 256) ws_l[i] = a.s1[(size_t)nblk * kb + i];
    __syncthreads();
  }

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.0f;

  using Round = GemvRound<OP, MT, R>;
  auto load = [&](Round& b, int j) {
    const int c = (j * KS + ks) * 64 + lane;
    const int cc = c < C ? c : C - 1;     // lanes past K re-read a valid chunk; zeroed when used
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) b.w[g][r] = load_nt(wp[g][r] + cc);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < XV; ++q) b.x[m][q] = xp[m][(size_t)cc * XV + q];
  };

  auto compute = [&](const Round& b0, int j, auto tail) {
    const int c = (j * KS + ks) * 64 + lane;
    Round b;
    if constexpr (decltype(tail)::value) {     // lanes past K contribute nothing
      const bool dead = c >= C;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < R; ++r) b.w[g][r] = dead ? u32x4{0, 0, 0, 0} : b0.w[g][r];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < XV; ++q) b.x[m][q] = b0.x[m][q];
    } else {
      b = b0;
    }
    if constexpr (OP == OP_BF16 || OP == OP_GATED) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float s = acc[(g * MT + m) * R + r];
#pragma unroll
            for (int d = 0; d < 4; ++d) s = dot2(b.x[m][0][d], b.w[g][r][d], s);
            acc[(g * MT + m) * R + r] = s;
          }
    } else if constexpr (OP == OP_FP8T) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        unsigned wb[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wb[2 * d] = fp8x2_to_bf16x2<false>(b.w[0][r][d]);
          wb[2 * d + 1] = fp8x2_to_bf16x2<true>(b.w[0][r][d]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float s = acc[m * R + r];
#pragma unroll
          for (int d = 0; d < 8; ++d) s = dot2(b.x[m][d >> 2][d & 3], wb[d], s);
          acc[m * R + r] = s;
        }
      }
    } else {  // OP_A8W8
      const int grp = (c < C ? c : C - 1) >> 3;   // 16 K per chunk, 128 K per group
      const float sw = ws_l[grp];
      unsigned xb[MT][8];
      float sxw[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        sxw[m] = xs_l[m * a.kb + grp] * sw;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          xb[m][2 * d] = fp8x2_to_bf16x2<false>(b.x[m][0][d]);
          xb[m][2 * d + 1] = fp8x2_to_bf16x2<true>(b.x[m][0][d]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        unsigned wb[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wb[2 * d] = fp8x2_to_bf16x2<false>(b.w[0][r][d]);
          wb[2 * d + 1] = fp8x2_to_bf16x2<true>(b.w[0][r][d]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float p = 0.0f;
#pragma unroll
          for (int d = 0; d < 8; ++d) p = dot2(xb[m][d], wb[d], p);
          acc[m * R + r] = __builtin_fmaf(p, sxw[m], acc[m * R + r]);
        }
      }
    }
  };

  const int first = ks * 64;
  const int rounds = C > first ? (C - first + 64 * KS - 1) / (64 * KS) : 0;
  Round buf[P];
  ring_pipeline<P>(buf, rounds, load, compute);

  // ---- combine: lanes (fixed reduce-scatter), then K-slices (LDS, in order)
  using RS = ReduceScatter<V, 32>;
  int off = 0;
  RS::run(acc, lane, off);
  if ((lane & RS::kBflyMask) == 0) {
#pragma unroll
    for (int t = 0; t < RS::VF; ++t) red[wave][off + t] = acc[t];
  }
  __syncthreads();

  float scale = 1.0f;
  if constexpr (OP == OP_FP8T) scale = a.s0[0];
  unsigned short* y = static_cast<unsigned short*>(a.y);
  for (int o = threadIdx.x; o < RG * MT * R; o += 256) {
    const int org = o / (MT * R);
    const int rem = o - org * (MT * R);
    const int m = rem / R, r = rem - (rem / R) * R;
    const int n = wg_row0 + org * R + r;
    if (m >= M || n >= N) continue;
    float v = 0.0f, u = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < KS; ++k2) {
      v += red[org * KS + k2][m * R + r];
      if constexpr (G == 2) u += red[org * KS + k2][(MT + m) * R + r];
    }
    if constexpr (OP == OP_GATED) v = silu_f32(v) * u;
    if constexpr (OP == OP_FP8T) v *= scale;
    y[(size_t)m * N + n] = f32_to_bf16(v);
  }
}

// =================================================================== TILE
// One workgroup = 4 waves = (4/KS) row groups x KS K-slices.  Wave (ng, ks)
// owns W rows nb + [0, 16*FN) (plus the up rows for the gated form) and the M
// rows m_base + [0, 16*FM) of this launch row, and the K-units (j*KS + ks) for
// rounds j; P units are in flight per wave.  A K-unit is 32 K (bf16), 64 K
// (fp8 weight with bf16 x) or one 128-K scale group (A8W8).
//
// Fragment layout (16x16x32 MFMA): lane l supplies, for its row l%16 of the
// A operand (W) and its column l%16 of the B operand (x), the 8 K-elements of
// slot l/16.  Which actual K-indices fill a slot does not matter as long as A
// and B agree; the loads below choose them so that the four lanes of one row
// read 64 contiguous bytes per instruction.  The 16x16 fp32 result sits with
// C[4*(l/16) + e][l%16] in lane l, register e.
//
// x rows past M read row M-1 and lanes past K read a valid K position: both
// give finite data.  The weight of a lane past K is zeroed before use, so it
// adds nothing; output columns past M are never stored.  Fragments wholly past
// M are loaded (clamped) but not multiplied.
template <int OP>
struct TileKUnit {
  static constexpr int value = OP == OP_A8W8 ? 128 : (OP == OP_FP8T ? 64 : 32);
};
template <int OP, int FM, int FN>
struct TileRound {
  static constexpr int WV = OP == OP_A8W8 ? 2 : 1;  // 16-byte W loads per fragment
  static constexpr int XVN = OP == OP_BF16 || OP == OP_GATED ? 1 : 2;
  u32x4 w[op_groups(OP)][FN][WV];
  u32x4 x[FM][XVN];
  float sx[OP == OP_A8W8 ? FM : 1];
  float sw[OP == OP_A8W8 ? FN : 1];
};

template <int OP, int FM, int FN, int KS, int P>
__global__ __launch_bounds__(256) void tile_kernel(const Args a) {
  constexpr int G = op_groups(OP);
  constexpr int NG = 4 / KS;
  constexpr int RPW = NG * FN * 16;
  constexpr int KU = TileKUnit<OP>::value;
  constexpr int WB = op_w_bytes(OP);
  constexpr int XB = op_x_bytes(OP);
  constexpr int NACC = G * FN * FM;
  using Round = TileRound<OP, FM, FN>;

  extern __shared__ float red[];     // KS > 1: [NG][KS-1][NACC*4][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int ng = wave / KS, ks = wave - (wave / KS) * KS;
  const int lr = lane & 15, lq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int m_base = blockIdx.y * 16 * FM;
  const int nb = blockIdx.x * RPW + ng * FN * 16;
  const int NU = (K + KU - 1) / KU;
  const int kb = a.kb;
  const int fm_live = min(FM, (M - m_base + 15) / 16);   // fragments holding rows < M

  const char* wrow[G][FN];
  int wblk[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int n = min(nb + f * 16 + lr, N - 1);
#pragma unroll
    for (int g = 0; g < G; ++g)
      wrow[g][f] = static_cast<const char*>(a.w) + (size_t)(n + g * N) * K * WB;
    wblk[f] = min(nb + f * 16, N - 1) >> 7;
  }
  const char* xrow[FM];
  int xm[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    xm[j] = min(m_base + j * 16 + lr, M - 1);
    xrow[j] = static_cast<const char*>(a.x) + (size_t)xm[j] * K * XB;
  }

  f32x4 acc[G][FN][FM];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[g][f][j] = f32x4{0, 0, 0, 0};

  // K position of this lane's first element in unit `unit` for load h.
  auto lane_k = [&](int unit, int h) {
    if constexpr (OP == OP_A8W8) return unit * KU + h * 64 + lq * 16;
    else if constexpr (OP == OP_FP8T) return unit * KU + lq * 16;
    else return unit * KU + lq * 8;
  };
  constexpr int LK = OP == OP_BF16 || OP == OP_GATED ? 8 : 16;   // K-elements per 16-byte W load

  auto load = [&](Round& b, int j) {
    const int unit = min(j * KS + ks, NU - 1);
#pragma unroll
    for (int h = 0; h < Round::WV; ++h) {
      const int k = min(lane_k(unit, h), K - LK);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
          b.w[g][f][h] = load_nt(reinterpret_cast<const u32x4*>(wrow[g][f] + (size_t)k * WB));
    }
    // every load is unconditional (rows past M are clamped) so the wait
    // counts stay exact and the ring keeps P units in flight
#pragma unroll
    for (int jj = 0; jj < FM; ++jj) {
      if constexpr (OP == OP_BF16 || OP == OP_GATED) {
        const int k = min(lane_k(unit, 0), K - 8);
        b.x[jj][0] = *reinterpret_cast<const u32x4*>(xrow[jj] + (size_t)k * 2);
      } else if constexpr (OP == OP_FP8T) {
        const int k = min(lane_k(unit, 0), K - 16);
        b.x[jj][0] = *reinterpret_cast<const u32x4*>(xrow[jj] + (size_t)k * 2);
        b.x[jj][1] = *reinterpret_cast<const u32x4*>(xrow[jj] + (size_t)(k + 8) * 2);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = min(lane_k(unit, h), K - 16);
          b.x[jj][h] = *reinterpret_cast<const u32x4*>(xrow[jj] + k);
        }
      }
    }
    if constexpr (OP == OP_A8W8) {
#pragma unroll
      for (int jj = 0; jj < FM; ++jj) b.sx[jj] = a.s0[(size_t)xm[jj] * kb + unit];
#pragma unroll
      for (int f = 0; f < FN; ++f) b.sw[f] = a.s1[(size_t)wblk[f] * kb + unit];
    }
  };

  auto compute = [&](const Round& b0, int j, auto tail) {
    const int unit = j * KS + ks;
    Round b = b0;
    if constexpr (decltype(tail)::value) {        // lanes past K contribute nothing
#pragma unroll
      for (int h = 0; h < Round::WV; ++h) {
        const bool dead = lane_k(unit, h) >= K;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f) b.w[g][f][h] = dead ? u32x4{0, 0, 0, 0} : b0.w[g][f][h];
      }
    }
    if constexpr (OP == OP_BF16 || OP == OP_GATED) {
#pragma unroll
      for (int jj = 0; jj < FM; ++jj) {
        if (jj < fm_live) {
          const bf16x8 B = __builtin_bit_cast(bf16x8, b.x[jj][0]);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int f = 0; f < FN; ++f)
              acc[g][f][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.w[g][f][0]), B,
                                                                      acc[g][f][jj], 0, 0, 0);
        }
      }
    } else if constexpr (OP == OP_FP8T) {
      // 16 fp8 of a W row per lane: K = unit*64 + lq*16 + [0, 16), two MFMAs.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          u32x4 wb;
          wb[0] = fp8x2_to_bf16x2<false>(b.w[0][f][0][2 * h]);
          wb[1] = fp8x2_to_bf16x2<true>(b.w[0][f][0][2 * h]);
          wb[2] = fp8x2_to_bf16x2<false>(b.w[0][f][0][2 * h + 1]);
          wb[3] = fp8x2_to_bf16x2<true>(b.w[0][f][0][2 * h + 1]);
          const bf16x8 A = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
          for (int jj = 0; jj < FM; ++jj)
            if (jj < fm_live)
              acc[0][f][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, b.x[jj][h]),
                                                                      acc[0][f][jj], 0, 0, 0);
        }
      }
    } else {  // OP_A8W8: one 128-K scale group per unit, four fp8 MFMAs
#pragma unroll
      for (int f = 0; f < FN; ++f) {
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) {
          if (jj < fm_live) {
            f32x4 t = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int h = q >> 1, p = (q & 1) * 2;
              const long A = static_cast<long>((static_cast<unsigned long>(b.w[0][f][h][p + 1]) << 32) |
                                               b.w[0][f][h][p]);
              const long B = static_cast<long>((static_cast<unsigned long>(b.x[jj][h][p + 1]) << 32) |
                                               b.x[jj][h][p]);
              t = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(A, B, t, 0, 0, 0);
            }
            const float s = b.sx[jj] * b.sw[f];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[0][f][jj][e] = __builtin_fmaf(t[e], s, acc[0][f][jj][e]);
          }
        }
      }
    }
  };

  const int rounds = NU > ks ? (NU - ks + KS - 1) / KS : 0;
  Round buf[P];
  ring_pipeline<P>(buf, rounds, load, compute);

  // ---- combine the K-slices in order through LDS, then the epilogue
  if constexpr (KS > 1) {
    if (ks > 0) {
      float* dst = red + (size_t)((ng * (KS - 1) + ks - 1) * NACC * 4) * 64;
      int i = 0;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e, ++i) dst[i * 64 + lane] = acc[g][f][j][e];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int s = 1; s < KS; ++s) {
      const float* src = red + (size_t)((ng * (KS - 1) + s - 1) * NACC * 4) * 64;
      int i = 0;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e, ++i) acc[g][f][j][e] += src[i * 64 + lane];
    }
  }

  float scale = 1.0f;
  if constexpr (OP == OP_FP8T) scale = a.s0[0];
  unsigned short* y = static_cast<unsigned short*>(a.y);
  const bool yvec = y_vec4(a.y, N);
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m_base + j * 16 + lr;
      const int n = nb + f * 16 + lq * 4;
      if (m >= M || n >= N) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[0][f][j][e];
        if constexpr (OP == OP_GATED) v[e] = silu_f32(v[e]) * acc[G - 1][f][j][e];
        if constexpr (OP == OP_FP8T) v[e] *= scale;
      }
      store_y4(y, (size_t)m, n, N, yvec, v);
    }
}

// ============================================================ TILE (LDS x)
// MFMA tile path.  The NW waves of a workgroup form NW/KW groups along N
// (each wave owns FN fragments of 16 W rows: 16*FN*NW/KW rows per workgroup)
// of KW waves that split K inside the workgroup; all of them share the x
// chunks in LDS, so x is read from L2 once per 16*FN*NW/KW W rows instead of
// once per 16.  A workgroup takes at most MC fragments of 16 x rows; more
// rows go to more workgroups along grid y.  K can also be split across S
// workgroups (grid z) so that the grid still covers every CU; with S > 1 the
// workgroups of a tile combine their fp32 partials as described below.  W
// streams through a ring of P rounds in registers as 128-byte row segments
// and reaches the MFMA fragment layout through a per-wave LDS stage; x chunks
// pass through registers into a double-buffered LDS tile (one barrier per
// round, which waits only for the x copy: each round's x loads are issued
// before its W loads, and loads retire in issue order).  After the loop the
// KW waves of an N group add their sums through LDS in a fixed order.
//
// Split-K (S > 1): every workgroup stores its fp32 partial tile with device-
// coherent stores, waits for them to complete, and counts itself in the
// tile's arrival word (split_arrive).  With S = 2 the workgroup that arrives
// last reads the S partials of the tile with device-coherent loads and adds
// them in split order 0..S-1 -- the same order whichever workgroup adds, so
// the result is reproducible -- applies the epilogue and stores y.  With S >= 4
// each split adds one slice of the tile the same way, after a bounded wait
// for the other arrivals, and the last to arrive adds any slice left
// unclaimed.  (Device-coherent accesses pass the per-XCD L2 coherently; a
// device-scope fence would instead write back and invalidate the whole L2
// under every co-resident workgroup.)
// A chunk is 128 bytes of every W row: 64 K for bf16 weights, 128 K for fp8
// weights (for A8W8 also one 128-K scale group).  Its x rows are 128 bytes
// (bf16 and fp8 x with 128-byte W rows) or 256 bytes (bf16 x with fp8 W).
// With x quantised in the kernel (OP_A8W8Q) the 256 bytes of bf16 x per row
// become 128 fp8 codes in LDS, with the row's float32 scale after the chunk.
template <int OP>
struct LdsChunk {
  static constexpr int value = tlds_kch(OP);
};

template <int OP, int FM, int FN, int NW, int KW, int XD>
struct LdsRound {
  static constexpr int BO = op_base(OP);
  static constexpr int WPF = 2;                                              // 16-byte W loads per fragment per chunk
  static constexpr int XPIECES = KW * 16 * FM * tlds_xg_bytes(OP) / 16;    // 16-byte pieces of the round's x chunks
  static constexpr int XPT = tlds_xpt(OP, FM, NW, KW, XD);              // pieces per thread (direct x: FM * XV)
  u32x4 w[op_groups(OP)][FN][WPF];
  u32x4 x[XPT > 0 ? XPT : 1];
  float sx[BO == OP_A8W8 ? FM : 1];
  float sw[BO == OP_A8W8 || BO == OP_A8W8Q ? FN : 1];
};

// The maximum of v over each row of 16 lanes, in every lane of the row (DPP
// within the row: swap neighbours, swap pairs, mirror the half rows, mirror
// the row).  Every lane of the row must be active.
__device__ __forceinline__ unsigned row16_max(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));   // row_half_mirror
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));   // row_mirror
  return v;
}

// Eight bf16 x of one 128-K group, whose largest magnitude is amax (> 0),
// -> eight OCP e4m3fn codes (byte e of the result holds element e), and the
// group's scale s = amax / 448 rounded once to float32.  Each code is the
// round-to-nearest-even e4m3fn value of x / s, the float32 quotient clamped
// to +-448 first.
// No division is issued for amax >= 2^-55 (s >= 2^-64); every step below was
// checked against the divisions it replaces by enumerating all of its
// inputs, which are bf16 (8 significant bits):
//  - s: s0 = amax * RN(1/448), then one correction s0 + (amax - 448 s0) RN(1/448)
//    (the remainder is exact in one fma): equals RN(amax / 448) for every amax;
//  - y = RN(1/s): the hardware reciprocal (within 1 ulp) and one Newton step
//    y0 + y0 (1 - s y0): exact from either float neighbour of 1/s;
//  - x / s: q0 = x y, remainder r = x - q0 s (exact in one fma), q0 + r y
//    (Markstein's correction step for a correctly rounded reciprocal): equals
//    the correctly rounded quotient wherever |x / s| >= 2^-11 for every pair
//    x <= amax; below that the e4m3fn code is 0 either way.
// Smaller groups divide.  The e4m3fn rounding is the hardware conversion
// (round to nearest even; a magnitude that rounds to zero may keep its sign,
// which no product sees).
__device__ __forceinline__ uint2 quant8_e4m3fn(const u32x4 xv, float amax, float& s) {
  float q[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    q[2 * e] = __uint_as_float(xv[e] << 16);
    q[2 * e + 1] = __uint_as_float(xv[e] & 0xFFFF0000u);
  }
  if (__builtin_expect(amax >= 0x1p-55f, 1)) {
    constexpr float kInv448 = 1.0f / 448.0f;
    const float s0 = amax * kInv448;
    s = __builtin_fmaf(__builtin_fmaf(-s0, 448.0f, amax), kInv448, s0);
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float y = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q0 = q[e] * y;
      q[e] = __builtin_fmaf(__builtin_fmaf(-q0, s, q[e]), y, q0);
    }
  } else {
    s = amax / 448.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = q[e] / s;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(q[e], -448.0f, 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return make_uint2((unsigned)lo, (unsigned)hi);
}

// One wave instruction that copies 16 bytes per lane from global memory
// straight into LDS: lane l's bytes land at d + 16*l (d wave-uniform).  It has
// no register result; the copy is complete once the wave's vector-memory
// counter has passed it (the callers wait for that explicitly).  Written as
// a bare instruction so that the compiler's own counter bookkeeping for the
// weight loads is not made to wait for the copies as well.
__device__ __forceinline__ void copy16_to_lds(const void* g, unsigned char* d) {
  const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)d;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}

// s_waitcnt on the vector-memory counter alone: wait until at most V of this
// wave's vector memory instructions are outstanding (V above the counter's
// 6-bit range waits for 63, which is stricter).
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int C = V < 0 ? 0 : (V > 63 ? 63 : V);
  __builtin_amdgcn_s_waitcnt((C & 15) | ((C >> 4) << 14) | 0x0F70);
}
// Wait for the x copies of the round whose loads were followed by n more
// rounds of loads (n < N, wave-uniform): each round issues DPW copies and then
// WLD weight loads, and a wave's vector loads complete in issue order.
template <int WLD, int DPW, int N>
__device__ __forceinline__ void wait_round_copies(int n) {
  if constexpr (N > 1) {
    if (n >= N - 1) {
      wait_vmcnt<WLD + (N - 1) * (DPW + WLD)>();
      return;
    }
    wait_round_copies<WLD, DPW, N - 1>(n);
  } else {
    wait_vmcnt<WLD>();
  }
}

// W rows move as 128-byte row segments (8 rows per wave instruction, whole
// cache lines) and pass through a per-wave LDS stage into the MFMA fragment
// layout: the fragment layout itself would read 16 rows x 64 bytes per
// instruction, and that load pattern is limited by the vector L1 (its address
// stage stalls on the cache), not by HBM.
// A fragment-packed weight (packed ops) is stored in fragment layout, chunk
// by chunk: one wave load reads 1 KiB of contiguous bytes straight into the
// MFMA operand, with no stage, and the workgroups running at one time read
// neighbouring blocks of the same chunk.
// With direct x (XD = 1) every lane loads its own x fragments (from L2, as
// the rows are few) and no x tile, and no barrier per chunk, is needed.
template <int OP, int FM, int FN, int S, int P, int NW, int KW, int XD>
__global__ __launch_bounds__(64 * NW) void tlds_kernel(const Args a) {
  constexpr int BO = op_base(OP);                 // the form
  constexpr bool PK = op_packed(OP);              // weight in the fragment-packed layout
  constexpr int NT = 64 * NW;                     // threads of the workgroup
  constexpr int NG = NW / KW;                     // wave groups along N (KW waves each split K)
  constexpr int G = op_groups(OP);
  constexpr int KCH = LdsChunk<OP>::value;
  constexpr int WB = op_w_bytes(OP);
  constexpr int XB = op_x_bytes(OP);
  using Round = LdsRound<OP, FM, FN, NW, KW, XD>;
  constexpr int XPIECES = Round::XPIECES;
  constexpr int XPT = Round::XPT;
  constexpr bool QX = BO == OP_A8W8Q;             // x quantised here: bf16 in, fp8 codes + scales in LDS
  constexpr int XS = tlds_xl_stride(OP);          // LDS x row stride
  constexpr int PPR = tlds_xg_bytes(OP) / 16;     // 16-byte x pieces per chunk row (as loaded)
  constexpr bool XDMA = XD == 2;                  // x copied by DMA into swizzled stages
  constexpr int NSTG = XDMA ? P + 1 : 2;          // LDS x buffers (rounds) in use at once
  constexpr int SUBB = XDMA ? tlds_dma_chunk_bytes(OP, FM) : tlds_sub_bytes(OP, FM);   // one x chunk in LDS
  constexpr int BUFB = KW * SUBB;                 // bytes of one LDS x buffer (a round's KW chunks)
  constexpr int XTB = XD == 1 ? 0 : NSTG * BUFB + (XDMA ? 1024 : 0);   // the x tile (+ the DMA spare block)
  constexpr int DPW = XDMA ? tlds_dma_per_wave(OP, FM, NW, KW) : 0;     // DMA copies per wave per round
  constexpr int WLD = 2 * G * FN;                 // weight loads per wave per round
  constexpr int XBUF = XTB > tlds_red_bytes(OP, FM, FN, NW, KW) ? XTB : tlds_red_bytes(OP, FM, FN, NW, KW);
  constexpr int XV = tlds_xv(OP);                 // direct x: 16-byte pieces per fragment per chunk
  constexpr int WSTB = tlds_wstage_bytes(OP, FN);  // bytes of one wave's W stage

  extern __shared__ __align__(16) unsigned char xl[];   // [2][KW][x chunk] x, then [NW][G*FN*16][stride] W

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ng = wave % NG, kw = wave / NG;   // wave-uniform
  const int lr = lane & 15, lq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int m_base = blockIdx.y * 16 * FM;
  const int nb = blockIdx.x * 16 * FN * NG + ng * 16 * FN;
  const int split = blockIdx.z;
  const int kb = a.kb;
  const int NC = (K + KCH - 1) / KCH;          // chunks along K
  const int CPS = (NC + S - 1) / S;            // chunks per split
  const int c_begin = split * CPS;
  const int c_end = min(c_begin + CPS, NC);    // this split's chunks: [c_begin, c_end)
  // round r covers chunks c_begin + r*KW + [0, KW); K-group kw takes the kw-th
  const int rounds = max(0, (c_end - c_begin + KW - 1) / KW);

  // W row pointers of the 128-byte segments: load h of a fragment reads row
  // 8h + lane/8 at this lane's 16-byte column lane%8
  const char* wrow[G][FN][2];
  int wblk[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = min(nb + f * 16 + 8 * h + (lane >> 3), N - 1);
#pragma unroll
      for (int g = 0; g < G; ++g)
        wrow[g][f][h] = static_cast<const char*>(a.w) + (size_t)(n + g * N) * K * WB + (lane & 7) * 16;
    }
    wblk[f] = min(nb + f * 16, N - 1) >> 7;
  }
  unsigned char* wst = xl + XBUF + wave * WSTB;   // this wave's W stage
  // fragment-packed weight: the 2 KiB block of chunk c, group g and 16-row
  // block b starts at ((c*G + g)*N16 + b)*2048; load h of it at +1024h, this
  // lane's 16 bytes at +16*lane
  const int N16 = (N + 15) >> 4;
  const size_t cstride = (size_t)G * N16 * 2048;
  const char* wpk[G][FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int g = 0; g < G; ++g)
      wpk[g][f] = static_cast<const char*>(a.w) + ((size_t)g * N16 + (min(nb + f * 16, N - 1) >> 4)) * 2048 + lane * 16;
  // x pieces this thread copies into LDS: piece p -> the round's chunk
  // p / (16*FM*PPR), chunk row (p / PPR) % (16*FM) (x row m_base + that,
  // clamped to M-1), byte column 16*(p%PPR)
  // (x quantised here: the 8 codes of a piece land at byte 8*(p%PPR) of the
  // LDS row, and the 16 lanes of a row, lanes 16q..16q+15, share its scale)
  constexpr int XPA = XPT > 0 ? XPT : 1;          // (no pieces when x is copied by DMA)
  const char* xrowp[XPA];
  int xcolb[XPA], xdst[XPA], xsub[XPA], xrr[XPA];
  bool xmine[XPA];
#pragma unroll
  for (int i = 0; i < (XD ? 0 : XPT); ++i) {
    const int p = min((int)threadIdx.x + NT * i, XPIECES - 1);
    xmine[i] = (int)threadIdx.x + NT * i < XPIECES;
    xsub[i] = p / (16 * FM * PPR);
    xrr[i] = (p / PPR) % (16 * FM);
    xcolb[i] = (p % PPR) * 16;
    xrowp[i] = static_cast<const char*>(a.x) + (size_t)min(m_base + xrr[i], M - 1) * K * XB;
    xdst[i] = xsub[i] * SUBB + xrr[i] * XS + (QX ? (p % PPR) * 8 : xcolb[i]);
  }
  int xm[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) xm[j] = min(m_base + j * 16 + lr, M - 1);

  f32x4 acc[G][FN][FM];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[g][f][j] = f32x4{0, 0, 0, 0};

  // This wave's chunk in round c, and the first K of its 16-byte W piece h
  // (fragment layout) there
  auto chunk_of = [&](int c, int q) { return c_begin + c * KW + q; };
  auto wk = [&](int c, int h) {
    const int k0 = chunk_of(c, kw) * KCH;
    if constexpr (BO == OP_A8W8 || BO == OP_A8W8Q) return k0 + h * 64 + lq * 16;
    else if constexpr (BO == OP_FP8T) return k0 + lq * 32 + h * 16;
    else return k0 + h * 32 + lq * 8;
  };
  constexpr int LK = BO == OP_BF16 || BO == OP_GATED ? 8 : 16;   // K per 16-byte W load

  // Each round issues its x loads (and A8W8 scales) before its W loads: the
  // hardware retires a wave's loads in issue order, so the x copy into LDS,
  // which every wave must finish before the chunk's barrier, waits only for
  // L2-resident x and never for the wave's own HBM weight stream.
  auto load = [&](Round& b, int c) {
    const int stage = c % NSTG;     // x copied by DMA: the round's LDS buffer (from the unclamped round)
    c = min(c, max(rounds - 1, 0));
    const int chunk = min(chunk_of(c, kw), NC - 1);
    // x: 16-byte pieces of the round's chunk rows; a piece of a chunk past the
    // split or past K re-reads in-range data (finite, against zeroed weights)
    if constexpr (XDMA) {
      // copy the round's KW chunks straight into LDS, 1 KiB (8 rows of 128
      // bytes) per wave instruction: lane l fills row 8*block + l/8, 16-byte
      // column l%8, with the x piece of logical column (l%8) ^ ((row/2)%8), so
      // that the sixteen rows a fragment read touches fall in distinct bank
      // groups.  A wave without a block of its own this round copies into the
      // spare block, so every wave issues DPW copies per round.
      constexpr int BPC = SUBB / 1024;            // blocks per chunk
      unsigned char* sbase = xl + stage * BUFB;
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int blk = wave + NW * i;             // wave-uniform
        const bool real = blk < KW * BPC;
        const int q = real ? blk / BPC : 0, rb = real ? blk - (blk / BPC) * BPC : 0;
        const int r = rb * 8 + (lane >> 3);
        const int lc = (lane & 7) ^ ((r >> 1) & 7);
        const int ck = min(chunk_of(c, q), NC - 1);
        const char* g = static_cast<const char*>(a.x) + (size_t)min(m_base + r, M - 1) * K * XB +
                        min(ck * KCH * XB + lc * 16, K * XB - 16);
        unsigned char* d = real ? sbase + q * SUBB + rb * 1024 : xl + NSTG * BUFB;
        copy16_to_lds(g, d);
      }
      // the weight loads of the round follow the copies, so that the copy
      // wait below can count them
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (XD == 1) {
      // direct x: piece v of fragment j holds the bytes this lane's MFMA
      // operand takes (the weight's K permutation), from row xm[j]
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int v = 0; v < XV; ++v) {
          const int off = chunk * KCH * XB + (BO == OP_FP8T ? lq * 64 + v * 16 : v * 64 + lq * 16);
          b.x[j * XV + v] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + (size_t)xm[j] * K * XB +
                                                            min(off, K * XB - 16));
        }
    } else {
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int off = min(min(chunk_of(c, xsub[i]), NC - 1) * KCH * XB + xcolb[i], K * XB - 16);
        b.x[i] = *reinterpret_cast<const u32x4*>(xrowp[i] + off);
      }
    }
    if constexpr (BO == OP_A8W8) {
#pragma unroll
      for (int j = 0; j < FM; ++j) b.sx[j] = a.s0[(size_t)xm[j] * kb + chunk];
    }
    if constexpr (BO == OP_A8W8 || BO == OP_A8W8Q) {
#pragma unroll
      for (int f = 0; f < FN; ++f) b.sw[f] = a.s1[(size_t)wblk[f] * kb + chunk];
    }
    if constexpr (PK) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f)
            b.w[g][f][h] = load_nt(reinterpret_cast<const u32x4*>(wpk[g][f] + chunk * cstride + h * 1024));
    } else {
      // segment h of every fragment: 128 bytes of 8 rows; a segment piece past
      // K re-reads the last in-range piece (its weights are zeroed when used)
      const int off = min(chunk * KCH * WB, K * WB - 16 - (lane & 7) * 16);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f)
            b.w[g][f][h] = load_nt(reinterpret_cast<const u32x4*>(wrow[g][f][h] + off));
    }
  };

  auto compute = [&](const Round& b0, int c, auto tail) {
    Round b = b0;
    unsigned char* buf = xl + (c % NSTG) * BUFB;
    if constexpr (QX) {
      // quantise each 16-byte piece (8 bf16): the row's scale is the maximum
      // magnitude over its 16 lanes over 448 (bf16 magnitudes compare as
      // their bit patterns).  Padded rows (past M) and all-zero groups get
      // zero codes and the scale 1; a row's 16 lanes take the same branch.
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        uint2 qv = make_uint2(0u, 0u);
        float s = 1.0f;
        if (m_base + xrr[i] < M) {
          unsigned am = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            am = max(am, (b.x[i][e] << 16) & 0x7FFF0000u);
            am = max(am, b.x[i][e] & 0x7FFF0000u);
          }
          am = row16_max(am);
          if (am != 0u) qv = quant8_e4m3fn(b.x[i], __uint_as_float(am), s);
        }
        if (XPIECES % NT == 0 || xmine[i]) {
          *reinterpret_cast<uint2*>(buf + xdst[i]) = qv;
          if (xcolb[i] == 0) {
            *reinterpret_cast<float*>(buf + xsub[i] * SUBB + 16 * FM * XS + xrr[i] * 4) = s;
            // the first column of workgroups also hands the scales out
            const int m = m_base + xrr[i], ck = chunk_of(c, xsub[i]);
            if (a.xs_out && blockIdx.x == 0 && m < M && ck < c_end) a.xs_out[(size_t)m * kb + ck] = s;
          }
        }
      }
    } else if constexpr (XD == 0) {
#pragma unroll
      for (int i = 0; i < XPT; ++i)
        if (XPIECES % NT == 0 || xmine[i]) *reinterpret_cast<u32x4*>(buf + xdst[i]) = b.x[i];
    }
    if constexpr (XDMA) {
      // this wave's copies of round c have landed once at most the loads of
      // the rounds issued after it are outstanding; the barrier then makes
      // every wave's copies visible (and frees the buffer of round c - 1)
      if constexpr (decltype(tail)::value) wait_round_copies<WLD, DPW, P>(min(P - 1, max(rounds - 1 - c, 0)));
      else wait_round_copies<WLD, DPW, P>(P - 1);
      // a bare barrier: __syncthreads' release fence would wait for every
      // outstanding vector load (the copies write LDS), draining the weight
      // ring; the copy wait above is the ordering the x data needs, and the
      // compiler fences keep the fragment reads below the barrier
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    } else if constexpr (XD == 0) {
      __syncthreads();
    }
    if constexpr (!PK) {
      // the wave's own W stage needs no barrier (a wave's LDS accesses run in
      // order): stage the 128-byte segments (row 8h + lane/8, column lane%8) ...
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<u32x4*>(wst + ((g * FN + f) * 16 + 8 * h + (lane >> 3)) * kWRowStride +
                                      (lane & 7) * 16) = b0.w[g][f][h];
    }
    if constexpr (!PK) {
      // ... and read them back in fragment layout: row lr, the 16-byte piece h
      // of K-slot lq (fp8 weights with bf16 x: lane slot lq owns the 32
      // contiguous K of bytes 32*lq.., for W and x alike)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            b.w[g][f][h] = *reinterpret_cast<const u32x4*>(
                wst + ((g * FN + f) * 16 + lr) * kWRowStride + (BO == OP_FP8T ? lq * 32 + h * 16 : h * 64 + lq * 16));
    }
    if constexpr (decltype(tail)::value) {        // lanes past K or past the split contribute nothing
#pragma unroll
      for (int h = 0; h < Round::WPF; ++h) {
        const bool dead = wk(c, h) >= K || chunk_of(c, kw) >= c_end;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f) b.w[g][f][h] = dead ? u32x4{0, 0, 0, 0} : b.w[g][f][h];
      }
    }
    if constexpr (BO == OP_BF16 || BO == OP_GATED) {
      // every x fragment of the chunk is read before the first MFMA: with one
      // wave per SIMD nothing else hides an LDS read's latency, so the reads
      // go out back to back and the MFMAs consume them in issue order
      u32x4 B[2][FM];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          B[u][j] = XD == 1 ? b.x[j * XV + u]
                    : XDMA ? *reinterpret_cast<const u32x4*>(buf + kw * SUBB + (j * 16 + lr) * 128 +
                                                             (((u * 4 + lq) ^ (((j * 16 + lr) >> 1) & 7)) * 16))
                           : *reinterpret_cast<const u32x4*>(buf + kw * SUBB + (j * 16 + lr) * XS + u * 64 + lq * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int f = 0; f < FN; ++f)
              acc[g][f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, b.w[g][f][u]), __builtin_bit_cast(bf16x8, B[u][j]), acc[g][f][j], 0, 0, 0);
    } else if constexpr (BO == OP_FP8T) {
      // four MFMA steps of 8 K per lane slot: step u takes K 32*lq + 8u .. +7
      // of the chunk from W (fp8, converted exactly to bf16) and x alike
      u32x4 B[4][FM];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          B[u][j] = XD == 1 ? b.x[j * XV + u]
                            : *reinterpret_cast<const u32x4*>(buf + kw * SUBB + (j * 16 + lr) * XS + lq * 64 + u * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 A[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const unsigned lo = b.w[0][f][u >> 1][(u & 1) * 2], hi = b.w[0][f][u >> 1][(u & 1) * 2 + 1];
          u32x4 wb;
          wb[0] = fp8x2_to_bf16x2<false>(lo);
          wb[1] = fp8x2_to_bf16x2<true>(lo);
          wb[2] = fp8x2_to_bf16x2<false>(hi);
          wb[3] = fp8x2_to_bf16x2<true>(hi);
          A[f] = __builtin_bit_cast(bf16x8, wb);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int f = 0; f < FN; ++f)
            acc[0][f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[f], __builtin_bit_cast(bf16x8, B[u][j]),
                                                                   acc[0][f][j], 0, 0, 0);
      }
    } else {  // OP_A8W8 / OP_A8W8Q: the chunk is one 128-K scale group
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        u32x4 B16[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          B16[h] = XD == 1 ? b.x[j * XV + h]
                           : *reinterpret_cast<const u32x4*>(buf + kw * SUBB + (j * 16 + lr) * XS + h * 64 + lq * 16);
        float sxj;
        if constexpr (QX) sxj = *reinterpret_cast<const float*>(buf + kw * SUBB + 16 * FM * XS + (j * 16 + lr) * 4);
        else sxj = b.sx[j];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          f32x4 t = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int h = q >> 1, p = (q & 1) * 2;
            const long A = static_cast<long>((static_cast<unsigned long>(b.w[0][f][h][p + 1]) << 32) |
                                             b.w[0][f][h][p]);
            const long Bv = static_cast<long>((static_cast<unsigned long>(B16[h][p + 1]) << 32) | B16[h][p]);
            t = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(A, Bv, t, 0, 0, 0);
          }
          const float sc = sxj * b.sw[f];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[0][f][j][e] = __builtin_fmaf(t[e], sc, acc[0][f][j][e]);
        }
      }
    }
  };

  Round ring[P];
  ring_pipeline<P>(ring, rounds, load, compute);
  // no x copy may still be writing LDS when it is reused or released
  if constexpr (XDMA) wait_vmcnt<0>();

  // ---- K groups: waves kw > 0 hand their sums to wave kw = 0 of the same N
  // group through LDS (the x buffers are free once every wave is past its
  // last chunk), added in kw order
  const bool owner = KW == 1 || kw == 0;
  if constexpr (KW > 1) {
    constexpr int NV = G * FN * FM * 4;   // accumulator values per lane
    float* red = reinterpret_cast<float*>(xl);
    __syncthreads();
    if (kw > 0) {
      float* dst = red + ((size_t)((kw - 1) * NG + ng) * NV) * 64;
      int i = 0;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e, ++i) dst[i * 64 + lane] = acc[g][f][j][e];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int q = 1; q < KW; ++q) {
        const float* src = red + ((size_t)((q - 1) * NG + ng) * NV) * 64;
        int i = 0;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e, ++i) acc[g][f][j][e] += src[i * 64 + lane];
      }
    }
  }

  unsigned short* y = static_cast<unsigned short*>(a.y);
  const bool yvec = y_vec4(a.y, N);
  float scale = 1.0f;
  if constexpr (BO == OP_FP8T) scale = a.s0[0];
  if constexpr (S == 1) {
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m_base + j * 16 + lr;
        const int n = nb + f * 16 + lq * 4;
        if (!owner || m >= M || n >= N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[0][f][j][e];
          if constexpr (BO == OP_GATED) v[e] = silu_f32(v[e]) * acc[G - 1][f][j][e];
          if constexpr (BO == OP_FP8T) v[e] *= scale;
        }
        store_y4(y, (size_t)m, n, N, yvec, v);
      }
  } else {
    // ---- split-K: store this split's partials (device-coherent), count in,
    // and combine them (below)
    const size_t MN = (size_t)M * N;
    const auto ws = buffer_rsrc(a.ws, (unsigned)((size_t)S * G * MN * 4));
    const bool vec = (N & 3) == 0;                // 16-byte partial rows
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m_base + j * 16 + lr;
        if (!owner || m >= M) continue;
        const int n = nb + f * 16 + lq * 4;       // this lane's 4 consecutive outputs
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const size_t base = ((size_t)split * G + g) * MN + (size_t)m * N + n;
          if (vec && n + 3 < N) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[g][f][j]), ws,
                                                   (unsigned)(base * 4), 0, kCoherent);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N)
                __hip_atomic_store(a.ws + base + e, acc[g][f][j][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0): this thread's partial stores are done
    __syncthreads();
    // Combine.  With S = 2 the last split to arrive adds the whole tile.  With
    // S >= 4 the tile's outputs are cut into S slices; slice sl is added, all
    // S partials in split order, by exactly one workgroup: split sl's own
    // once it has seen all S arrivals (it waits for them at most
    // kSplitWaitTicks, and only when the whole grid is resident at once),
    // claiming the slice with an atomic OR on the epoch's claim word; the last
    // to arrive adds its own slice and then claims, in one atomic OR, every
    // slice not yet claimed.
    constexpr bool DIST = S >= 4;
    unsigned* const st = split_tile_state(a.cnt, blockIdx.y * gridDim.x + blockIdx.x);
    __shared__ int comb_last, comb_mine, comb_rest;
    if (threadIdx.x == 0) {
      const unsigned old = split_arrive<S>(st);
      const bool lst = (old & 7u) == (unsigned)(S - 1);
      bool mine = lst;
      if (DIST && !lst) {
        bool ready = false;
        if (a.split_wait > 0) {
          const unsigned base = old & ~7u;
          const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
          do {
            __builtin_amdgcn_s_sleep(1);
            ready = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base >= (unsigned)S;
          } while (!ready && __builtin_amdgcn_s_memrealtime() - t0 < kSplitWaitTicks);
        }
        const unsigned bit = 1u << split;
        mine = ready && !(__hip_atomic_fetch_or(st + 1 + ((old >> 3) & 1u), bit, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) & bit);
      }
      comb_last = lst;
      comb_mine = mine;
      comb_rest = (int)((old >> 3) & 1u);       // the epoch's claim word
    }
    __syncthreads();
    constexpr int TW = 16 * FN * NG, TH = 16 * FM;
    constexpr int NSL = DIST ? S : 1;               // slices of the tile
    const int n0 = blockIdx.x * TW;
    // add slice sl: quads (4 outputs) [sl*QS, (sl+1)*QS) of the tile, thread t
    // taking quads t, t + NT, ...; every load of a batch is issued before its sums
    auto add_slice = [&](int sl) {
      if (vec) {
        constexpr int QPR = TW / 4;               // quads per tile row
        constexpr int QS = TH * QPR / NSL;        // quads of a slice (NSL divides 64 * FM * FN * NG)
        constexpr int T = (QS + NT - 1) / NT;     // quads per thread
        constexpr int TB0 = 32 / (S * G);         // quads per batch: at most 128 registers in flight
        constexpr int TB = TB0 < 1 ? 1 : (TB0 > T ? T : TB0);
        const int q0 = sl * QS;
#pragma unroll
        for (int t0 = 0; t0 < T; t0 += TB) {
          f32x4 pv[TB][S][G];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            const int q = q0 + min((int)threadIdx.x + NT * min(t0 + tb, T - 1), QS - 1);
            const int m = min(m_base + q / QPR, M - 1), n = min(n0 + 4 * (q % QPR), N - 4);
#pragma unroll
            for (int sp = 0; sp < S; ++sp)
#pragma unroll
              for (int g = 0; g < G; ++g)
                pv[tb][sp][g] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               ws, (unsigned)((((size_t)sp * G + g) * MN + (size_t)m * N + n) * 4), 0, kCoherent));
          }
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            if (t0 + tb >= T) continue;
            const int qi = threadIdx.x + NT * (t0 + tb);
            const int q = q0 + qi;
            const int m = m_base + q / QPR, n = n0 + 4 * (q % QPR);
            if (qi >= QS || m >= M || n >= N) continue;
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = 0.0f, u = 0.0f;
#pragma unroll
              for (int sp = 0; sp < S; ++sp) {
                v += pv[tb][sp][0][e];
                if constexpr (G == 2) u += pv[tb][sp][G - 1][e];
              }
              if constexpr (BO == OP_GATED) v = silu_f32(v) * u;
              if constexpr (BO == OP_FP8T) v *= scale;
              o[e] = v;
            }
            store_y4(y, (size_t)m, n, N, yvec, o);
          }
        }
      } else {
        constexpr int ES = TW * TH / NSL;         // outputs of a slice
        for (int e = threadIdx.x; e < ES; e += NT) {
          const int eo = sl * ES + e;
          const int r = eo / TW, cc = eo - (eo / TW) * TW;
          const int m = m_base + r, n = n0 + cc;
          if (m >= M || n >= N) continue;
          const size_t i = (size_t)m * N + n;
          float v = 0.0f, u = 0.0f;
#pragma unroll
          for (int sp = 0; sp < S; ++sp) {
            v += __hip_atomic_load(a.ws + (size_t)sp * G * MN + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (G == 2)
              u += __hip_atomic_load(a.ws + ((size_t)sp * G + 1) * MN + i, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
          if constexpr (BO == OP_GATED) v = silu_f32(v) * u;
          if constexpr (BO == OP_FP8T) v *= scale;
          y[i] = f32_to_bf16(v);
        }
      }
    };
    if constexpr (!DIST) {
      if (comb_last) add_slice(0);                // workgroup-uniform
    } else {
      if (comb_mine) add_slice(split);            // workgroup-uniform
      if (comb_last) {
        __syncthreads();                          // every thread has read comb_mine
        if (threadIdx.x == 0) {
          const unsigned others = ((1u << S) - 1u) & ~(1u << split);
          comb_mine = (int)(others & ~__hip_atomic_fetch_or(st + 1 + comb_rest, others, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT));
        }
        __syncthreads();
        const unsigned got = (unsigned)comb_mine;
        for (int sl = 0; sl < S; ++sl)
          if ((got >> sl) & 1u) add_slice(sl);
      }
    }
  }
}

// y = 0 (the empty sum, K == 0).
__global__ void zero_kernel(unsigned short* y, size_t n);

// ------------------------------------------------------------- launch tables
typedef hipError_t (*LaunchFn)(const Args&, hipStream_t);

template <int OP, int MT, int R, int KS, int P>
hipError_t launch_gemv(const Args& a, hipStream_t s) {
  constexpr int RPW = (4 / KS) * R;
  const unsigned grid = (unsigned)((a.N + RPW - 1) / RPW);
  const size_t smem = OP == OP_A8W8 ? (size_t)(MT + 1) * a.kb * sizeof(float) : 0;
  hipLaunchKernelGGL((gemv_kernel<OP, MT, R, KS, P>), dim3(grid), dim3(256), smem, s, a);
  return hipGetLastError();
}

template <int OP, int FM, int FN, int KS, int P>
hipError_t launch_tile(const Args& a, hipStream_t s) {
  constexpr int RPW = (4 / KS) * FN * 16;
  const unsigned gx = (unsigned)((a.N + RPW - 1) / RPW);
  const unsigned gy = (unsigned)((a.M + 16 * FM - 1) / (16 * FM));
  const size_t smem = (size_t)tile_red_bytes(OP, FM, FN, KS);
  hipLaunchKernelGGL((tile_kernel<OP, FM, FN, KS, P>), dim3(gx, gy), dim3(256), smem, s, a);
  return hipGetLastError();
}

template <int OP, int FM, int FN, int S, int P, int NW, int KW, int XD>
hipError_t launch_tlds(const Args& a, hipStream_t s) {
  constexpr int TW = 16 * FN * (NW / KW);
  const unsigned gx = (unsigned)((a.N + TW - 1) / TW);
  const unsigned gy = (unsigned)((a.M + 16 * FM - 1) / (16 * FM));
  const size_t smem = (size_t)tlds_smem(OP, FM, FN, NW, KW, XD, P);
  Args b = a;
  if constexpr (S > 1) {
    // the resident capacity of this kernel, taken once (all devices are gfx950)
    static const unsigned long long cap =
        resident_workgroups((const void*)&tlds_kernel<OP, FM, FN, S, P, NW, KW, XD>, 64 * NW, smem);
    b.split_wait = a.split_wait >= 0 && (unsigned long long)gx * gy * S <= cap;
  }
  hipLaunchKernelGGL((tlds_kernel<OP, FM, FN, S, P, NW, KW, XD>), dim3(gx, gy, S), dim3(64 * NW), smem, s, b);
  return hipGetLastError();
}

template <int OP, int MT, int R, int KS, int P>
constexpr LaunchFn gemv_fn() {
  if constexpr (gemv_valid(OP, MT, R, KS, P)) return &launch_gemv<OP, MT, R, KS, P>;
  else return nullptr;
}
template <int OP, int FM, int FN, int KS, int P>
constexpr LaunchFn tile_fn() {
  if constexpr (tile_valid(OP, FM, FN, KS, P)) return &launch_tile<OP, FM, FN, KS, P>;
  else return nullptr;
}

template <int OP, int FM, int FN, int S, int P, int NW, int KW, int XD>
constexpr LaunchFn tlds_fn() {
  if constexpr (tlds_valid(OP, FM, FN, S, P, NW, KW, XD)) return &launch_tlds<OP, FM, FN, S, P, NW, KW, XD>;
  else return nullptr;
}

struct GemvRow { LaunchFn f[kNumGemvMT]; };
struct TileRow { LaunchFn f[kNumTileFM]; };

template <int OP, int R, int KS, int P>
constexpr GemvRow gemv_row() {
  return GemvRow{{gemv_fn<OP, 1, R, KS, P>(), gemv_fn<OP, 2, R, KS, P>(), gemv_fn<OP, 3, R, KS, P>(),
                  gemv_fn<OP, 4, R, KS, P>(), gemv_fn<OP, 6, R, KS, P>(), gemv_fn<OP, 8, R, KS, P>(),
                  gemv_fn<OP, 12, R, KS, P>(), gemv_fn<OP, 16, R, KS, P>()}};
}
template <int OP, int FN, int KS, int P>
constexpr TileRow tile_row() {
  return TileRow{{tile_fn<OP, 1, FN, KS, P>(), tile_fn<OP, 2, FN, KS, P>(), tile_fn<OP, 4, FN, KS, P>(),
                  tile_fn<OP, 6, FN, KS, P>(), tile_fn<OP, 8, FN, KS, P>()}};
}

// Buckets above MC fragments launch the MC-fragment kernel over more grid rows.
template <int OP, int FN, int S, int P, int MC, int NW, int KW, int XD>
constexpr TileRow tlds_row() {
  return TileRow{{tlds_fn<OP, tlds_fm(1, MC), FN, S, P, NW, KW, XD>(), tlds_fn<OP, tlds_fm(2, MC), FN, S, P, NW, KW, XD>(),
                  tlds_fn<OP, tlds_fm(4, MC), FN, S, P, NW, KW, XD>(), tlds_fn<OP, tlds_fm(6, MC), FN, S, P, NW, KW, XD>(),
                  tlds_fn<OP, tlds_fm(8, MC), FN, S, P, NW, KW, XD>()}};
}

// Launch tables, one pair per op, defined in ops_<op>.hip:
// gemv_table<OP>()[variant][MT index], tile_table<OP>()[variant][FM index].
template <int OP> const GemvRow* gemv_table();
template <int OP> const TileRow* tile_table();
template <> const GemvRow* gemv_table<OP_BF16>();
template <> const GemvRow* gemv_table<OP_GATED>();
template <> const GemvRow* gemv_table<OP_FP8T>();
template <> const GemvRow* gemv_table<OP_A8W8>();
template <> const GemvRow* gemv_table<OP_A8W8Q>();
template <> const TileRow* tile_table<OP_BF16>();
template <> const TileRow* tile_table<OP_GATED>();
template <> const TileRow* tile_table<OP_FP8T>();
template <> const TileRow* tile_table<OP_A8W8>();
template <> const TileRow* tile_table<OP_A8W8Q>();
template <int OP> const TileRow* tlds_table();
template <> const TileRow* tlds_table<OP_BF16>();
template <> const TileRow* tlds_table<OP_GATED>();
template <> const TileRow* tlds_table<OP_FP8T>();
template <> const TileRow* tlds_table<OP_A8W8>();
template <> const TileRow* tlds_table<OP_A8W8Q>();
template <> const TileRow* tlds_table<OP_PACKED + OP_BF16>();
template <> const TileRow* tlds_table<OP_PACKED + OP_GATED>();
template <> const TileRow* tlds_table<OP_PACKED + OP_FP8T>();
template <> const TileRow* tlds_table<OP_PACKED + OP_A8W8>();
template <> const TileRow* tlds_table<OP_PACKED + OP_A8W8Q>();

// Writes the fragment-packed copy of W [G*N, K] (G = 2 for the gated form)
// for op into Wp (packed_weight_bytes(op, N, K) bytes), on stream s.
hipError_t launch_pack(int op, const void* W, void* Wp, int N, int K, hipStream_t s);

// Measurement kernels (calib.hip): a read stream of n16 16-byte pieces over
// `grid` workgroups (slice per workgroup, or a grid-wide sweep), and `iters` rounds of 8 bf16 32x32x16 MFMA chains per wave.
hipError_t launch_calib_read(const void* buf, unsigned long long n16, int grid, int sweep, unsigned* sink,
                             hipStream_t s);
hipError_t launch_calib_mfma(int grid, int iters, unsigned* sink, hipStream_t s);

}  // namespace skg

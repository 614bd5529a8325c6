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

#include <type_traits>

#include "variants.hpp"

namespace skg {

struct Args {
  const void* x;
  const void* w;
  const float* s0;  // fp8 tensor: w_scale[1]; a8w8: x_scales[M, kb]
  const float* s1;  // a8w8: w_scales[ceil(N/128), kb]
  void* y;
  int M, N, K;
  int kb;           // ceil(K / 128): scale groups along K
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ float silu_f32(float g) {
  // g * sigmoid(g) = g / (1 + e^-g); for very negative g, e^-g overflows to
  // +inf and the quotient is -0, the correctly signed limit.
  return g / (1.0f + __expf(-g));
}

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

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

// =================================================================== GEMV
// One workgroup = 4 waves = (4/KS) row groups x KS K-slices.  Wave (rg, ks)
// owns rows n0 + rg*R + [0, R) (and the matching up rows N + ... for the gated
// form) and the K-chunks ((j*KS + ks)*64 + lane) for rounds j = 0, 1, ...; a
// chunk is one 16-byte load of a W row (8 bf16 or 16 fp8 K-elements).
template <int OP, int MT, int R, int KS, int U>
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
  const int wave = threadIdx.x >> 6;
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
  const u32x4* xp[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xp[m] = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) +
                                           (size_t)(m < M ? m : 0) * K * XB);

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

  // Load NU rounds starting at round j0, then accumulate them.
  auto rounds = [&](int j0, auto nu_tag, auto masked_tag) {
    constexpr int NU = decltype(nu_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    u32x4 wv[NU][G][R];
    u32x4 xv[NU][MT][XV];
    int cidx[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = ((j0 + u) * KS + ks) * 64 + lane;
      cidx[u] = c;
      const bool ok = !MASKED || c < C;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < R; ++r) wv[u][g][r] = ok ? load_nt(wp[g][r] + c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < XV; ++q)
          xv[u][m][q] = (ok && m < M) ? xp[m][(size_t)c * XV + q] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if constexpr (OP == OP_BF16 || OP == OP_GATED) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              float s = acc[(g * MT + m) * R + r];
#pragma unroll
              for (int d = 0; d < 4; ++d) s = dot2(xv[u][m][0][d], wv[u][g][r][d], s);
              acc[(g * MT + m) * R + r] = s;
            }
      } else if constexpr (OP == OP_FP8T) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          unsigned wb[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            wb[2 * d] = fp8x2_to_bf16x2<false>(wv[u][0][r][d]);
            wb[2 * d + 1] = fp8x2_to_bf16x2<true>(wv[u][0][r][d]);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float s = acc[m * R + r];
#pragma unroll
            for (int d = 0; d < 8; ++d) s = dot2(xv[u][m][d >> 2][d & 3], wb[d], s);
            acc[m * R + r] = s;
          }
        }
      } else {  // OP_A8W8
        const int c = cidx[u];
        const bool ok = !MASKED || c < C;
        const int grp = ok ? (c >> 3) : 0;   // 16 K per chunk, 128 K per group
        const float sw = ws_l[grp];
        unsigned xb[MT][8];
        float sxw[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          sxw[m] = xs_l[m * a.kb + grp] * sw;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            xb[m][2 * d] = fp8x2_to_bf16x2<false>(xv[u][m][0][d]);
            xb[m][2 * d + 1] = fp8x2_to_bf16x2<true>(xv[u][m][0][d]);
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          unsigned wb[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            wb[2 * d] = fp8x2_to_bf16x2<false>(wv[u][0][r][d]);
            wb[2 * d + 1] = fp8x2_to_bf16x2<true>(wv[u][0][r][d]);
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
    }
  };

  using I1 = std::integral_constant<int, 1>;
  using IU = std::integral_constant<int, U>;
  using BF = std::integral_constant<bool, false>;
  using BT = std::integral_constant<bool, true>;
  const int full = C / (64 * KS);     // rounds in which every lane of every wave has a chunk
  int j = 0;
  for (; j + U <= full; j += U) rounds(j, IU{}, BF{});
  for (; j < full; ++j) rounds(j, I1{}, BF{});
  if (full * 64 * KS < C) rounds(full, I1{}, BT{});

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
// rows m_base + [0, 16*FM) of this launch row, and the K-units
// (j*KS + ks) for rounds j.  A K-unit is 32 K (bf16), 64 K (fp8 weight with
// bf16 x) or one 128-K scale group (A8W8).
//
// Fragment layout (16x16x32 MFMA): lane l supplies, for its row l%16 of the
// A operand (W) and its column l%16 of the B operand (x), the 8 K-elements of
// slot l/16.  Which actual K-indices fill a slot does not matter as long as A
// and B agree; the loads below choose them so that the four lanes of one row
// read 64 contiguous bytes per instruction.  The 16x16 fp32 result sits with
// C[4*(l/16) + e][l%16] in lane l, register e.
template <int OP>
struct TileKUnit {
  static constexpr int value = OP == OP_A8W8 ? 128 : (OP == OP_FP8T ? 64 : 32);
};

template <int OP, int FM, int FN, int KS, int U>
__global__ __launch_bounds__(256) void tile_kernel(const Args a) {
  constexpr int G = op_groups(OP);
  constexpr int NG = 4 / KS;
  constexpr int RPW = NG * FN * 16;
  constexpr int KU = TileKUnit<OP>::value;
  constexpr int WB = op_w_bytes(OP);
  constexpr int XB = op_x_bytes(OP);
  constexpr int NACC = G * FN * FM;

  extern __shared__ float red[];     // KS > 1: [NG][KS-1][NACC*4][64]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ng = wave / KS, ks = wave - (wave / KS) * KS;
  const int lr = lane & 15, lq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int m_base = blockIdx.y * 16 * FM;
  const int nb = blockIdx.x * RPW + ng * FN * 16;
  const int NU = (K + KU - 1) / KU;

  const char* wrow[G][FN];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int n = min(nb + f * 16 + lr, N - 1);
      wrow[g][f] = static_cast<const char*>(a.w) + (size_t)(n + g * N) * K * WB;
    }
  const char* xrow[FM];
  bool mok[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m_base + j * 16 + lr;
    mok[j] = m < M;
    xrow[j] = static_cast<const char*>(a.x) + (size_t)(mok[j] ? m : 0) * K * XB;
  }

  f32x4 acc[G][FN][FM];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[g][f][j] = f32x4{0, 0, 0, 0};

  const int kb = a.kb;
  const int rounds = (NU + KS - 1) / KS;
  for (int j0 = 0; j0 < rounds; j0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = (j0 + u) * KS + ks;
      if (j0 + u >= rounds || unit >= NU) break;   // wave-uniform
      const int k0 = unit * KU;
      if constexpr (OP == OP_BF16 || OP == OP_GATED) {
        const int k = k0 + lq * 8;
        const bool kok = k < K;
        bf16x8 wa[G][FN], xb[FM];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const u32x4 v = kok ? *reinterpret_cast<const u32x4*>(wrow[g][f] + (size_t)k * 2)
                                : u32x4{0, 0, 0, 0};
            wa[g][f] = __builtin_bit_cast(bf16x8, v);
          }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const u32x4 v = (kok && mok[j]) ? *reinterpret_cast<const u32x4*>(xrow[j] + (size_t)k * 2)
                                          : u32x4{0, 0, 0, 0};
          xb[j] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int j = 0; j < FM; ++j)
              acc[g][f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[g][f], xb[j], acc[g][f][j], 0, 0, 0);
      } else if constexpr (OP == OP_FP8T) {
        // 16 fp8 of a W row per lane (K = k0 + lq*16 + [0,16)): two MFMAs.
        const int k = k0 + lq * 16;
        const bool kok = k < K;
        u32x4 wv[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f)
          wv[f] = kok ? *reinterpret_cast<const u32x4*>(wrow[0][f] + k) : u32x4{0, 0, 0, 0};
        u32x4 xv[FM][2];
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            xv[j][h] = (kok && mok[j]) ? *reinterpret_cast<const u32x4*>(xrow[j] + (size_t)(k + 8 * h) * 2)
                                       : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            u32x4 wb;
            wb[0] = fp8x2_to_bf16x2<false>(wv[f][2 * h]);
            wb[1] = fp8x2_to_bf16x2<true>(wv[f][2 * h]);
            wb[2] = fp8x2_to_bf16x2<false>(wv[f][2 * h + 1]);
            wb[3] = fp8x2_to_bf16x2<true>(wv[f][2 * h + 1]);
            const bf16x8 A = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
            for (int j = 0; j < FM; ++j)
              acc[0][f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, xv[j][h]),
                                                                     acc[0][f][j], 0, 0, 0);
          }
        }
      } else {  // OP_A8W8: one 128-K scale group per unit, four fp8 MFMAs.
        // lane (row lr, slot lq) holds K = k0 + h*64 + lq*16 + [0,16) for h = 0, 1
        u32x4 wv[FN][2], xv[FM][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = k0 + h * 64 + lq * 16;
          const bool kok = k < K;
#pragma unroll
          for (int f = 0; f < FN; ++f)
            wv[f][h] = kok ? *reinterpret_cast<const u32x4*>(wrow[0][f] + k) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < FM; ++j)
            xv[j][h] = (kok && mok[j]) ? *reinterpret_cast<const u32x4*>(xrow[j] + k) : u32x4{0, 0, 0, 0};
        }
        float sx[FM];
#pragma unroll
        for (int j = 0; j < FM; ++j)
          sx[j] = mok[j] ? a.s0[(size_t)(m_base + j * 16 + lr) * kb + unit] : 0.0f;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int nrow = min(nb + f * 16, N - 1);
          const float sw = a.s1[(size_t)(nrow >> 7) * kb + unit];
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            f32x4 t = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int h = q >> 1, p = (q & 1) * 2;
              const long A = static_cast<long>((static_cast<unsigned long>(wv[f][h][p + 1]) << 32) | wv[f][h][p]);
              const long B = static_cast<long>((static_cast<unsigned long>(xv[j][h][p + 1]) << 32) | xv[j][h][p]);
              t = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(A, B, t, 0, 0, 0);
            }
            const float s = sx[j] * sw;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[0][f][j][e] = __builtin_fmaf(t[e], s, acc[0][f][j][e]);
          }
        }
      }
    }
  }

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
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m_base + j * 16 + lr;
      if (m >= M) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nb + f * 16 + lq * 4 + e;
        if (n >= N) continue;
        float v = acc[0][f][j][e];
        if constexpr (OP == OP_GATED) v = silu_f32(v) * acc[G - 1][f][j][e];
        if constexpr (OP == OP_FP8T) v *= scale;
        y[(size_t)m * N + n] = f32_to_bf16(v);
      }
    }
}

// y = 0 (the empty sum, K == 0).
__global__ void zero_kernel(unsigned short* y, size_t n);

// ------------------------------------------------------------- launch tables
typedef hipError_t (*LaunchFn)(const Args&, hipStream_t);

template <int OP, int MT, int R, int KS, int U>
hipError_t launch_gemv(const Args& a, hipStream_t s) {
  constexpr int RPW = (4 / KS) * R;
  const unsigned grid = (unsigned)((a.N + RPW - 1) / RPW);
  const size_t smem = OP == OP_A8W8 ? (size_t)(MT + 1) * a.kb * sizeof(float) : 0;
  hipLaunchKernelGGL((gemv_kernel<OP, MT, R, KS, U>), dim3(grid), dim3(256), smem, s, a);
  return hipGetLastError();
}

template <int OP, int FM, int FN, int KS, int U>
hipError_t launch_tile(const Args& a, hipStream_t s) {
  constexpr int RPW = (4 / KS) * FN * 16;
  const unsigned gx = (unsigned)((a.N + RPW - 1) / RPW);
  const unsigned gy = (unsigned)((a.M + 16 * FM - 1) / (16 * FM));
  const size_t smem = (size_t)tile_red_bytes(OP, FM, FN, KS);
  hipLaunchKernelGGL((tile_kernel<OP, FM, FN, KS, U>), dim3(gx, gy), dim3(256), smem, s, a);
  return hipGetLastError();
}

template <int OP, int MT, int R, int KS, int U>
constexpr LaunchFn gemv_fn() {
  if constexpr (gemv_valid(OP, MT, R, KS, U)) return &launch_gemv<OP, MT, R, KS, U>;
  else return nullptr;
}
template <int OP, int FM, int FN, int KS, int U>
constexpr LaunchFn tile_fn() {
  if constexpr (tile_valid(OP, FM, FN, KS, U)) return &launch_tile<OP, FM, FN, KS, U>;
  else return nullptr;
}

struct GemvRow { LaunchFn f[kNumGemvMT]; };
struct TileRow { LaunchFn f[kNumTileFM]; };

template <int OP, int R, int KS, int U>
constexpr GemvRow gemv_row() {
  return GemvRow{{gemv_fn<OP, 1, R, KS, U>(), gemv_fn<OP, 2, R, KS, U>(), gemv_fn<OP, 3, R, KS, U>(),
                  gemv_fn<OP, 4, R, KS, U>(), gemv_fn<OP, 6, R, KS, U>(), gemv_fn<OP, 8, R, KS, U>(),
                  gemv_fn<OP, 12, R, KS, U>(), gemv_fn<OP, 16, R, KS, U>()}};
}
template <int OP, int FN, int KS, int U>
constexpr TileRow tile_row() {
  return TileRow{{tile_fn<OP, 1, FN, KS, U>(), tile_fn<OP, 2, FN, KS, U>(), tile_fn<OP, 4, FN, KS, U>(),
                  tile_fn<OP, 6, FN, KS, U>(), tile_fn<OP, 8, FN, KS, U>()}};
}

// Launch tables, one pair per op, defined in ops_<op>.hip:
// gemv_table<OP>()[variant][MT index], tile_table<OP>()[variant][FM index].
template <int OP> const GemvRow* gemv_table();
template <int OP> const TileRow* tile_table();
template <> const GemvRow* gemv_table<OP_BF16>();
template <> const GemvRow* gemv_table<OP_GATED>();
template <> const GemvRow* gemv_table<OP_FP8T>();
template <> const GemvRow* gemv_table<OP_A8W8>();
template <> const TileRow* tile_table<OP_BF16>();
template <> const TileRow* tile_table<OP_GATED>();
template <> const TileRow* tile_table<OP_FP8T>();
template <> const TileRow* tile_table<OP_A8W8>();

}  // namespace skg

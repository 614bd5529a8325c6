// kernels_mt.hpp -- the two-operand LDS tile (mt_kernel): the mid-M rows
// (speculative verification and drafting, 64 .. 512 rows), where the call is
// a dense contraction that the weight stream no longer hides.
//
// A workgroup owns an output tile of BM = 16*FM*WM x rows by BN = 16*FN*WN
// weight rows and walks K in chunks of 128 bytes per row (64 K of bf16, 128 K
// of fp8).  Both operands of a chunk are copied by DMA (global_load_lds) into
// one of P + 1 LDS stages, so every byte of the tile's W and x crosses the
// CU's memory path once per workgroup; P chunks are in flight while one is
// multiplied.  The WM x WN waves each own a 16*FM x 16*FN sub-tile and read
// both operands from LDS (v_mfma_f32_16x16x32_bf16 for bf16; for A8W8 one
// v_mfma_f32_16x16x128_f8f6f4 per 128-K scale group, scaled into fp32).
//
// LDS stage: [W: BN rows x 128 B][x: BM rows x 128 B][A8W8: x scales, 4 B per
// row in blocks of 64 rows, then W block scales 64 x 4 B].  A fragment-packed
// W arrives as its 2 KiB units (already in MFMA operand order: lane l reads 16
// contiguous bytes); a row-major operand arrives as 128-byte row segments
// whose 16-byte columns are XOR-swizzled by (row / 2) % 8, so the 16 rows of a
// fragment read fall in distinct bank groups.
//
// Split-K (S > 1): as in the LDS tile path, each workgroup stores its fp32
// partial tile with device-coherent stores, waits for them, counts itself in
// the tile's arrival word with a relaxed device-scope add (split_arrive), and
// the last arriver adds the S partials in split order 0..S-1 (its own from
// registers) and stores y.
#pragma once

#include "kernels.hpp"

namespace skg {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 4 bytes per lane from global memory into LDS at d + 4*l (see copy16_to_lds).
__device__ __forceinline__ void copy4_to_lds(const void* g, unsigned char* d) {
  const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)d;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}

// Wait until at most n * D of this wave's copies are outstanding (n < N,
// wave-uniform): the s_waitcnt immediate must be a constant.
template <int D, int N>
__device__ __forceinline__ void wait_copies(int n) {
  if constexpr (N > 1) {
    if (n >= N - 1) {
      wait_vmcnt<(N - 1) * D>();
      return;
    }
    wait_copies<D, N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// A bare workgroup barrier: the copies each wave waited for above are the
// ordering the LDS data needs; __syncthreads' release fence would also wait
// for the copies still in flight.  The compiler fences keep LDS accesses on
// their side of it.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int OP, int FM, int FN, int WM, int WN, int S, int P>
__global__ __launch_bounds__(64 * WM * WN) void mt_kernel(const Args a) {
  constexpr int BO = op_base(OP);
  constexpr bool PK = op_packed(OP);
  constexpr bool A8 = BO == OP_A8W8;
  constexpr int NW = WM * WN;
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  constexpr int KCH = A8 ? 128 : 64;             // K per 128-byte chunk
  constexpr int XB = A8 ? 1 : 2;                 // bytes per x element (== per W element)
  constexpr int STB = mt_stage_bytes(OP, FM, FN, WM, WN);
  constexpr int NSTG = P + 1;
  constexpr int WBLK = BN / 8;                   // 1 KiB copy blocks of W per chunk
  constexpr int XBLK = BM / 8;                   // 1 KiB copy blocks of x per chunk
  constexpr int XSB = (BM + 63) / 64;            // 256 B blocks of x scales (64 rows each) per chunk
  constexpr int SBLK = A8 ? XSB + 1 : 0;         // 256 B copy blocks of scales per chunk
  constexpr int NBLK = WBLK + XBLK + SBLK;
  constexpr int DPW = (NBLK + NW - 1) / NW;      // copies per wave per chunk
  constexpr int XOFF = BN * 128, SOFF = (BN + BM) * 128;

  __shared__ __align__(16) unsigned char lds[NSTG * STB + 1024];   // + a spare block for idle copies

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int split = blockIdx.z;
  const int kb = a.kb;
  const int NC = (K * XB + 127) / 128;           // chunks along K
  const int CPS = (NC + S - 1) / S;
  const int c_begin = min(split * CPS, NC);
  const int rounds = min(c_begin + CPS, NC) - c_begin;
  const int N16 = (N + 15) >> 4;
  const size_t cstride = (size_t)N16 * 2048;     // packed: bytes per chunk

  // The copies of chunk c into stage st: wave w issues blocks w, w + NW, ...;
  // blocks past the list go to the spare block so that every wave issues DPW.
  auto issue = [&](int c, int st) {
    unsigned char* sb = lds + st * STB;
    const int ck = c_begin + c;
#pragma unroll
    for (int t = 0; t < DPW; ++t) {
      const int blk = wave + NW * t;             // wave-uniform
      if (blk < WBLK) {
        if constexpr (PK) {
          const int u = blk >> 1, h = blk & 1;   // 16-row unit of the tile, its half
          const char* g = static_cast<const char*>(a.w) + (size_t)ck * cstride +
                          (size_t)min((n0 >> 4) + u, N16 - 1) * 2048 + h * 1024 + lane * 16;
          copy16_to_lds(g, sb + u * 2048 + h * 1024);
        } else {
          const int r = blk * 8 + (lane >> 3);
          const int lc = (lane & 7) ^ ((r >> 1) & 7);
          const char* g = static_cast<const char*>(a.w) + (size_t)min(n0 + r, N - 1) * K * XB +
                          min(ck * 128 + lc * 16, K * XB - 16);
          copy16_to_lds(g, sb + blk * 1024);
        }
      } else if (blk < WBLK + XBLK) {
        const int xb = blk - WBLK;
        const int r = xb * 8 + (lane >> 3);
        const int lc = (lane & 7) ^ ((r >> 1) & 7);
        const char* g = static_cast<const char*>(a.x) + (size_t)min(m0 + r, M - 1) * K * XB +
                        min(ck * 128 + lc * 16, K * XB - 16);
        copy16_to_lds(g, sb + XOFF + xb * 1024);
      } else if (A8 && blk < NBLK - 1) {
        const int sbk = blk - WBLK - XBLK;       // x scales of rows 64*sbk + lane
        copy4_to_lds(a.s0 + (size_t)min(m0 + sbk * 64 + lane, M - 1) * kb + ck, sb + SOFF + sbk * 256);
      } else if (A8 && blk == NBLK - 1) {        // W block scales of 128-row blocks n0/128 + lane
        copy4_to_lds(a.s1 + (size_t)min((n0 >> 7) + lane, ((N + 127) >> 7) - 1) * kb + ck, sb + SOFF + XSB * 256);
      } else {
        copy16_to_lds(static_cast<const char*>(a.x), lds + NSTG * STB);
      }
    }
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[f][j] = f32x4{0, 0, 0, 0};

  // a row-major operand's 16-byte piece (row r, logical column col) in a stage
  auto swz = [](int r, int col) { return r * 128 + ((col ^ ((r >> 1) & 7)) << 4); };

  auto compute = [&](int c, int st) {
    const unsigned char* sb = lds + st * STB;
    const int ck = c_begin + c;
    // pieces of the chunk at or past K (a partial last chunk) multiply zeros:
    // the copies clamp them to in-range bytes of the row
    const bool tail = (ck + 1) * 128 > K * XB;
    if constexpr (!A8) {
      // both halves' fragment reads go out first; the MFMAs of half 0 then
      // run while those of half 1 are still arriving (LDS reads return in
      // issue order)
      u32x4 A[2][FN], B[2][FM];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int rr = (wn * FN + f) * 16 + lr;
          A[u][f] = PK ? *reinterpret_cast<const u32x4*>(sb + (wn * FN + f) * 2048 + u * 1024 + lane * 16)
                       : *reinterpret_cast<const u32x4*>(sb + swz(rr, u * 4 + lq));
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
          B[u][j] = *reinterpret_cast<const u32x4*>(sb + XOFF + swz((wm * FM + j) * 16 + lr, u * 4 + lq));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (tail) {
          const bool dead = ck * KCH + u * 32 + lq * 8 >= K;
#pragma unroll
          for (int j = 0; j < FM; ++j) B[u][j] = dead ? u32x4{0, 0, 0, 0} : B[u][j];
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int f = 0; f < FN; ++f)
            acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[u][f]),
                                                                __builtin_bit_cast(bf16x8, B[u][j]), acc[f][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // lane (lr, lq) holds K bytes 16*lq .. +15 and 64 + 16*lq .. +15 of the
      // chunk, for W and x alike
      u32x4 A[2][FN], B[2][FM];
      float sx[FM], sw[FN];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int rr = (wn * FN + f) * 16 + lr;
          A[h][f] = PK ? *reinterpret_cast<const u32x4*>(sb + (wn * FN + f) * 2048 + h * 1024 + lane * 16)
                       : *reinterpret_cast<const u32x4*>(sb + swz(rr, h * 4 + lq));
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
          B[h][j] = *reinterpret_cast<const u32x4*>(sb + XOFF + swz((wm * FM + j) * 16 + lr, h * 4 + lq));
      }
#pragma unroll
      for (int j = 0; j < FM; ++j)
        sx[j] = *reinterpret_cast<const float*>(sb + SOFF + ((wm * FM + j) * 16 + lr) * 4);
#pragma unroll
      for (int f = 0; f < FN; ++f)
        sw[f] = *reinterpret_cast<const float*>(sb + SOFF + XSB * 256 +
                                                (((n0 + (wn * FN + f) * 16) >> 7) - (n0 >> 7)) * 4);
      if (tail) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool dead = ck * KCH + h * 64 + lq * 16 >= K;
#pragma unroll
          for (int j = 0; j < FM; ++j) B[h][j] = dead ? u32x4{0, 0, 0, 0} : B[h][j];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const i32x8 Bv = i32x8{(int)B[0][j][0], (int)B[0][j][1], (int)B[0][j][2], (int)B[0][j][3],
                               (int)B[1][j][0], (int)B[1][j][1], (int)B[1][j][2], (int)B[1][j][3]};
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const i32x8 Av = i32x8{(int)A[0][f][0], (int)A[0][f][1], (int)A[0][f][2], (int)A[0][f][3],
                                 (int)A[1][f][0], (int)A[1][f][1], (int)A[1][f][2], (int)A[1][f][3]};
          // both operands e4m3fn (format 0), no block scales (scale operands 0)
          const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Av, Bv, f32x4{0, 0, 0, 0}, 0, 0, 0, 0, 0, 0);
          const float sc = sx[j] * sw[f];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[f][j][e] = __builtin_fmaf(t[e], sc, acc[f][j][e]);
        }
      }
    }
  };

  // ---- the chunk loop: P chunks in flight, one multiplied
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < rounds) issue(p, p);
  for (int c = 0; c < rounds; ++c) {
    // this wave's copies of chunk c have landed once at most those of the
    // chunks issued after it (min(P - 1, rounds - 1 - c) of them) are left
    wait_copies<DPW, P>(min(P - 1, rounds - 1 - c));
    bare_barrier();                              // every wave's copies of chunk c, and all done with c - 1
    // chunk c + P goes into the stage of chunk c - 1, free since the barrier,
    // so that P chunks stay in flight while chunk c is multiplied
    if (c + P < rounds) issue(c + P, (c + P) % NSTG);
    compute(c, c % NSTG);
  }

  // ---- epilogue
  unsigned short* y = static_cast<unsigned short*>(a.y);
  const bool yvec = y_vec4(a.y, N);
  auto store_y = [&](int m, int n, const float (&v)[4]) { store_y4(y, (size_t)m, n, N, yvec, v); };

  if constexpr (S == 1) {
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m0 + (wm * FM + j) * 16 + lr;
        const int n = n0 + (wn * FN + f) * 16 + lq * 4;
        if (m >= M || n >= N) continue;
        const float v[4] = {acc[f][j][0], acc[f][j][1], acc[f][j][2], acc[f][j][3]};
        store_y(m, n, v);
      }
  } else {
    const size_t MN = (size_t)M * N;
    const auto ws = buffer_rsrc(a.ws, (unsigned)((size_t)S * MN * 4));
    const bool vec = (N & 3) == 0;               // 16-byte partial rows
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m0 + (wm * FM + j) * 16 + lr;
        const int n = n0 + (wn * FN + f) * 16 + lq * 4;
        if (m >= M || n >= N) continue;
        const size_t base = (size_t)split * MN + (size_t)m * N + n;
        if (vec) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[f][j]), ws, (unsigned)(base * 4), 0,
                                                 kCoherent);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) __hip_atomic_store(a.ws + base + e, acc[f][j][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    __shared__ unsigned last;
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this thread's partial stores are done
    __syncthreads();
    if (threadIdx.x == 0)
      last = (split_arrive<S>(split_tile_state(a.cnt, blockIdx.y * gridDim.x + blockIdx.x)) & 7u) == (unsigned)(S - 1);
    __syncthreads();
    if (last) {                                  // workgroup-uniform
      // the other splits' partials of FB fragments of W rows at a time (at
      // most 96 registers of loads in flight), all loads issued before the sums
      constexpr int FB0 = 96 / (4 * FM * (S - 1));
      constexpr int FB = FB0 < 1 ? 1 : (FB0 > FN ? FN : FB0);
#pragma unroll
      for (int f0 = 0; f0 < FN; f0 += FB) {
        f32x4 pv[FB][FM][S];
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const int f = min(f0 + fb, FN - 1);
            const int m = min(m0 + (wm * FM + j) * 16 + lr, M - 1);
            const int n = min(n0 + (wn * FN + f) * 16 + lq * 4, N - 1);
#pragma unroll
            for (int sp = 0; sp < S; ++sp) {
              if (sp == split) {
                pv[fb][j][sp] = acc[f][j];
              } else if (vec) {
                pv[fb][j][sp] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               ws, (unsigned)(((size_t)sp * MN + (size_t)m * N + n) * 4), 0, kCoherent));
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  pv[fb][j][sp][e] = __hip_atomic_load(a.ws + (size_t)sp * MN + (size_t)m * N + min(n + e, N - 1),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const int f = f0 + fb;
            const int m = m0 + (wm * FM + j) * 16 + lr;
            const int n = n0 + (wn * FN + min(f, FN - 1)) * 16 + lq * 4;
            if (f >= FN || m >= M || n >= N) continue;
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sp = 0; sp < S; ++sp)
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += pv[fb][j][sp][e];
            store_y(m, n, v);
          }
      }
    }
  }
}

template <int OP, int FM, int FN, int WM, int WN, int S, int P>
hipError_t launch_mt(const Args& a, hipStream_t s) {
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  const unsigned gx = (unsigned)((a.N + BN - 1) / BN);
  const unsigned gy = (unsigned)((a.M + BM - 1) / BM);
  hipLaunchKernelGGL((mt_kernel<OP, FM, FN, WM, WN, S, P>), dim3(gx, gy, S), dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

template <int OP, int FM, int FN, int WM, int WN, int S, int P>
constexpr LaunchFn mt_fn() {
  if constexpr (mt_valid(OP, FM, FN, WM, WN, S, P)) return &launch_mt<OP, FM, FN, WM, WN, S, P>;
  else return nullptr;
}

// Launch tables of the two-operand tile, one entry per SKG_MT variant
// (ops_mt.hip); nullptr where a variant does not serve the op.
template <int OP> const LaunchFn* mt_table();
template <> const LaunchFn* mt_table<OP_BF16>();
template <> const LaunchFn* mt_table<OP_A8W8>();
template <> const LaunchFn* mt_table<OP_PACKED + OP_BF16>();
template <> const LaunchFn* mt_table<OP_PACKED + OP_A8W8>();

}  // namespace skg

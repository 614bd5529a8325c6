/*
 * skinny_gemm.h -- C ABI of the MI355X (gfx950) skinny decode-linear library.
 *
 * The operation is the decode-shaped linear
 *
 *     y[M, N] = x[M, K] . W[N, K]^T        (M = 1..128 rows, large N and K)
 *
 * in the four forms that the decode-linear pages route and tune, and a fifth
 * that folds the A8W8 activation quantisation into the call:
 *
 *   skinny_gemm_bf16        bf16 x, bf16 W                     (mstar PR #1104,
 *                           "Why": decode linears served by skinny GEMM / GEMV)
 *   skinny_gemm_gated       fused gate/up: silu(x Wg^T) * (x Wu^T)
 *                           (mstar PR #1104, "Why": decode_gemv_silu_mul, and
 *                           "What changed": the gate/up's own gated1- entry)
 *   skinny_gemm_fp8_tensor  bf16 x, fp8 W with one scale for the whole weight
 *                           (mstar PR #1102, "What changed": the fp8 draft head)
 *   skinny_gemm_a8w8_block  fp8 x with one scale per row per 128 K-columns, fp8
 *                           W with one scale per 128 x 128 block (Decode
 *                           optimization round 3, "Retained change 2")
 *   skinny_gemm_a8w8_block_quant
 *                           the same with bf16 x, quantised inside the call
 *                           (the same page leaves that fusion open in
 *                           "Rejected paths")
 *
 * and each of the five with the weight pre-shuffled once into a fragment-
 * packed layout (skinny_gemm_pack_weight, then skinny_gemm_<form>_packed):
 * the A8W8 table the decode page tunes is the one for its pre-shuffled
 * ("bpreshuffle") weight (Decode optimization round 3, "Retained change 2").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is a DEVICE pointer to caller-owned memory,
 *           contiguous and row-major; the caller allocates and frees it.
 *           bf16 is passed as its 16-bit pattern, fp8 as OCP e4m3fn bytes (1 sign, 4 exponent with bias 7, 3 fraction
 *           bits; largest finite 448; 0x7F/0xFF are NaN), scales as float32.
 *           x and W must be 16-byte aligned.  y must not overlap any input.
 *           The library never allocates, frees, syncs on or reads device
 *           memory from the host; every call is ordered on `stream` (NULL =
 *           the null stream) and can be captured into a HIP graph.
 * Sizes.    M, N, K >= 0.  M == 0 or N == 0 is a no-op that returns OK.
 *           K == 0 writes y = 0 (the empty sum).  K must be a multiple of 8 for
 *           bf16 weights and of 16 for fp8 weights (one 16-byte load per lane).
 * Result.   y[M, N] bf16, each element rounded once (round-to-nearest-even)
 *           from a float32 accumulation.  The same call with the same inputs and
 *           the same dispatch table gives the same bits every time: reductions
 *           run in a fixed order and no atomics are used.
 * Errors.   A status code; nothing is thrown across the ABI.  Arguments are
 *           checked on the host before any launch.  skinny_gemm_last_error()
 *           returns the calling thread's text for its last non-OK status.  A
 *           fault inside a kernel surfaces at the caller's next synchronisation.
 * Dispatch. Each call rounds M up to its rows bucket {1,2,3,4,6,8,12,16,24,32,
 *           64,96,128}, or for mid-M rows {144,160,...,256} (steps of 16) and
 *           {288,320,...,512} (steps of 32: the verify and drafter grid of
 *           Decode optimization round 3, "Retained change 3"), and looks
 *           (op, bucket, N, K) up in
 *           the per-device table (Decode optimization round 3, "Retained
 *           change 2": padded-M lookup with no nearest fallback; mstar PR
 *           #1104, "What changed": one per-device table).  A miss, an absent
 *           table or a refused table uses the built-in default for the op and
 *           bucket; M above 512 uses the untuned default.  Rows above 128 run
 *           on the MFMA tile paths (launch rows of at most 128 x rows, or the
 *           two-operand tile's own row tiles).
 * Threads.  GEMM calls are reentrant.  skinny_gemm_load_table must not run
 *           concurrently with other calls.
 * Workspace. Some variants split K across workgroups and pass float32
 *           partials through a split-K workspace: caller-owned device memory
 *           registered once with skinny_gemm_set_workspace (one stream) or
 *           skinny_gemm_set_device_workspace (every stream of the device that
 *           has none of its own).  skinny_gemm_workspace_bytes tells how much a
 *           call needs; a call whose dispatch choice needs more than its
 *           stream's workspace holds, or 4 GiB or more of partials, returns
 *           SKG_EUNSUPPORTED and launches nothing.  GEMM calls never
 *           allocate, free or synchronise, and
 *           which kernel runs does not depend on the workspace, on graph
 *           capture or on earlier calls (no host sync in the decode step:
 *           mstar PR #1102, "Verification"; every kernel served from graph
 *           replay: mstar PR #1104, "Verification").  Calls that share one
 *           workspace must be ordered (one stream, or synchronised streams):
 *           calls that overlap in time on one workspace race on it and give
 *           wrong results.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int skg_status;
#define SKG_OK 0
#define SKG_EINVAL 1        /* null pointer, negative size, overlap, host memory */
#define SKG_EUNSUPPORTED 2  /* outside the contract: alignment, K multiple, size */
#define SKG_ELAUNCH 3       /* the HIP runtime rejected a launch */
#define SKG_ETABLE 4        /* table file unreadable (the table then stays off) */

/* Operation ids, as used by the query / variant calls. */
#define SKG_OP_BF16 0
#define SKG_OP_GATED 1
#define SKG_OP_FP8_TENSOR 2
#define SKG_OP_A8W8_BLOCK 3
#define SKG_OP_A8W8_QUANT 4
/* The same five forms with a fragment-packed weight: SKG_OP_PACKED + the form. */
#define SKG_OP_PACKED 5
#define SKG_OP_BF16_PACKED 5
#define SKG_OP_GATED_PACKED 6
#define SKG_OP_FP8_TENSOR_PACKED 7
#define SKG_OP_A8W8_BLOCK_PACKED 8
#define SKG_OP_A8W8_QUANT_PACKED 9

/* y[M,N] = x[M,K] . W[N,K]^T.  x, W: bf16.  scales: unused, may be NULL. */
skg_status skinny_gemm_bf16(const void* x, const void* W, const float* scales,
                            void* y, int M, int N, int K, hipStream_t stream);

/* Fused gate/up.  W is ONE [2N, K] bf16 buffer: rows [0, N) are the gate
 * weight Wg, rows [N, 2N) the up weight Wu.  y[M, N] = silu(g) * u with
 * g = x Wg^T and u = x Wu^T kept in float32 (not rounded) before the product;
 * silu(g) = g / (1 + exp(-g)).  scales: unused, may be NULL. */
skg_status skinny_gemm_gated(const void* x, const void* W, const float* scales,
                             void* y, int M, int N, int K, hipStream_t stream);

/* fp8 weight with one per-tensor scale: y = scales[0] * (x . dec(W)^T).
 * x: bf16 [M, K] (not quantised).  W: e4m3fn [N, K].  scales: device float32[1]. */
skg_status skinny_gemm_fp8_tensor(const void* x, const void* W, const float* scales,
                                  void* y, int M, int N, int K, hipStream_t stream);

/* A8W8 block scale.  x: e4m3fn [M, K]; x_scales: float32 [M, ceil(K/128)]
 * (one per row per 128 K-columns).  W: e4m3fn [N, K]; w_scales: float32
 * [ceil(N/128), ceil(K/128)] (one per 128 x 128 block).
 * y[m, n] = sum_k xs[m, k/128] dec(x[m, k]) * ws[n/128, k/128] dec(W[n, k]). */
skg_status skinny_gemm_a8w8_block(const void* x, const void* W, const float* x_scales,
                                  const float* w_scales, void* y, int M, int N, int K,
                                  hipStream_t stream);

/* A8W8 block scale with bf16 activations quantised inside the call.
 * x: bf16 [M, K], finite.  For every row m and 128-K group g (the last group
 * may be shorter) the call takes
 *     s[m, g] = max |x[m, k]| over the group / 448, one float32 division
 *               (1 when that maximum is 0), and
 *     q[m, k] = e4m3fn code of x[m, k] / s[m, g] (one float32 division),
 *               clamped to +-448 and rounded once to nearest even,
 * then computes the A8W8 product above with x_scales = s and x = q.
 * W: e4m3fn [N, K]; w_scales: float32 [ceil(N/128), ceil(K/128)].
 * x_scales_out: NULL, or device float32 [M, ceil(K/128)] that receives s (it
 * must not overlap the other arguments).  Served by the MFMA tile kernels
 * only.  (Decode optimization round 3: the activation quantisation runs as
 * its own kernels in "Profiling: why M=1-8 decode is dispatch-bound", and
 * "Rejected paths" leaves folding it into the GEMM open.) */
skg_status skinny_gemm_a8w8_block_quant(const void* x, const void* W, const float* w_scales,
                                        float* x_scales_out, void* y, int M, int N, int K,
                                        hipStream_t stream);

/* ---- Fragment-packed weights -------------------------------------------
 * The weight of form `op` (SKG_OP_BF16 .. SKG_OP_A8W8_QUANT; a packed op id
 * means its form), laid out once so that every 16-byte load of the MFMA tile
 * kernels is one lane's operand and a wave's load is 1 KiB of contiguous
 * bytes.  With WB bytes per weight element (2 for bf16, 1 for e4m3fn), G = 2
 * for the gated form (gate rows, then up rows) else 1, NC = ceil(K*WB/128)
 * chunks of 128 bytes along each row and N16 = ceil(N/16) blocks of 16 rows:
 *   the 2048-byte unit of chunk c, group g, block b starts at byte
 *   ((c*G + g)*N16 + b) * 2048 (chunk-major: the blocks of one chunk are
 *   contiguous); its 16 bytes at 1024*h + 16*l (h = 0, 1; l = 0..63) hold
 *   row 16*b + l%16 of group g, row bytes 128*c + off .. +15, where with
 *   q = l/16, off = 32*q + 16*h for the fp8_tensor form and 64*h + 16*q for
 *   the others; bytes of rows >= N or past the row (K*WB) are zero.
 * Scales keep their row-major layouts.  Results equal those of the row-major
 * form up to float32 summation order (bit-identical run to run). */

/* Bytes of the packed weight of form `op` with N rows (per half for the gated
 * form) and K columns; 0 for an unknown op, N or K <= 0, or a K that is not a
 * multiple of the form's K multiple. */
size_t skinny_gemm_packed_weight_bytes(int op, int N, int K);

/* Write the packed copy of the row-major weight W (as the form's row-major
 * entry point takes it: [N, K], or [2N, K] for gated) into W_packed (device,
 * skinny_gemm_packed_weight_bytes(op, N, K) bytes, 16-byte aligned, must not
 * overlap W), ordered on `stream`.  W is only read.  N == 0 or K == 0 is a
 * no-op. */
skg_status skinny_gemm_pack_weight(int op, const void* W, void* W_packed, int N, int K,
                                   hipStream_t stream);

/* The five forms with a packed weight: the arguments, result and errors of
 * the row-major entry point of the same name without "_packed", with
 * W_packed written by skinny_gemm_pack_weight for that form, N and K.  Served
 * by the MFMA tile kernels only. */
skg_status skinny_gemm_bf16_packed(const void* x, const void* W_packed, const float* scales,
                                   void* y, int M, int N, int K, hipStream_t stream);
skg_status skinny_gemm_gated_packed(const void* x, const void* W_packed, const float* scales,
                                    void* y, int M, int N, int K, hipStream_t stream);
skg_status skinny_gemm_fp8_tensor_packed(const void* x, const void* W_packed, const float* scales,
                                         void* y, int M, int N, int K, hipStream_t stream);
skg_status skinny_gemm_a8w8_block_packed(const void* x, const void* W_packed, const float* x_scales,
                                         const float* w_scales, void* y, int M, int N, int K,
                                         hipStream_t stream);
skg_status skinny_gemm_a8w8_block_quant_packed(const void* x, const void* W_packed,
                                               const float* w_scales, float* x_scales_out, void* y,
                                               int M, int N, int K, hipStream_t stream);

/* ---- Split-K workspace ---------------------------------------------------
 * Layout: 256 KiB of split-K tile state (65536 words: three per output tile
 * of a launch, at most 20480 tiles; a launch leaves them consistent for the
 * next), then the float32 partials [S][G][M][N] of the call (S = the
 * variant's K split, G = 2 for the gated form).  The tile state is the only
 * part that must start at zero; the registration clears it. */

/* Bytes of split-K workspace the call (op, M, N, K) needs under the current
 * dispatch (table or default), or 0 when its kernel needs none (also 0 for an
 * unknown op or sizes outside the contract).  Loads the table on first use,
 * like a GEMM call. */
size_t skinny_gemm_workspace_bytes(int op, int M, int N, int K);

/* The same for one variant of op at M rows and N outputs. */
size_t skinny_gemm_variant_workspace_bytes(int op, int variant, int M, int N);

/* Register `workspace` (device memory of `bytes` bytes, 256-byte aligned,
 * caller-owned) for the GEMM calls ordered on `stream` of the current device;
 * NULL removes the stream's registration.  The call clears the counters with
 * a kernel ordered on `stream` (so it must not run under graph capture:
 * SKG_EINVAL) and allocates nothing.  The caller keeps the memory alive while
 * it is registered and while a graph captured with it may still replay; a new
 * registration applies to later calls only.  Errors: SKG_EINVAL (fewer than
 * 256 KiB, host or short memory, capture), SKG_EUNSUPPORTED (alignment). */
skg_status skinny_gemm_set_workspace(hipStream_t stream, void* workspace, size_t bytes);

/* Register the current device's workspace, used by calls on any stream of the
 * device that has no workspace of its own; the counters are cleared on
 * `stream`, so calls on other streams must be ordered after that (for
 * instance by synchronising `stream` once).  NULL removes it.  Otherwise as
 * skinny_gemm_set_workspace. */
skg_status skinny_gemm_set_device_workspace(void* workspace, size_t bytes, hipStream_t stream);

/* For callers that cannot allocate device memory or manage a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the entry point of form `op` (SKG_OP_*: any of the ten forms)
 * with its split-K partials in the library's static device scratch instead
 * of a registered workspace.  Arguments as skinny_gemm_run_variant (s0/s1 =
 * the op's scale arrays, W = the packed weight for a packed op), result and
 * dispatch as the op's own entry point; it allocates nothing and needs no
 * registration.  The scratch is a static device array of the library, one
 * copy per device, held until the process ends: 256 KiB of split-K tile state and
 * skinny_gemm_static_scratch_bytes() (16 MiB) of partials.  A call whose
 * dispatch choice needs more partials returns SKG_EUNSUPPORTED and launches
 * nothing.  Every call on a device shares that device's scratch: calls that
 * overlap in time (on different streams) race on it and give wrong results;
 * calls ordered on one stream are safe.  The first call on a device clears
 * the counters with a kernel ordered before its own. */
skg_status skinny_gemm_run_static(int op, const void* x, const void* W, const float* s0,
                                  const float* s1, void* y, int M, int N, int K,
                                  hipStream_t stream);

/* Bytes of split-K partials the static scratch holds (16 MiB). */
size_t skinny_gemm_static_scratch_bytes(void);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* skinny_gemm_last_error(void);

/* Load the dispatch table.  path NULL: $SKINNY_GEMM_TABLE, else the table
 * installed beside the library for this device's architecture.  A table whose
 * identity header does not match this build and device, or one loaded while a
 * dispatch override ($SKINNY_GEMM_FORCE) is set, is REFUSED: one line on
 * stderr, built-in defaults stay in effect, and the call returns SKG_OK.  A
 * missing or malformed file returns SKG_ETABLE (defaults stay in effect).
 * (A table is valid only for the software stack it was tuned on: mstar PR
 * #1104, "What changed"; identity, stale and knob refusals: Strata PR #1297,
 * "The second commit: the seam rework", items 1-2.) */
skg_status skinny_gemm_load_table(const char* path);

/* Same, with the identity string given instead of read from the device and
 * runtime: lets the table logic run on a machine without a GPU. */
skg_status skinny_gemm_load_table_as(const char* path, const char* identity);

/* Identity this build and device give a table:
 * "arch=<gfx>;hip=<runtime version>;cc=<compiler hash>;space=<selection token>".
 * Writes a NUL-terminated string into buf[len]; SKG_EINVAL if it does not fit,
 * SKG_EUNSUPPORTED without a HIP device.  (The identity header a table carries
 * and is checked against: Strata PR #1297, "The second commit: the seam
 * rework", item 1.) */
skg_status skinny_gemm_identity(char* buf, int len);

/* 1 if a table is engaged, 0 if defaults are in effect. Also reports, in buf,
 * the table status line ("engaged ...", "refused ...", "none"). */
int skinny_gemm_table_status(char* buf, int len);

/* Which variant dispatch picks for (op, M, N, K), as
 * "<variant> <source>" where source is table|default|force. */
skg_status skinny_gemm_query(int op, int M, int N, int K, char* buf, int len);

/* Number of compiled variants for an op (0 for an unknown op), and the name of
 * variant i.  The variant list is one X-macro list from which the launch
 * tables, the table parser and the selection-space token all derive (one
 * rows and kernel list for every consumer: Strata PR #1297, "The second
 * commit: the seam rework", item 3). */
int skinny_gemm_num_variants(int op);
skg_status skinny_gemm_variant_name(int op, int variant, char* buf, int len);

/* 1 if variant `variant` of `op` can run M rows (its kernels are compiled for
 * that rows bucket), else 0. */
int skinny_gemm_variant_supports(int op, int variant, int M);

/* Run one named variant, bypassing the table: the tuner measures every
 * candidate this way and checks it against the true default's output before
 * it can be promoted (Strata PR #1297, "The second commit: the seam rework",
 * item 4).  s0/s1 are the op's scale arrays (fp8_tensor: s0 = w_scale; a8w8:
 * s0 = x_scales, s1 = w_scales; a8w8_quant: s0 = x_scales_out (written, may be
 * NULL), s1 = w_scales; others NULL); a packed op takes its form's arrays and
 * the packed weight as W.  knobs: reserved, pass NULL.  Arguments, errors and
 * workspace as for the op's entry point. */
skg_status skinny_gemm_run_variant(int op, int variant, const int* knobs,
                                   const void* x, const void* W, const float* s0,
                                   const float* s1, void* y, int M, int N, int K,
                                   hipStream_t stream);

/* Measurement helpers.  They compute nothing of the linear: they give the
 * rates a kernel on this device can reach, against which the linear's
 * kernels are reported (the pages weigh decode kernels by a per-launch
 * latency floor against bandwidth: Decode optimization round 3, "Profiling:
 * why M=1-8 decode is dispatch-bound").
 *
 * skinny_gemm_calib_read: one launch of `grid` workgroups of 256 threads
 * that read every byte of buf[0, bytes) once with 16-byte non-temporal loads,
 * 8 loads per thread in flight: sweep 0, each workgroup one contiguous slice;
 * sweep 1, the whole grid one sweep (thread t of T reads pieces t, t + T, ...).
 * buf is device memory, 16-byte aligned, bytes a nonzero multiple of 16; grid
 * in 1..65536.  sink is 256 device words that the kernel writes only if the
 * words it read fold (xor) to one NaN pattern, so callers ignore its value.
 *
 * skinny_gemm_calib_mfma: one launch of `grid` workgroups of 4 waves, each
 * wave issuing iters x 8 v_mfma_f32_32x32x16_bf16 (32768 flops each) on
 * register operands: grid * 4 * iters * 8 * 32768 flops.  grid in 1..65536,
 * iters in 1..2^20; sink as above.
 *
 * Both are stream-ordered, allocate nothing and return the usual statuses
 * (EINVAL for sizes out of range and host or short buffers, EUNSUPPORTED for
 * misalignment, ELAUNCH). */
skg_status skinny_gemm_calib_read(const void* buf, size_t bytes, int grid, int sweep, unsigned* sink,
                                  hipStream_t stream);
skg_status skinny_gemm_calib_mfma(int grid, int iters, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */

// variants.hpp -- compile-time facts about the variant list, shared by the
// kernels (device) and the dispatch/table code (host).  No HIP dependencies.
#pragma once

#include <cstdint>

namespace skg {

// OP_A8W8Q: A8W8 block scale with bf16 x, quantised per row and 128-K group
// inside the kernel (LDS tile path only).  Ops OP_PACKED + o are op o with
// the weight in the fragment-packed layout (LDS tile path only).
enum Op : int { OP_BF16 = 0, OP_GATED = 1, OP_FP8T = 2, OP_A8W8 = 3, OP_A8W8Q = 4, OP_PACKED = 5, NUM_OPS = 10 };
constexpr int op_base(int op) { return op >= OP_PACKED ? op - OP_PACKED : op; }
constexpr bool op_packed(int op) { return op >= OP_PACKED; }
enum Family : int { FAM_GEMV = 0, FAM_TILE = 1, FAM_TLDS = 2, FAM_MT = 3, FAM_PG = 4 };

// Rows buckets: M is rounded up to the next one (padded-M lookup with no
// nearest fallback: Decode optimization round 3, "Retained change 2";
// rows 3, 6 and 12 as in mstar PR #1102, "What changed").  Above the decode
// rows, the mid-M rows of speculative verification and drafting: steps of 16
// up to 256 and of 32 up to 512 (the padded-M grid the verify and drafter
// rows were tuned at: the same page, "Retained change 3").
constexpr int kBuckets[] = {1,   2,   3,   4,   6,   8,   12,  16,  24,  32,  64,  96,  128, 144, 160,
                            176, 192, 208, 224, 240, 256, 288, 320, 352, 384, 416, 448, 480, 512};
constexpr int kNumBuckets = sizeof(kBuckets) / sizeof(kBuckets[0]);
constexpr int kMaxBucket = 512;

// The GEMV path is compiled for each rows bucket up to 16 (MT = bucket).
constexpr int kGemvMT[] = {1, 2, 3, 4, 6, 8, 12, 16};
constexpr int kNumGemvMT = sizeof(kGemvMT) / sizeof(kGemvMT[0]);
constexpr int kGemvMaxM = 16;
// The tile path is compiled for 1, 2, 4, 6 and 8 fragments of 16 rows.
constexpr int kTileFM[] = {1, 2, 4, 6, 8};
constexpr int kNumTileFM = sizeof(kTileFM) / sizeof(kTileFM[0]);

constexpr int bucket_of(int M) {
  for (int b : kBuckets)
    if (M <= b) return b;
  return 0;  // above the largest bucket
}
constexpr int gemv_mt_index(int M) {
  for (int i = 0; i < kNumGemvMT; ++i)
    if (M <= kGemvMT[i]) return i;
  return -1;
}
constexpr int tile_fm_index(int M) {  // M rows in one launch row (<= 128)
  const int f = (M + 15) / 16;
  for (int i = 0; i < kNumTileFM; ++i)
    if (f <= kTileFM[i]) return i;
  return kNumTileFM - 1;
}

constexpr int op_groups(int op) { return op_base(op) == OP_GATED ? 2 : 1; }
constexpr bool op_w_fp8(int op) {
  return op_base(op) == OP_FP8T || op_base(op) == OP_A8W8 || op_base(op) == OP_A8W8Q;
}
constexpr bool op_x_fp8(int op) { return op_base(op) == OP_A8W8; }
constexpr int op_w_bytes(int op) { return op_w_fp8(op) ? 1 : 2; }
constexpr int op_x_bytes(int op) { return op_x_fp8(op) ? 1 : 2; }
// K elements in one 16-byte weight load of one lane.
constexpr int op_kc(int op) { return op_w_fp8(op) ? 16 : 8; }
// dwords of x that pair with one lane's 16-byte weight chunk, per row of x.
constexpr int op_xd(int op) { return op_kc(op) * op_x_bytes(op) / 4; }
// K multiple the op requires (one 16-byte load per lane never straddles K).
constexpr int op_k_multiple(int op) { return op_kc(op); }

// Register budgets that keep a variant compiled for a bucket (per lane, in
// 32-bit registers): accumulators plus P rounds of weight and x loads.
constexpr int kRegBudget = 200;
constexpr int gemv_regs(int op, int MT, int R, int P) {
  const int G = op_groups(op);
  return P * (R * G * 4 + MT * op_xd(op)) + MT * R * G;
}
constexpr bool gemv_valid(int op, int MT, int R, int KS, int P) {
  const int G = op_groups(op);
  return op != OP_A8W8Q && !op_packed(op) && (KS == 1 || KS == 2 || KS == 4) && P >= 1 && MT * R * G <= 64 &&
         gemv_regs(op, MT, R, P) <= kRegBudget && (128 % ((4 / KS) * R)) == 0;
}
constexpr int tile_red_bytes(int op, int FM, int FN, int KS) {
  return (4 / KS) * (KS - 1) * op_groups(op) * FN * FM * 4 * 64 * 4;
}
constexpr int tile_regs(int op, int FM, int FN, int P) {
  const int G = op_groups(op);
  const int per_unit = op == OP_A8W8 ? FN * 8 + FM * 8 + FM + FN
                                     : (op == OP_FP8T ? FN * 4 + FM * 8 : G * FN * 4 + FM * 4);
  return P * per_unit + G * FN * FM * 4;
}
constexpr bool tile_valid(int op, int FM, int FN, int KS, int P) {
  const int G = op_groups(op);
  return op != OP_A8W8Q && !op_packed(op) && (KS == 1 || KS == 2 || KS == 4) && P >= 1 && G * FN * FM * 4 <= 128 &&
         tile_regs(op, FM, FN, P) <= kRegBudget && tile_red_bytes(op, FM, FN, KS) <= 65536 &&
         (128 % ((4 / KS) * FN * 16)) == 0;
}
// LDS-shared-x tile path (tlds).  A chunk is 128 bytes of every W row (64 K
// of bf16 weights, 128 K of fp8 weights); its x rows arrive as KCH*XB bytes
// and sit in LDS as the same bytes, or, for OP_A8W8Q, as the 128 fp8 codes
// followed (per chunk) by one float32 scale per row.
constexpr int tlds_kch(int op) { return op_w_fp8(op) ? 128 : 64; }
constexpr int tlds_xg_bytes(int op) { return tlds_kch(op) * op_x_bytes(op); }                  // x row in HBM
constexpr int tlds_xl_bytes(int op) {                                    // x row in LDS
  return op_base(op) == OP_A8W8Q ? tlds_kch(op) : tlds_xg_bytes(op);
}
constexpr int tlds_xl_stride(int op) { return tlds_xl_bytes(op) + 16; }   // rows start 4 banks apart
constexpr int tlds_sub_bytes(int op, int FM) {                            // one chunk of x in LDS
  return 16 * FM * tlds_xl_stride(op) + (op_base(op) == OP_A8W8Q ? 16 * FM * 4 : 0);
}
// With x loaded by each lane itself (direct x, no LDS x tile): 16-byte x
// pieces per fragment per chunk.
constexpr int tlds_xv(int op) { return tlds_xg_bytes(op) / 64; }
constexpr int kWRowStride = 144;   // W stage rows: 128 bytes + 16 of padding
constexpr int tlds_wstage_bytes(int op, int FN) { return op_groups(op) * FN * 16 * kWRowStride; }
constexpr int tlds_red_bytes(int op, int FM, int FN, int NW, int KW) {   // K-group partials after the loop
  return (KW - 1) * (NW / KW) * 64 * op_groups(op) * FN * FM * 4 * 4;
}
// x copied by DMA (XD = 2): each round's KW chunks land unpadded, 16-byte
// columns swizzled per row, in one of P + 1 LDS stages; one more 1 KiB block
// takes the copies of waves that have no block of their own in a round.
constexpr int tlds_dma_chunk_bytes(int op, int FM) { return 16 * FM * tlds_xg_bytes(op); }
constexpr int tlds_dma_blocks(int op, int FM, int KW) { return KW * tlds_dma_chunk_bytes(op, FM) / 1024; }
constexpr int tlds_dma_per_wave(int op, int FM, int NW, int KW) { return (tlds_dma_blocks(op, FM, KW) + NW - 1) / NW; }
// LDS bytes of a workgroup: the x chunks (double-buffered and padded, or P + 1
// DMA stages; none with direct x), reused after the loop for the K-group
// partials, then one W stage per wave (none with a packed weight, which
// arrives in fragment layout).
constexpr int tlds_smem(int op, int FM, int FN, int NW, int KW, int XD, int P) {
  const int xb = XD == 1 ? 0
                 : XD == 2 ? (P + 1) * KW * tlds_dma_chunk_bytes(op, FM) + 1024
                           : 2 * KW * tlds_sub_bytes(op, FM);
  const int rb = tlds_red_bytes(op, FM, FN, NW, KW);
  return (xb > rb ? xb : rb) + (op_packed(op) ? 0 : NW * tlds_wstage_bytes(op, FN));
}
constexpr int tlds_xpt(int op, int FM, int NW, int KW, int XD) {   // 16-byte x pieces per thread per round
  return XD == 2 ? 0 : XD ? FM * tlds_xv(op) : (KW * 16 * FM * (tlds_xg_bytes(op) / 16) + 64 * NW - 1) / (64 * NW);
}
constexpr int tlds_regs(int op, int FM, int FN, int P, int NW, int KW, int XD) {
  const int G = op_groups(op), b = op_base(op);
  const bool a8 = b == OP_A8W8 || b == OP_A8W8Q;
  const int per_chunk = G * FN * 2 * 4 + tlds_xpt(op, FM, NW, KW, XD) * 4 + (b == OP_A8W8 ? FM + FN : (a8 ? FN : 0));
  const int acc = G * FN * FM * 4;
  const int xfrag = b == OP_FP8T ? 16 * FM : (b == OP_BF16 || b == OP_GATED ? 8 * FM : (a8 ? 8 : 0));
  const int quant = b == OP_A8W8Q ? 8 * tlds_xpt(op, FM, NW, KW, XD) : 0;   // decoded x of the pieces being quantised
  return P * per_chunk + acc * (a8 ? 2 : 1) + FM * 4 + xfrag + quant;
}
constexpr bool tlds_valid(int op, int FM, int FN, int S, int P, int NW, int KW, int XD) {
  const int G = op_groups(op);
  const bool q = op_base(op) == OP_A8W8Q;
  return (S == 1 || S == 2 || S == 4 || S == 8) && (NW == 4 || NW == 8) && (KW == 1 || KW == 2 || KW == 4 || KW == 8) &&
         NW % KW == 0 && P >= 1 && G * FN * FM * 4 <= 128 &&
         (XD == 0 || (XD == 1 && !q && FM <= 2) ||
          (XD == 2 && (op_base(op) == OP_BF16 || op_base(op) == OP_GATED) && P <= 8 &&
           tlds_dma_chunk_bytes(op, FM) % 1024 == 0)) &&
         tlds_regs(op, FM, FN, P, NW, KW, XD) <= (q && NW == 8 ? 160 : 224) &&
         tlds_smem(op, FM, FN, NW, KW, XD, P) <= 64 * 1024 && (128 % (64 * FN)) == 0;
}
// Bytes of split-K partials a tlds launch with S > 1 needs, and the number of
// output tiles (one arrival counter each) its grid has.
constexpr unsigned long long tlds_ws_bytes(int op, int S, int M, int N) {
  return S > 1 ? (unsigned long long)S * op_groups(op) * M * N * 4ull : 0ull;
}
constexpr unsigned long long tlds_tiles(int FN, int NG, int FM, int M, int N) {
  return (unsigned long long)((N + 16 * FN * NG - 1) / (16 * FN * NG)) *
         (unsigned long long)((M + 16 * FM - 1) / (16 * FM));
}
// Bytes of the fragment-packed weight of op: G groups of ceil(N/16) blocks
// of 16 rows, each cut into ceil(K*WB/128) chunks of 128 bytes per row, each
// (chunk, group, block) 2 KiB in MFMA fragment layout.
constexpr unsigned long long packed_weight_bytes(int op, int N, int K) {
  return (unsigned long long)((K * op_w_bytes(op) + 127) / 128) * op_groups(op) * ((N + 15) / 16) * 2048ull;
}
// M fragments a tlds workgroup takes: the bucket's count, capped at MC.
constexpr int tlds_fm(int FM, int MC) { return FM < MC ? FM : MC; }
constexpr int kSplitCounters = 65536;   // words of split-K tile state kept in the workspace
// A split-K output tile's state is 3 words (arrivals, two claim words); tile t
// sits in the 128-byte line t % kSplitLines, at word 3 * (t / kSplitLines) of
// it, so tiles that run together queue their atomics on different lines.
constexpr int kSplitLines = kSplitCounters / 32;
constexpr int kSplitMaxTiles = kSplitLines * 10;

// Two-operand LDS tile (mt): a workgroup of WM x WN waves owns BM = 16*FM*WM x
// rows by BN = 16*FN*WN weight rows; each chunk (128 bytes of every row) of
// both operands is copied by DMA into one of P + 1 LDS stages.  Served forms:
// bf16 and A8W8, row-major or fragment-packed weights.
constexpr bool mt_op(int op) { return op_base(op) == OP_BF16 || op_base(op) == OP_A8W8; }
constexpr int mt_stage_bytes(int op, int FM, int FN, int WM, int WN) {
  return 128 * (16 * FM * WM + 16 * FN * WN) + (op_base(op) == OP_A8W8 ? (16 * FM * WM + 63) / 64 * 256 + 256 : 0);
}
constexpr int mt_lds_bytes(int op, int FM, int FN, int WM, int WN, int P) {
  return (P + 1) * mt_stage_bytes(op, FM, FN, WM, WN) + 1024;
}
constexpr int mt_copies_per_wave(int op, int FM, int FN, int WM, int WN) {
  const int blocks = 2 * FN * WN + 2 * FM * WM + (op_base(op) == OP_A8W8 ? (FM * WM + 3) / 4 + 1 : 0);
  return (blocks + WM * WN - 1) / (WM * WN);
}
constexpr bool mt_valid(int op, int FM, int FN, int WM, int WN, int S, int P) {
  return mt_op(op) && FM >= 1 && FN >= 1 && FM * FN <= 32 && (WM * WN == 4 || WM * WN == 8) &&
         S >= 1 && S <= 8 && P >= 1 && P <= 4 &&
         mt_lds_bytes(op, FM, FN, WM, WN, P) <= 160 * 1024 &&
         (P - 1) * mt_copies_per_wave(op, FM, FN, WM, WN) <= 63;
}
constexpr unsigned long long mt_tiles(int FM, int FN, int WM, int WN, int M, int N) {
  return (unsigned long long)((N + 16 * FN * WN - 1) / (16 * FN * WN)) *
         (unsigned long long)((M + 16 * FM * WM - 1) / (16 * FM * WM));
}

// Packed-weight stream (pg): RW weight rows per workgroup of KS waves, for
// the packed bf16 and gated forms at the rows buckets up to 8.
constexpr int kPgMaxM = 8;
// VGPRs a lane needs (estimate): P rounds of the weight pieces and the x of
// each row, the sums, and ~44 more.  With KS waves a SIMD holds KS/4 of them,
// so the budget is 512 / (KS/4); past it the compiler spills.
constexpr int pg_regs(int op, int MT, int P) { return 4 * P * (op_groups(op) + MT) + op_groups(op) * MT + 44; }
constexpr bool pg_valid(int op, int MT, int RW, int KS, int P) {
  return op_packed(op) && (op_base(op) == OP_BF16 || op_base(op) == OP_GATED) && MT >= 1 && MT <= kPgMaxM &&
         (RW == 2 || RW == 4 || RW == 8) && (KS == 4 || KS == 8 || KS == 16) && P >= 1 && P <= 4 &&
         pg_regs(op, MT, P) <= 512 / (KS / 4);
}

// The MFMA tile path serves every rows bucket: rows past M inside a 16-row
// fragment re-read row M-1 and are never stored, so a table may pick it
// wherever it streams the weight faster than the VALU path, even for one row.

struct VariantDesc {
  const char* name;
  int family;
  int p0, p1, p2, p3, p4, p5, p6;  // GEMV: R, KS, U.  TILE: FN, KS, U.  TLDS: FN, S, P, MC, NW, KW, XD.
                                   // MT: FM, FN, WM, WN, S, P.  PG: RW, KS, P.
};

constexpr VariantDesc kVariants[] = {
#define SKG_GEMV(name, R, KS, U) {#name, FAM_GEMV, R, KS, U, 0, 0, 0, 0},
#define SKG_TILE(name, FN, KS, U) {#name, FAM_TILE, FN, KS, U, 0, 0, 0, 0},
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD) {#name, FAM_TLDS, FN, S, P, MC, NW, KW, XD},
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
#define SKG_MT(name, FM, FN, WM, WN, S, P) {#name, FAM_MT, FM, FN, WM, WN, S, P, 0},
#include "variants_mt.def"
#undef SKG_MT
#define SKG_PG(name, RW, KS, P) {#name, FAM_PG, RW, KS, P, 0, 0, 0, 0},
#include "variants_pg.def"
#undef SKG_PG
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

constexpr int count_family(int fam) {
  int n = 0;
  for (const auto& v : kVariants) n += v.family == fam;
  return n;
}
constexpr int kNumGemv = count_family(FAM_GEMV);
constexpr int kNumTile = count_family(FAM_TILE);
constexpr int kNumTlds = count_family(FAM_TLDS);
constexpr int kNumMt = count_family(FAM_MT);
constexpr int kNumPg = count_family(FAM_PG);
// index of variant i inside its family's launch table
constexpr int family_index(int i) {
  int n = 0;
  for (int j = 0; j < i; ++j) n += kVariants[j].family == kVariants[i].family;
  return n;
}

// Whether variant i of op can run M rows (M >= 1).
constexpr bool variant_supports(int op, int i, int M) {
  const VariantDesc& v = kVariants[i];
  if (v.family == FAM_GEMV) {
    const int mi = gemv_mt_index(M);
    return mi >= 0 && gemv_valid(op, kGemvMT[mi], v.p0, v.p1, v.p2);
  }
  if (v.family == FAM_MT) return mt_valid(op, v.p0, v.p1, v.p2, v.p3, v.p4, v.p5);
  if (v.family == FAM_PG) {
    const int mi = gemv_mt_index(M);
    return mi >= 0 && pg_valid(op, kGemvMT[mi], v.p0, v.p1, v.p2);
  }
  const int fm = M > kMaxBucket ? kNumTileFM - 1 : tile_fm_index(M);
  if (v.family == FAM_TLDS) return tlds_valid(op, tlds_fm(kTileFM[fm], v.p3), v.p0, v.p1, v.p2, v.p4, v.p5, v.p6);
  return tile_valid(op, kTileFM[fm], v.p0, v.p1, v.p2);
}

// Whether variant i's output tiles at M rows and N outputs fit the split-K
// tile state (kSplitMaxTiles); variants that do not split K always fit.
constexpr bool split_tiles_fit(int i, int M, int N) {
  const VariantDesc& d = kVariants[i];
  if (d.family == FAM_MT)
    return d.p4 == 1 || mt_tiles(d.p0, d.p1, d.p2, d.p3, M, N) <= (unsigned long long)kSplitMaxTiles;
  if (d.family != FAM_TLDS || d.p1 == 1) return true;
  const int fm = M > kMaxBucket ? kNumTileFM - 1 : tile_fm_index(M);
  return tlds_tiles(d.p0, d.p4 / d.p5, tlds_fm(kTileFM[fm], d.p3), M, N) <= (unsigned long long)kSplitMaxTiles;
}

// FNV-1a over the list's text: the kernel-selection-space token.
constexpr uint32_t fnv1a(const char* s, uint32_t h = 2166136261u) {
  for (; *s; ++s) h = (h ^ static_cast<uint8_t>(*s)) * 16777619u;
  return h;
}
constexpr const char kSpaceText[] =
    "buckets=1,2,3,4,6,8,12,16,24,32,64,96,128,144,160,176,192,208,224,240,256,288,320,352,384,416,448,480,512;"
    "gemv_mt=1,2,3,4,6,8,12,16;tile_fm=1,2,4,6,8;tile_min=1;"
#define SKG_GEMV(name, R, KS, U) "G:" #name "," #R "," #KS "," #U ";"
#define SKG_TILE(name, FN, KS, U) "T:" #name "," #FN "," #KS "," #U ";"
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD) "L:" #name "," #FN "," #S "," #P "," #MC "," #NW "," #KW "," #XD ";"
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
#define SKG_MT(name, FM, FN, WM, WN, S, P) "X:" #name "," #FM "," #FN "," #WM "," #WN "," #S "," #P ";"
#include "variants_mt.def"
#undef SKG_MT
#define SKG_PG(name, RW, KS, P) "Q:" #name "," #RW "," #KS "," #P ";"
#include "variants_pg.def"
#undef SKG_PG
    "kernels=19";  // bump when a kernel's arithmetic or indexing changes
constexpr uint32_t kSpaceToken = fnv1a(kSpaceText);

}  // namespace skg

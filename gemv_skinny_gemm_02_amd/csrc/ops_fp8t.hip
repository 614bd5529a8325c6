// ops_fp8t.hip -- instantiates every compiled variant of the fp8t form.
#include "kernels.hpp"

namespace skg {

namespace {
constexpr GemvRow kGemv[kNumGemv] = {
#define SKG_GEMV(name, R, KS, U) gemv_row<OP_FP8T, R, KS, U>(),
#define SKG_TILE(name, FN, KS, U)
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD)
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
constexpr TileRow kTile[kNumTile] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U) tile_row<OP_FP8T, FN, KS, U>(),
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD)
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
constexpr TileRow kTlds[kNumTlds] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U)
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD) tlds_row<OP_FP8T, FN, S, P, MC, NW, KW, XD>(),
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
}  // namespace

template <> const GemvRow* gemv_table<OP_FP8T>() { return kGemv; }
template <> const TileRow* tile_table<OP_FP8T>() { return kTile; }
template <> const TileRow* tlds_table<OP_FP8T>() { return kTlds; }

}  // namespace skg

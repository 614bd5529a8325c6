// ops_a8w8q.hip -- instantiates every compiled variant of the a8w8 form with x
// quantised in the kernel (the LDS tile family; the others compile to nothing).
#include "kernels.hpp"

namespace skg {

namespace {
constexpr GemvRow kGemv[kNumGemv] = {
#define SKG_GEMV(name, R, KS, U) gemv_row<OP_A8W8Q, R, KS, U>(),
#define SKG_TILE(name, FN, KS, U)
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD)
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
constexpr TileRow kTile[kNumTile] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U) tile_row<OP_A8W8Q, FN, KS, U>(),
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD)
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
constexpr TileRow kTlds[kNumTlds] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U)
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD) tlds_row<OP_A8W8Q, FN, S, P, MC, NW, KW, XD>(),
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
}  // namespace

template <> const GemvRow* gemv_table<OP_A8W8Q>() { return kGemv; }
template <> const TileRow* tile_table<OP_A8W8Q>() { return kTile; }
template <> const TileRow* tlds_table<OP_A8W8Q>() { return kTlds; }

}  // namespace skg

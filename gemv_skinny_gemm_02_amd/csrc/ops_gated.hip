// ops_gated.hip -- instantiates every compiled variant of the gated form.
#include "kernels.hpp"

namespace skg {

namespace {
constexpr GemvRow kGemv[kNumGemv] = {
#define SKG_GEMV(name, R, KS, U) gemv_row<OP_GATED, R, KS, U>(),
#define SKG_TILE(name, FN, KS, U)
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
};
constexpr TileRow kTile[kNumTile] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U) tile_row<OP_GATED, FN, KS, U>(),
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
};
}  // namespace

template <> const GemvRow* gemv_table<OP_GATED>() { return kGemv; }
template <> const TileRow* tile_table<OP_GATED>() { return kTile; }

}  // namespace skg

// ops_a8w8qp.hip -- instantiates the LDS tile variants of the A8W8 (x quantised in the call) form with
// a fragment-packed weight (the only family that reads that layout).
#include "kernels.hpp"

namespace skg {

namespace {
constexpr TileRow kTlds[kNumTlds] = {
#define SKG_GEMV(name, R, KS, U)
#define SKG_TILE(name, FN, KS, U)
#define SKG_TLDS(name, FN, S, P, MC, NW, KW, XD) tlds_row<OP_PACKED + OP_A8W8Q, FN, S, P, MC, NW, KW, XD>(),
#include "variants.def"
#undef SKG_GEMV
#undef SKG_TILE
#undef SKG_TLDS
};
}  // namespace

template <> const TileRow* tlds_table<OP_PACKED + OP_A8W8Q>() { return kTlds; }

}  // namespace skg

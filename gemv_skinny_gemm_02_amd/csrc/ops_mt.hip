// ops_mt.hip -- instantiates the two-operand LDS tile variants (kernels_mt.hpp)
// for the forms it serves: bf16 and A8W8, row-major and fragment-packed.
#include "kernels_mt.hpp"

namespace skg {

namespace {
template <int OP>
struct MtTable {
  LaunchFn f[kNumMt];
};
template <int OP>
constexpr MtTable<OP> make_mt() {
  return MtTable<OP>{{
#define SKG_MT(name, FM, FN, WM, WN, S, P) mt_fn<OP, FM, FN, WM, WN, S, P>(),
#include "variants_mt.def"
#undef SKG_MT
  }};
}
constexpr MtTable<OP_BF16> kBf16 = make_mt<OP_BF16>();
constexpr MtTable<OP_A8W8> kA8w8 = make_mt<OP_A8W8>();
constexpr MtTable<OP_PACKED + OP_BF16> kBf16p = make_mt<OP_PACKED + OP_BF16>();
constexpr MtTable<OP_PACKED + OP_A8W8> kA8w8p = make_mt<OP_PACKED + OP_A8W8>();
}  // namespace

template <> const LaunchFn* mt_table<OP_BF16>() { return kBf16.f; }
template <> const LaunchFn* mt_table<OP_A8W8>() { return kA8w8.f; }
template <> const LaunchFn* mt_table<OP_PACKED + OP_BF16>() { return kBf16p.f; }
template <> const LaunchFn* mt_table<OP_PACKED + OP_A8W8>() { return kA8w8p.f; }

}  // namespace skg

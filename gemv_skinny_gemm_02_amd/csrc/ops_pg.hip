// ops_pg.hip -- instantiates the packed-weight stream variants (kernels_pg.hpp)
// for the packed bf16 and gated forms.
#include "kernels_pg.hpp"

namespace skg {

namespace {
template <int OP, int RW, int KS, int P>
constexpr GemvRow pg_row() {
  return GemvRow{{pg_fn<OP, 1, RW, KS, P>(), pg_fn<OP, 2, RW, KS, P>(), pg_fn<OP, 3, RW, KS, P>(),
                  pg_fn<OP, 4, RW, KS, P>(), pg_fn<OP, 6, RW, KS, P>(), pg_fn<OP, 8, RW, KS, P>(),
                  pg_fn<OP, 12, RW, KS, P>(), pg_fn<OP, 16, RW, KS, P>()}};
}
constexpr GemvRow kBf16p[kNumPg] = {
#define SKG_PG(name, RW, KS, P) pg_row<OP_PACKED + OP_BF16, RW, KS, P>(),
#include "variants_pg.def"
#undef SKG_PG
};
constexpr GemvRow kGatedp[kNumPg] = {
#define SKG_PG(name, RW, KS, P) pg_row<OP_PACKED + OP_GATED, RW, KS, P>(),
#include "variants_pg.def"
#undef SKG_PG
};
}  // namespace

template <> const GemvRow* pg_table<OP_PACKED + OP_BF16>() { return kBf16p; }
template <> const GemvRow* pg_table<OP_PACKED + OP_GATED>() { return kGatedp; }

}  // namespace skg

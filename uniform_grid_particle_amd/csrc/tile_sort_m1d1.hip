// tile_sort_m1d1.hip -- instantiates the staged tile kernel variants with
// records moved, with the overflow diagnostics: every tile shift, with and without stable order and single-tile
// mode (tile_launch.h).
#define UGP_TILE_LAUNCH_DEFINE
#include "tile_launch.h"

namespace ugp {
UGP_TILE_INSTANTIATE(true, true)
}  // namespace ugp

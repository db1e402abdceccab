// kernels_bf16.hip -- launch table of the scan kernels with a, b and h stored as bf16.
#include "instances.hpp"

namespace linrec_host {

const Launch* pick_launch_bf16(const TileShape& s, bool ahead) { return pick_launch<linrec::Bf16>(s, ahead); }

}  // namespace linrec_host

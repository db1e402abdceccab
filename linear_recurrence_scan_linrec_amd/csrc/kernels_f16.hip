// kernels_f16.hip -- launch table of the scan kernels with a, b and h stored as f16.
#include "instances.hpp"

namespace linrec_host {

const Launch* pick_launch_f16(const TileShape& s, bool ahead) { return pick_launch<linrec::F16>(s, ahead); }

}  // namespace linrec_host

// kernels_f32.hip -- launch table of the scan kernels with a, b and h stored as f32.
#include "instances.hpp"

namespace linrec_host {

const Launch* pick_launch_f32(const TileShape& s, bool ahead) { return pick_launch<float>(s, ahead); }

}  // namespace linrec_host

// Kernel instances for storage type F16 with A stored as (k, m).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_f16_lay1(int ep, int cfg) { return pick_t<F16, 1>(ep, cfg); }
}  // namespace gek

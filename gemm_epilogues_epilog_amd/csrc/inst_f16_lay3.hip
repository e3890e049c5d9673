// Kernel instances for storage type F16 with A stored as (k, m) and B as (n, k).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_f16_lay3(int ep, int cfg) { return pick_t<F16, 3>(ep, cfg); }
}  // namespace gek

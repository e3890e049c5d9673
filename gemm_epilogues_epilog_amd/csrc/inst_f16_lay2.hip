// Kernel instances for storage type F16 with B stored as (n, k).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_f16_lay2(int ep, int cfg) { return pick_t<F16, 2>(ep, cfg); }
}  // namespace gek

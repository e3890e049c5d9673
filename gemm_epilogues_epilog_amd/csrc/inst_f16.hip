// Kernel instances for storage type F16.
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_f16(int ep, int cfg) { return pick<F16>(ep, cfg); }
}  // namespace gek

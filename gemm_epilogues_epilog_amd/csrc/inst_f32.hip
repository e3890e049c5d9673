// Kernel instances for storage type F32.
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_f32(int ep, int cfg) { return pick<F32>(ep, cfg); }
}  // namespace gek

// Kernel instances for storage type BF16.
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_bf16(int ep, int cfg) { return pick<BF16>(ep, cfg); }
}  // namespace gek

// Kernel instances for storage type BF16 with A stored as (k, m).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_bf16_lay1(int ep, int cfg) { return pick_t<BF16, 1>(ep, cfg); }
}  // namespace gek

// Kernel instances for storage type BF16 with A stored as (k, m) and B as (n, k).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_bf16_lay3(int ep, int cfg) { return pick_t<BF16, 3>(ep, cfg); }
}  // namespace gek

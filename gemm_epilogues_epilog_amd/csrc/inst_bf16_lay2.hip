// Kernel instances for storage type BF16 with B stored as (n, k).
#include "launch.hpp"

namespace gek {
LaunchFn get_launch_bf16_lay2(int ep, int cfg) { return pick_t<BF16, 2>(ep, cfg); }
}  // namespace gek

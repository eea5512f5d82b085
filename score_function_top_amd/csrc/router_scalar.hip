// Element-wise router kernels (any E), 64-lane token groups.
#include "router_launch.h"
ROUTER_DEFINE_PART(scalar, 64, false, 1, 2, 4, 8, 16)

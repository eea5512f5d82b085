// Element-wise router kernels (any E), 64-lane token groups, rows of 1 to 6
// chunks (router_scalar2.hip: 8 to 16).
#include "router_launch.h"
ROUTER_DEFINE_PART(scalar, 64, false, 1, 2, 3, 4, 6)

// Vector router kernels, 64-lane token groups, 1024 < E <= 2304.
#include "router_launch.h"
ROUTER_DEFINE_PART(lpt64b, 64, true, 6, 8, 9)

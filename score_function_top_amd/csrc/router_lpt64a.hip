// Vector router kernels, 64-lane token groups, E <= 1024.
#include "router_launch.h"
ROUTER_DEFINE_PART(lpt64a, 64, true, 1, 2, 3, 4)

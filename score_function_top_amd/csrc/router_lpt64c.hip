// Vector router kernels, 64-lane token groups, 2304 < E <= 4096.
#include "router_launch.h"
ROUTER_DEFINE_PART(lpt64c, 64, true, 12, 16)

// Vector router kernels, 32-lane token groups (two tokens per wave).
#include "router_launch.h"
ROUTER_DEFINE_PART(lpt32, 32, true, 1, 2, 4)

// Vector router kernels, 16-lane token groups (four tokens per wave).
#include "router_launch.h"
ROUTER_DEFINE_PART(lpt16, 16, true, 1, 2, 4)

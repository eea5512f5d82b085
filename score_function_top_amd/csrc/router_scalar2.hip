// Element-wise router kernels (any E), 64-lane token groups, rows of 8 to 16
// chunks (a unit of its own so that the two halves compile in parallel).
#include "router_launch.h"
ROUTER_DEFINE_PART(scalar2, 64, false, 8, 9, 12, 16)

// Head-dim-256 main-kernel instantiations of the IlpSched set (main_launch.h), built with the
// latency-oriented scheduler: every route without a bias (the bias variants spill under it and
// stay in main_d256.hip).
#include "main_ilp.h"

SDPA_ILP_PF(256, 4, DQ_ATOMIC, 0)
SDPA_ILP_PF(256, 4, DQ_DS, 0)
SDPA_ILP_PF(256, 4, DQ_PARTIAL, 0)
SDPA_ILP_PF(256, 4, DQ_RELAY, 0)

// Head-dim-128 main-kernel instantiations of the IlpSched set (main_launch.h), built with the
// latency-oriented scheduler.
#include "main_ilp.h"

// 8 waves, no bias: atomic, dS-panel and relay routes (the dQ-partial kernels are slower under
// this scheduler and stay in main_d128.hip)
SDPA_ILP_PF(128, 8, DQ_ATOMIC, 0)
SDPA_ILP_PF(128, 8, DQ_DS, 0)
SDPA_ILP_PF(128, 8, DQ_RELAY, 0)
// 4 waves, additive bias (1) and bias with dBias (2), every route
SDPA_ILP_PF(128, 4, DQ_ATOMIC, 1)
SDPA_ILP_PF(128, 4, DQ_DS, 1)
SDPA_ILP_PF(128, 4, DQ_PARTIAL, 1)
SDPA_ILP_PF(128, 4, DQ_RELAY, 1)
SDPA_ILP_PF(128, 4, DQ_ATOMIC, 2)
SDPA_ILP_PF(128, 4, DQ_DS, 2)
SDPA_ILP_PF(128, 4, DQ_PARTIAL, 2)
SDPA_ILP_PF(128, 4, DQ_RELAY, 2)
// NVFP4 QAT (bf16, exact head dims, no bias) on the relay route, the one route where it keeps
// 4 waves
SDPA_ILP(128, 4, DQ_RELAY, false, 0, false, true)

// The jagged forward kernels that run faster under LLVM's iterative ILP
// scheduler: the causal ones at d = 128 and all of them at d = 192 and 256
// (long rows per lane, one workgroup per CU above d = 128).  The kernel is
// defined in fwd.hip, which this unit includes with JFA_FWD_ILP_UNIT defined so
// that it emits only those instantiations and their launcher.
#define JFA_FWD_ILP_UNIT 1
#include "fwd.hip"

// Causal instantiations of the jagged forward kernel ("Optimizing Jagged Flash
// Attention with TLX": the masked diagonal tiles of the peeled key loop).  The
// kernel is defined in fwd.hip; this unit emits only its causal variants and
// their launcher, so that they can be compiled with a scheduling strategy of
// their own (LLVM's iterative ILP scheduler: about 3.5 % faster on long causal
// rows, 3 % slower on short non-causal ones).
#define JFA_FWD_CAUSAL_TU 1
#include "fwd.hip"

// The dK/dV kernels at d = 192 and 256 and the dQ kernels at d = 192.  Built with
// the MFMA builtins in their VGPR form, so that the S/dP products feed the
// softmax without copies while the dK/dV accumulators stay in AGPRs through
// hand-written MFMAs (DkvTile::ACC_AGPR).  The kernels are defined in bwd.hip,
// which this unit includes with JFA_BWD_WIDE_UNIT defined so that it emits only
// those kernels.
#define JFA_BWD_WIDE_UNIT 1
#include "bwd.hip"

// stubs.hip -- launchers for variants not built yet.
#include "kernels.h"

hipError_t lw_launch_gemv_mfma(const KArgs &, int, SadPlan, int, hipStream_t) { return hipErrorNotSupported; }

// Register-staged MFMA macro-tile GEMM instances for f16 inputs.
#include "launch.h"

#define DGE_DT IN_F16
#define DGE_REGSTAGED 1
#define DGE_LAUNCHER launch_mfma_f16
#include "mfma_instances.inc"

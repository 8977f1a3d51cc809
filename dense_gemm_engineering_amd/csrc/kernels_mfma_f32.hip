// Register-staged MFMA macro-tile GEMM instances for f32 inputs.
#include "launch.h"

#define DGE_DT IN_F32
#define DGE_REGSTAGED 1
#define DGE_LAUNCHER launch_mfma_f32
#include "mfma_instances.inc"

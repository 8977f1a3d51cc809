// Register-staged MFMA macro-tile GEMM instances for bf16 inputs.
#include "launch.h"

#define DGE_DT IN_BF16
#define DGE_REGSTAGED 1
#define DGE_LAUNCHER launch_mfma_bf16
#include "mfma_instances.inc"

// Direct-to-LDS MFMA macro-tile GEMM instances for bf16 inputs, K x N B.
#include "launch.h"
#include "mfma_direct.h"

#define DGE_DT IN_BF16
#define DGE_DIRECT 1
#define DGE_DIRECT_TB 0
#define DGE_DIRECT_LAUNCHER launch_mfma_direct_bf16_nn
#include "mfma_instances.inc"

// MFMA macro-tile GEMM instances for f32 inputs.
#include "launch.h"
#include "mfma_direct.h"

#define DGE_DT IN_F32
#define DGE_LAUNCHER launch_mfma_f32
#define DGE_DIRECT 0
#define DGE_DIRECT_LAUNCHER launch_mfma_direct_f32
#include "mfma_instances.inc"

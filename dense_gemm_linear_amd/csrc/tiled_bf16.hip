#include "internal.hpp"
#define DT_VALUE DT_BF16
#define LAUNCH_NAME launch_tiled_bf16
#define LAUNCH_AB_NAME launch_ab_bf16
#define LAUNCH_PP_NAME launch_pp_bf16
#include "tiled.inc"

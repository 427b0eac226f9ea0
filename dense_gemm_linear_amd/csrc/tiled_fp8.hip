#include "internal.hpp"
#define DT_VALUE DT_FP8
#define LAUNCH_NAME launch_tiled_fp8
#define LAUNCH_AB_NAME launch_ab_fp8
#define LAUNCH_PP_NAME launch_pp_fp8
#include "tiled.inc"

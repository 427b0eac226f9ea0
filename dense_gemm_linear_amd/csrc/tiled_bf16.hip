#include "internal.hpp"
#define DT_VALUE DT_BF16
#define LAUNCH_NAME launch_tiled_bf16
#include "tiled.inc"

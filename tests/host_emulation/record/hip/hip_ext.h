// Record-only build: hipExtLaunchKernelGGL is defined in hip_runtime.h.
#pragma once
#include "hip_runtime.h"

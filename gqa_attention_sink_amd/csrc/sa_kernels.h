// Kernel-side view of the launch interface: the host-visible argument structs and
// launch declarations (sa_launch.h), the shared chunk plan (sa_plan.h) and the device
// YaRN helpers (sa_rope.h).
#pragma once

#include <hip/hip_runtime.h>

#include "sa_launch.h"
#include "sa_plan.h"
#include "sa_rope.h"

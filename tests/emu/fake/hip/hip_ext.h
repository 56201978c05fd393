// Host emulation: hipExtLaunchKernelGGL launches like hipLaunchKernelGGL
// (events are not emulated).
#pragma once
#include <hip/hip_runtime.h>
typedef void* hipEvent_t;
#define hipExtLaunchKernelGGL(K, G, B, SH, S, START, STOP, FLAGS, ...) \
    ((void)(START), (void)(STOP), emu::launch(dim3(G), dim3(B), [=]() { K(__VA_ARGS__); }))

"""MI355X-native (gfx950) MoE expert-parallel route / dispatch / combine.

The compute lives in libep_route_topk.so (HIP kernels behind the C ABI in
include/ep_route_topk.h).  Submodules:
  combine_ep_route_topk_amd.ep         Python binding; loads the library on
                                       import (no CPU fallback)
  combine_ep_route_topk_amd.workloads  seeded synthetic inputs
"""

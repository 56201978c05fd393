// fused.hip -- flag-in-payload persistent mode (layout + dispatch + combine in
// one launch).  Workspace initialisation lives here too.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

__global__ void fused_init_kernel(WsHeader* hdr, uint64_t first_epoch) {
    if (threadIdx.x == 0) {
        hdr->magic = kFusedMagic;
        hdr->error = kDevOk;
        hdr->scan_ticket = 0;
        hdr->timeout = 0;
        hdr->work_ticket = 0;
        hdr->hist_done = 0;
        hdr->exit_count = 0;
        hdr->epoch = first_epoch;
        hdr->last_epoch = 0;
    }
}

}  // namespace

hipError_t launch_fused_init(void* ws, uint64_t first_epoch, hipStream_t s) {
    hipLaunchKernelGGL(fused_init_kernel, dim3(1), dim3(64), 0, s,
                       static_cast<WsHeader*>(ws), first_epoch);
    return hipGetLastError();
}

hipError_t launch_fused(const uint16_t*, const int32_t*, const float*, int, int, int, int,
                        int, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, uint8_t*,
                        uint16_t*, void*, uint32_t, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace ep

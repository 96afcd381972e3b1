// ssq_copy.hip -- a streaming device-to-device copy for gfx950, the reference a state
// step's bandwidth is compared with: one 16-byte load and one 16-byte store per lane,
// non-temporal, a 256-thread workgroup per 4 KiB.  Of the shapes tried (more pieces per
// lane, cached stores, the runtime's copy) this one sustained the highest rate.
#include "ssq_device.h"
#include "ssq_internal.h"

namespace ssq {

__global__ __launch_bounds__(256) void k_stream_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) st_stream(dst + i, ld_stream(src + i));
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t st)
{
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = (n16 + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

} // namespace ssq

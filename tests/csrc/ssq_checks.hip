// ssq_checks.hip -- exhaustive GPU checks of the refit fast path's arithmetic shortcuts, as
// the library compiles them (the same ssq_device.h functions, the same flags).  Test support
// only: built next to the tests, never linked into the library.
//
// counts[0..3]  div_by_const<Q>(a) != a/Q for Q = 7, 15, 127, 255, every fp32 a with
//               2^-100 <= a <= 2^100 (the range refit_fast admits)
// counts[4]     recip_rn(s) != 1/s, every fp32 s with 2^-110 <= s < 2^100 (every step the
//               admitted ranges can produce)
// counts[5]     the reference quotients themselves: a/Q from the build's fp32 division against
//               the double quotient rounded once (a correctly rounded double is never within
//               2^-53 of an fp32 midpoint here, so rounding it again is exact)
// counts[6]     negative control: q = a*RN(1/255) without the correction step, wrong somewhere
// counts[7]     negative control: v_rcp_f32 without the Newton step, wrong somewhere
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssq_device.h"

namespace {

__device__ __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b); }

// a = m * 2^e for m over all 2^23 mantissas and e in [e_lo, e_lo + n_bin)
__global__ __launch_bounds__(256) void k_check_div(int e_lo, int n_bin, unsigned long long* counts)
{
    const uint64_t total = (uint64_t)n_bin << 23;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long bad[4] = {0, 0, 0, 0}, ref_bad = 0, ctrl = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = e_lo + (int)(i >> 23);
        const float a = from_bits(((uint32_t)(e + 127) << 23) | (uint32_t)(i & 0x7FFFFFu));
        bad[0] += ssq::div_by_const<7>(a) != a / 7.0f;
        bad[1] += ssq::div_by_const<15>(a) != a / 15.0f;
        bad[2] += ssq::div_by_const<127>(a) != a / 127.0f;
        bad[3] += ssq::div_by_const<255>(a) != a / 255.0f;
        ref_bad += (float)((double)a / 255.0) != a / 255.0f;
        ctrl += a * (1.0f / 255.0f) != a / 255.0f;
    }
    for (int q = 0; q < 4; ++q)
        if (bad[q]) atomicAdd(&counts[q], bad[q]);
    if (ref_bad) atomicAdd(&counts[5], ref_bad);
    if (ctrl) atomicAdd(&counts[6], ctrl);
}

__global__ __launch_bounds__(256) void k_check_div_at(float a, unsigned long long* counts)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        counts[0] += ssq::div_by_const<7>(a) != a / 7.0f;
        counts[1] += ssq::div_by_const<15>(a) != a / 15.0f;
        counts[2] += ssq::div_by_const<127>(a) != a / 127.0f;
        counts[3] += ssq::div_by_const<255>(a) != a / 255.0f;
    }
}

__global__ __launch_bounds__(256) void k_check_rcp(int e_lo, int n_bin, unsigned long long* counts)
{
    const uint64_t total = (uint64_t)n_bin << 23;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long bad = 0, ref_bad = 0, ctrl = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = e_lo + (int)(i >> 23);
        const float s = from_bits(((uint32_t)(e + 127) << 23) | (uint32_t)(i & 0x7FFFFFu));
        const float ref = 1.0f / s;
        bad += ssq::recip_rn(s) != ref;
        ref_bad += (float)(1.0 / (double)s) != ref;
        ctrl += __builtin_amdgcn_rcpf(s) != ref;
    }
    if (bad) atomicAdd(&counts[4], bad);
    if (ref_bad) atomicAdd(&counts[5], ref_bad);
    if (ctrl) atomicAdd(&counts[7], ctrl);
}

} // namespace

// counts: 8 device words, zeroed by the caller; every launch only enqueues on `stream`
extern "C" int ssq_check_refit_shortcuts(unsigned long long* counts, hipStream_t stream)
{
    if (!counts) return 1;
    hipLaunchKernelGGL(k_check_div, dim3(16384), dim3(256), 0, stream, -100, 200, counts);
    hipLaunchKernelGGL(k_check_div_at, dim3(1), dim3(64), 0, stream, 0x1p100f, counts);
    hipLaunchKernelGGL(k_check_rcp, dim3(16384), dim3(256), 0, stream, -110, 210, counts);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// gdn_clock.hip -- measurement aid: the shader clock of the GPU while it is
// under load, for reports that state a kernel's cycles or its fraction of a
// clock-derived peak.  Each workgroup reads the shader cycle counter
// (s_memtime) and the constant 100 MHz real-time counter (s_memrealtime)
// around a spin of a given real-time length; their ratio is the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long *out, unsigned long long ticks) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    // bounded: the loop ends once `ticks` real-time ticks have passed
    while (r1 - r0 < ticks) r1 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" gdn_status gdn_clock_probe(unsigned long long *out, int nblocks, int spin_us, void *stream) {
    if (!out || nblocks < 1 || nblocks > 65536 || spin_us < 1 || spin_us > 100000) return GDN_ERR_INVALID_ARG;
    const unsigned long long ticks = (unsigned long long)spin_us * 100ull;  // 100 MHz real-time counter
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)nblocks), dim3(64), 0, (hipStream_t)stream, out, ticks);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

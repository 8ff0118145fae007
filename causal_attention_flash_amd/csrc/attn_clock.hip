// Shader-clock samples for measurement (attn_clock_sample in include/attn.h).
//
// A cold GPU runs at a lower DVFS clock state, and a throughput figure means
// little without the clock it ran at (Iron "Kernel Engineering Guide", §6.1: warm
// the clock before the first sample).  Each workgroup of this kernel records,
// from its first lane, the shader-cycle counter (s_memtime, which advances at the
// current shader clock), the constant 100 MHz counter (s_memrealtime) and the id
// of the XCC it ran on.  Two samples around a timed region give each XCC's
// average shader clock over the region: cycles / (ticks / 100 MHz).
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace attn {

__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t* __restrict__ out) {
    if (threadIdx.x != 0) return;
    const uint64_t cycles = __builtin_amdgcn_s_memtime();
    const uint64_t ticks = __builtin_amdgcn_s_memrealtime();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    out[blockIdx.x * 4 + 0] = cycles;
    out[blockIdx.x * 4 + 1] = ticks;
    out[blockIdx.x * 4 + 2] = xcc & 0xfu;
    out[blockIdx.x * 4 + 3] = 0;
}

}  // namespace attn

extern "C" attn_status attn_clock_sample(uint64_t* out, int64_t n, void* stream) {
    if (n < 1 || n > ATTN_CLOCK_SAMPLE_MAX) return ATTN_ERR_SHAPE;
    if (!out) return ATTN_ERR_NULL;
    if (((uintptr_t)out & 15u) != 0) return ATTN_ERR_ALIGNMENT;
    hipLaunchKernelGGL(attn::clock_sample_kernel, dim3((unsigned)n), dim3(64), 0, (hipStream_t)stream, out);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

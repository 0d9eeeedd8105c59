// Shader-clock probe for the bench (libtplclock.so, not part of the
// tensor-parallel ABI).  MI355X lowers its shader clock under sustained
// matrix-core load, so a TFLOP/s figure alone does not say how close a GEMM
// runs to what the chip can issue at the clock it actually ran at.
//
// Each block is one wave.  It waits `delay` ticks of the 100 MHz constant
// real-time counter (s_memrealtime), then counts shader-clock ticks
// (s_memtime) over `window` real-time ticks, and writes the two tick counts
// to out[2*b], out[2*b+1] with a vector store.  Launched on a second stream
// next to a running kernel it co-resides with that kernel's workgroups (64
// threads, no LDS, a few registers) and reads the clock the chip runs at
// meanwhile.  Both waits end when the real-time counter passes their bound.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__global__ void clock_probe_kernel(unsigned long long *out, unsigned delay, unsigned window) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - r0 < delay) __builtin_amdgcn_s_sleep(20);
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - r1 < window) __builtin_amdgcn_s_sleep(20);
    const unsigned long long c2 = __builtin_amdgcn_s_memtime();
    const unsigned long long r2 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c2 - c1;
        out[2 * blockIdx.x + 1] = r2 - r1;
    }
}

}  // namespace

// out: device buffer of 2*nblocks uint64 (shader ticks, real-time ticks per
// block).  delay/window in 100 MHz real-time ticks.  Returns a hipError_t.
extern "C" int tp_clock_probe(unsigned long long *out, int nblocks, unsigned delay,
                              unsigned window, hipStream_t stream) {
    if (out == nullptr || nblocks <= 0 || nblocks > 1024) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(nblocks), dim3(64), 0, stream, out, delay, window);
    return (int)hipGetLastError();
}

// clock_probe.hip -- test infrastructure: samples the shader clock while
// other kernels run on another stream.  Not part of the library; shares no
// code with it.
#include <hip/hip_runtime.h>
#include <stdint.h>

// One wave per workgroup; lane 0 takes nsamp samples, one every `period`
// ticks of the constant 100 MHz counter (s_memrealtime), of that counter and
// of the shader-clock counter (s_memtime), each as an offset from the wave's
// first reading: out[(wg * nsamp + i) * 2 + {0, 1}].  Every wave ends after
// nsamp * period ticks.
__global__ void clock_monitor(unsigned long long* out, int nsamp, unsigned period) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_readcyclecounter();
  unsigned long long* o = out + (size_t)blockIdx.x * nsamp * 2;
  for (int i = 0; i < nsamp; ++i) {
    const unsigned long long target = r0 + (unsigned long long)(i + 1) * period;
    unsigned long long r = __builtin_amdgcn_s_memrealtime();
    while (r < target) {
      __builtin_amdgcn_s_sleep(2);
      r = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long c = __builtin_readcyclecounter();
    o[2 * i] = r - r0;
    o[2 * i + 1] = c - c0;
  }
}

// out: nwg * nsamp * 2 uint64 on the device; stream: a hipStream_t (null:
// the default stream).  The waves run for nsamp * period / 100 MHz.
extern "C" int probe_clock_monitor(void* out, int nwg, int nsamp, unsigned period, void* stream) {
  if (nwg <= 0 || nsamp <= 0 || period == 0) return -1;
  hipLaunchKernelGGL(clock_monitor, dim3(nwg), dim3(64), 0, (hipStream_t)stream,
                     (unsigned long long*)out, nsamp, period);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

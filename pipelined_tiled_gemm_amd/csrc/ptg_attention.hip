// ptg_attention.hip - the IKBO attention kernel (ptg_attention.hpp) and its watchdog word, in a
// translation unit of its own: it is compiled with the backend's default instruction
// scheduler, while the GEMM kernels take the latency-oriented one (the build script gives
// each source its flags).
#include <hip/hip_runtime.h>

#include "ptg_attention.hpp"

namespace ptg {

hipError_t read_attention_watchdog(uint32_t* value, int clear) {
  hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(g_watchdog), sizeof(uint32_t), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_watchdog), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice);
}

}  // namespace ptg

// Measurement helper of libstc for gfx950: a plain streaming copy, the
// practical ceiling of a read + write pattern beside which the codec kernels'
// rates are read. It computes nothing of the method.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "stc_internal.h"

namespace stc {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));

// 16-byte loads, four in flight per thread over a grid-stride loop,
// non-temporal 16-byte stores; 2048 workgroups of 256 threads (eight per CU).
__global__ void __launch_bounds__(256) k_stream_copy(const u32x4c* __restrict__ src, u32x4c* __restrict__ dst,
                                                     long long n16) {
  const long long nth = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * nth < n16; i += 4 * nth) {
    const u32x4c v0 = src[i], v1 = src[i + nth], v2 = src[i + 2 * nth], v3 = src[i + 3 * nth];
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + nth);
    __builtin_nontemporal_store(v2, dst + i + 2 * nth);
    __builtin_nontemporal_store(v3, dst + i + 3 * nth);
  }
  for (; i < n16; i += nth) __builtin_nontemporal_store(src[i], dst + i);
}

int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  hipLaunchKernelGGL(k_stream_copy, dim3(2048), dim3(256), 0, (hipStream_t)stream, static_cast<const u32x4c*>(src),
                     static_cast<u32x4c*>(dst), (long long)(bytes / 16));
  return hipGetLastError() != hipSuccess;
}

}  // namespace stc

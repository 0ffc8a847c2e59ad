// Zero-copy notification of the host (PSA, section 3.3: once the
// accumulated weight passes the threshold, the GPU writes a signal variable
// into pinned host memory, so the CPU learns of it asynchronously, with no
// device synchronisation).
//
// One workgroup, enqueued after the producing kernels on their stream: it
// copies n int32 values (e.g. the per-(sequence, head) page counts of the
// progressive selection) into pinned host memory with system-scope stores,
// makes them visible system-wide, then writes the sequence number `seq` to
// the host flag with a system-scope release.  A host that sees flag == seq
// also sees the values.
#include "dsa_host.hpp"

namespace dsa {

__global__ __launch_bounds__(256) void signal_host_kernel(const int32_t* __restrict__ src, int n,
                                                          int32_t* host_dst, int32_t* host_flag, int seq) {
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    __hip_atomic_store(&host_dst[i], src[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(host_flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_signal_host(const int32_t* src, int32_t n, int32_t* host_dst, int32_t* host_flag, int32_t seq,
                               void* stream) {
  if (n < 0) return DSA_ERR_SHAPE;
  if (!host_flag || (n > 0 && (!src || !host_dst))) return DSA_ERR_NULL;
  hipLaunchKernelGGL(signal_host_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, src, (int)n, host_dst,
                     host_flag, (int)seq);
  return launch_status();
}

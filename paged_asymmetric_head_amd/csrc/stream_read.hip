// A plain streaming read of one device buffer: the achievable-bandwidth
// reference that the KV-read rates of the attention kernels are quoted
// against beside HBM peak.  Measurement infrastructure only: it lives in its
// own library (libdiffkv_stream.so), outside the attention ABI.
//
// Every thread reads 16-byte pieces in a grid-stride loop, 4 or 8
// independent loads per trip, XORs them into one register and stores that
// once, so the loads cannot be dropped and the kernel moves only the
// buffer's bytes in (plus 4 bytes per thread out).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(src[i]);
  sink[tid] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, src 16-byte aligned) with `blocks`
// workgroups of 256 threads, `unroll` (4 or 8) loads in flight per thread,
// on `stream`; sink receives blocks * 256 words.  Returns 0, 1 for an
// invalid argument, 2 for a launch error.
int diffkv_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int unroll,
                       hipStream_t stream) {
  if (!src || !sink || blocks <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (unroll != 4 && unroll != 8))
    return 1;
  const u32x4* s = static_cast<const u32x4*>(src);
  size_t n16 = bytes / 16;
  void* args[] = {&s, &n16, &sink};
  const void* fn = unroll == 8 ? reinterpret_cast<const void*>(&stream_read_kernel<8>)
                               : reinterpret_cast<const void*>(&stream_read_kernel<4>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, stream) == hipSuccess ? 0 : 2;
}

}  // extern "C"

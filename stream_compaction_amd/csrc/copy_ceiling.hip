// Measurement aid, not part of the scan library: a plain 16-byte-vector copy
// kernel.  The benchmark times it over the same number of bytes a scan moves
// (its practical HBM ceiling) and the hardware-counter runs use it as the
// reference of known size that calibrates FETCH_SIZE / WRITE_SIZE.  Its shape
// is the fastest plain copy measured on MI355X: one nontemporal 16-byte load
// and store per thread, 256-thread workgroups.  Built into its own library,
// libscan_copy.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlock) void copy16_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Copy `bytes` (a multiple of 16) between 16-byte-aligned device buffers on
// `stream`.  Returns the hipError_t of the launch (0 on success); bad
// arguments return hipErrorInvalidValue without launching.
int copy_ceiling_copy16(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return (int)hipErrorInvalidValue;
  if (bytes == 0) return 0;
  const int64_t nvec = bytes / 16;
  const int64_t blocks = (nvec + kBlock - 1) / kBlock;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  copy16_kernel<<<dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)stream>>>(
      (const u32x4*)src, (u32x4*)dst, nvec);
  return (int)hipGetLastError();
}

}  // extern "C"

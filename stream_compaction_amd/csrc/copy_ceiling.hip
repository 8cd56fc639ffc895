// Measurement aid, not part of the scan library: a plain 16-byte-vector copy
// kernel.  The benchmark times it over the same number of bytes a scan moves
// (its practical HBM ceiling) and the hardware-counter runs use it as the
// reference of known size that calibrates FETCH_SIZE / WRITE_SIZE.  Its shape
// is the fastest plain copy measured on MI355X over 1 GiB each way (three
// buffer sets rotated): one 16-byte load (nontemporal) and one 16-byte store
// (sc1 cache policy) per thread, 64-thread workgroups, 6.78 TB/s; 256-thread
// groups with nontemporal stores reached 6.45 TB/s.  Built into its own
// library, libscan_copy.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 64;
constexpr int kNT = 2;      // buffer cache-policy bits: nontemporal
constexpr int kSC1 = 16;    // buffer cache-policy bits: sc1
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b copies the 16-byte vectors [b*64, b*64 + 64) that lie below nvec.
__global__ __launch_bounds__(kBlock) void copy16_kernel(uintptr_t src, uintptr_t dst, int64_t nvec) {
  const int64_t v0 = (int64_t)blockIdx.x * kBlock;
  const int64_t left = nvec - v0;
  const int nrec = (int)((left < kBlock ? left : kBlock) * 16);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(src + v0 * 16), (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t w =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dst + v0 * 16), (short)0, nrec, 0x00020000);
  const u32x4 v = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, threadIdx.x * 16, 0, kNT));
  __builtin_amdgcn_raw_buffer_store_b128(v, w, threadIdx.x * 16, 0, kSC1);
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
  if (blocks * kBlock >= (1ll << 32)) return (int)hipErrorInvalidValue;   // 32-bit work-item count
  copy16_kernel<<<dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)stream>>>(
      (uintptr_t)src, (uintptr_t)dst, nvec);
  return (int)hipGetLastError();
}

}  // extern "C"

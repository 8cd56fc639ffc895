// Internal host-side interface between the C ABI (api.cpp) and the kernel
// translation units.  Arguments reaching these launchers are already
// validated; each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sca {

enum class Fmt : int { F32, F16, BF16, F64, I32, U32, I64, U64 };

// Workgroup size of every kernel (four wave64s).
constexpr int kBlock = 256;

// Row-wise scan; op: 0 add, 1 min, 2 max, 3 mul (floating formats).
hipError_t launch_scan_rows(const void* in, void* out, int64_t rows, int64_t n, Fmt fmt, int op,
                            bool exclusive, hipStream_t stream);

// Device-wide exclusive (or inclusive) scan; op: 0 add, 1 min, 2 max.
size_t scan_device_tiles(int64_t n, Fmt fmt);       // descriptors needed
// n_dev (all launchers below): when not null, the live count is read from it
// on the device and clamped to [0, n]; n is then the capacity that grids and
// scratch are sized for.
// descs_clear: the caller has already zeroed the first scan_device_tiles(n,
// fmt) descriptors of `scratch` earlier on `stream`, so no fill kernel runs.
hipError_t launch_scan_device(const void* in, void* out, int64_t n, Fmt fmt, int op,
                              bool inclusive, void* scratch, hipStream_t stream,
                              const int32_t* n_dev = nullptr, bool descs_clear = false);

// Device-wide reduction into out[0]; op: 0 add, 1 min, 2 max.  n == 0 writes
// the identity.  Scratch holds one partial per workgroup of the first launch.
size_t reduce_partials(int64_t n, Fmt fmt);         // partials (8-byte slots) needed
hipError_t launch_reduce(const void* in, void* out, int64_t n, Fmt fmt, int op, void* scratch,
                         hipStream_t stream, const int32_t* n_dev = nullptr);

// Reduce-by-key (32-bit keys and values): one descriptor (four 64-bit words)
// per tile.
size_t reduce_by_key_tiles(int64_t n);
hipError_t launch_reduce_by_key(const void* keys, const void* values, void* keys_out,
                                void* values_out, int32_t* num_runs, int64_t n, Fmt kfmt,
                                Fmt vfmt, void* scratch, hipStream_t stream,
                                const int32_t* n_dev = nullptr);

// Radix sort (0 <= n <= INT32_MAX); value_bytes 0 (keys only), 4 or 8.
size_t radix_sort_scratch(int64_t n, size_t key_bytes);
hipError_t launch_radix_sort(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                             Fmt kfmt, int value_bytes, int end_bit, void* scratch,
                             hipStream_t stream, const int32_t* n_dev = nullptr);

// Stream compaction.
size_t select_tiles(int64_t n, size_t elem_bytes);
hipError_t launch_select(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                         int64_t n, size_t elem_bytes, void* scratch, hipStream_t stream,
                         const int32_t* n_dev = nullptr);

// Scratch of the look-back kernels holds only the tile descriptors, one per
// 128-byte line (kDescBytes), whose used words are zeroed at the start of
// every call by a small fill kernel (no hipMemsetAsync, so the call can sit
// in a captured graph).
// The descriptors start at the first 128-byte boundary of the caller's
// (16-byte aligned) scratch, so scratch sizes carry one line of slack.
constexpr size_t kDescBytes = 128;
inline size_t desc_scratch_bytes(size_t ntiles) {
  return ntiles == 0 ? 0 : ntiles * kDescBytes + kDescBytes;
}
inline uint64_t* desc_base(void* scratch) {
  return (uint64_t*)(((uintptr_t)scratch + kDescBytes - 1) & ~(uintptr_t)(kDescBytes - 1));
}
hipError_t launch_fill_desc(uint64_t* desc, int64_t ntiles, int words, hipStream_t stream);

// The allocation-free device scan keeps its descriptors in a static device
// array of this many bytes per GPU; noalloc_scratch() returns the current
// device's copy (hipGetSymbolAddress, once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace sca

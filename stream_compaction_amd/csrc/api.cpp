// C ABI of libscan_amd.so (declared in include/scan.h): host-side validation,
// then one launcher call.  Nothing here allocates, frees or synchronizes.
#include "../../include/scan.h"

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool fmt_of(scan_dtype d, sca::Fmt* f, size_t* bytes) {
  switch (d) {
    case SCAN_F32: *f = sca::Fmt::F32; *bytes = 4; return true;
    case SCAN_F16: *f = sca::Fmt::F16; *bytes = 2; return true;
    case SCAN_BF16: *f = sca::Fmt::BF16; *bytes = 2; return true;
    case SCAN_F64: *f = sca::Fmt::F64; *bytes = 8; return true;
    case SCAN_I32: *f = sca::Fmt::I32; *bytes = 4; return true;
    case SCAN_U32: *f = sca::Fmt::U32; *bytes = 4; return true;
    case SCAN_I64: *f = sca::Fmt::I64; *bytes = 8; return true;
    case SCAN_U64: *f = sca::Fmt::U64; *bytes = 8; return true;
  }
  return false;
}

int op_index(scan_op op) {
  switch (op) {
    case SCAN_ADD: return 0;
    case SCAN_MIN: return 1;
    case SCAN_MAX: return 2;
    case SCAN_MUL: return 3;
  }
  return -1;
}

// Half-open byte ranges [a, a + na) and [b, b + nb) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round16(size_t b) { return (b + 15) & ~(size_t)15; }

// The device count of the *_devn entry points: present, 4-byte aligned and
// outside every range the call writes (each workgroup reads it once, so the
// call must not change it).
scan_status devn_check(const int32_t* n_dev, const void* const* written, const size_t* sizes,
                       int count) {
  if (n_dev == nullptr || !aligned(n_dev, 4)) return SCAN_EINVAL;
  for (int i = 0; i < count; ++i)
    if (overlap(n_dev, 4, written[i], sizes[i])) return SCAN_EALIAS;
  return SCAN_OK;
}

scan_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SCAN_OK;
  g_last_hip_error = (int)e;
  return SCAN_EHIP;
}

constexpr int64_t kMaxN = 2147483647;  // INT32_MAX

}  // namespace

extern "C" {

const char* scan_status_str(scan_status s) {
  switch (s) {
    case SCAN_OK: return "ok";
    case SCAN_EINVAL: return "invalid argument";
    case SCAN_ENOTSUP: return "unsupported dtype/op";
    case SCAN_EALIAS: return "argument ranges overlap";
    case SCAN_ESCRATCH: return "scratch too small";
    case SCAN_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

int scan_last_hip_error(void) { return g_last_hip_error; }

scan_status scan_rows(const void* in, void* out, int64_t rows, int64_t n, scan_dtype dtype,
                      scan_op op, int exclusive, void* stream) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb)) return SCAN_ENOTSUP;
  if (fmt != sca::Fmt::F32 && fmt != sca::Fmt::F16 && fmt != sca::Fmt::BF16) return SCAN_ENOTSUP;
  const int opi = op_index(op);
  if (opi < 0) return SCAN_ENOTSUP;
  if (exclusive != 0 && exclusive != 1) return SCAN_EINVAL;
  if (rows < 0 || n < 0 || rows > kMaxN || n > kMaxN) return SCAN_EINVAL;
  if (rows == 0 || n == 0) return SCAN_OK;
  if (in == nullptr || out == nullptr) return SCAN_EINVAL;
  if (!aligned(in, eb) || !aligned(out, eb)) return SCAN_EINVAL;
  const size_t bytes = (size_t)rows * (size_t)n * eb;
  if (overlap(in, bytes, out, bytes)) return SCAN_EALIAS;
  return hip_status(sca::launch_scan_rows(in, out, rows, n, fmt, opi, exclusive == 1,
                                          (hipStream_t)stream));
}

size_t scan_device_scratch_bytes(int64_t n, scan_dtype dtype) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb) || n < 0) return 0;
  return sca::desc_scratch_bytes(sca::scan_device_tiles(n, fmt));
}

static scan_status scan_device_any(const void* in, void* out, int64_t n, scan_dtype dtype,
                                   scan_op op, bool inclusive, void* scratch,
                                   size_t scratch_bytes, void* stream, bool devn,
                                   const int32_t* n_dev) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb)) return SCAN_ENOTSUP;
  if (fmt == sca::Fmt::F16 || fmt == sca::Fmt::BF16) return SCAN_ENOTSUP;
  const int opi = op_index(op);
  if (opi < 0 || opi > 2) return SCAN_ENOTSUP;
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  if (n == 0) return SCAN_OK;
  if (in == nullptr || out == nullptr || scratch == nullptr) return SCAN_EINVAL;
  if (!aligned(in, eb) || !aligned(out, eb) || !aligned(scratch, 16)) return SCAN_EINVAL;
  const size_t need = scan_device_scratch_bytes(n, dtype);
  if (scratch_bytes < need) return SCAN_ESCRATCH;
  const size_t bytes = (size_t)n * eb;
  if (overlap(in, bytes, out, bytes)) return SCAN_EALIAS;
  if (overlap(scratch, need, in, bytes) || overlap(scratch, need, out, bytes)) return SCAN_EALIAS;
  if (devn) {
    const void* w[2] = {out, scratch};
    const size_t z[2] = {bytes, need};
    const scan_status dv = devn_check(n_dev, w, z, 2);
    if (dv != SCAN_OK) return dv;
  }
  return hip_status(sca::launch_scan_device(in, out, n, fmt, opi, inclusive, scratch,
                                            (hipStream_t)stream, n_dev));
}

scan_status scan_device(const void* in, void* out, int64_t n, scan_dtype dtype, scan_op op,
                        void* scratch, size_t scratch_bytes, void* stream) {
  return scan_device_any(in, out, n, dtype, op, false, scratch, scratch_bytes, stream, false,
                         nullptr);
}

scan_status scan_device_devn(const void* in, void* out, const int32_t* n_live, int64_t capacity,
                             scan_dtype dtype, scan_op op, void* scratch, size_t scratch_bytes,
                             void* stream) {
  if (n_live == nullptr) return SCAN_EINVAL;
  return scan_device_any(in, out, capacity, dtype, op, false, scratch, scratch_bytes, stream, true,
                         n_live);
}

static_assert(SCAN_NOALLOC_SCRATCH_BYTES == sca::kNoAllocScratchBytes,
              "the header states the static scratch size");

scan_status scan_device_noalloc(const void* in, void* out, int64_t n, scan_dtype dtype,
                                scan_op op, void* stream) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb)) return SCAN_ENOTSUP;
  if (fmt == sca::Fmt::F16 || fmt == sca::Fmt::BF16) return SCAN_ENOTSUP;
  const int opi = op_index(op);
  if (opi < 0 || opi > 2) return SCAN_ENOTSUP;
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  // the static scratch bounds n: rejected before any pointer is looked at
  if (scan_device_scratch_bytes(n, dtype) > SCAN_NOALLOC_SCRATCH_BYTES) return SCAN_ESCRATCH;
  if (n == 0) return SCAN_OK;
  if (in == nullptr || out == nullptr) return SCAN_EINVAL;
  if (!aligned(in, eb) || !aligned(out, eb)) return SCAN_EINVAL;
  const size_t bytes = (size_t)n * eb;
  if (overlap(in, bytes, out, bytes)) return SCAN_EALIAS;
  void* scratch = nullptr;
  const hipError_t e = sca::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(sca::launch_scan_device(in, out, n, fmt, opi, false, scratch,
                                            (hipStream_t)stream));
}

scan_status scan_device_inclusive(const void* in, void* out, int64_t n, scan_dtype dtype,
                                  scan_op op, void* scratch, size_t scratch_bytes,
                                  void* stream) {
  return scan_device_any(in, out, n, dtype, op, true, scratch, scratch_bytes, stream, false,
                         nullptr);
}

scan_status scan_device_inclusive_devn(const void* in, void* out, const int32_t* n_live,
                                       int64_t capacity, scan_dtype dtype, scan_op op,
                                       void* scratch, size_t scratch_bytes, void* stream) {
  if (n_live == nullptr) return SCAN_EINVAL;
  return scan_device_any(in, out, capacity, dtype, op, true, scratch, scratch_bytes, stream, true,
                         n_live);
}

size_t reduce_device_scratch_bytes(int64_t n, scan_dtype dtype) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb) || n < 0) return 0;
  return round16(sca::reduce_partials(n, fmt) * 8);
}

static scan_status reduce_any(const void* in, void* out, int64_t n, scan_dtype dtype, scan_op op,
                              void* scratch, size_t scratch_bytes, void* stream, bool devn,
                              const int32_t* n_dev) {
  sca::Fmt fmt;
  size_t eb;
  if (!fmt_of(dtype, &fmt, &eb)) return SCAN_ENOTSUP;
  if (fmt == sca::Fmt::F16 || fmt == sca::Fmt::BF16) return SCAN_ENOTSUP;
  const int opi = op_index(op);
  if (opi < 0 || opi > 2) return SCAN_ENOTSUP;
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  if (out == nullptr || !aligned(out, eb)) return SCAN_EINVAL;
  const size_t need = reduce_device_scratch_bytes(n, dtype);
  if (n > 0) {
    if (in == nullptr || scratch == nullptr) return SCAN_EINVAL;
    if (!aligned(in, eb) || !aligned(scratch, 16)) return SCAN_EINVAL;
    if (scratch_bytes < need) return SCAN_ESCRATCH;
    const size_t bytes = (size_t)n * eb;
    if (overlap(in, bytes, out, eb)) return SCAN_EALIAS;
    if (overlap(scratch, need, in, bytes) || overlap(scratch, need, out, eb)) return SCAN_EALIAS;
  }
  if (devn) {
    const void* w[2] = {out, scratch};
    const size_t z[2] = {eb, n > 0 ? need : 0};
    const scan_status dv = devn_check(n_dev, w, z, 2);
    if (dv != SCAN_OK) return dv;
  }
  return hip_status(
      sca::launch_reduce(in, out, n, fmt, opi, scratch, (hipStream_t)stream, n_dev));
}

scan_status reduce_device(const void* in, void* out, int64_t n, scan_dtype dtype, scan_op op,
                          void* scratch, size_t scratch_bytes, void* stream) {
  return reduce_any(in, out, n, dtype, op, scratch, scratch_bytes, stream, false, nullptr);
}

scan_status reduce_device_devn(const void* in, void* out, const int32_t* n_live, int64_t capacity,
                               scan_dtype dtype, scan_op op, void* scratch, size_t scratch_bytes,
                               void* stream) {
  if (n_live == nullptr) return SCAN_EINVAL;
  return reduce_any(in, out, capacity, dtype, op, scratch, scratch_bytes, stream, true, n_live);
}

size_t reduce_by_key_scratch_bytes(int64_t n) {
  if (n < 0) return 0;
  return sca::desc_scratch_bytes(sca::reduce_by_key_tiles(n));
}

static scan_status rbk_any(const void* keys_in, const void* values_in, void* keys_out,
                           void* values_out, int32_t* num_runs, int64_t n, scan_dtype key_dtype,
                           scan_dtype value_dtype, void* scratch, size_t scratch_bytes,
                           void* stream, bool devn, const int32_t* n_dev) {
  sca::Fmt kf, vf;
  size_t keb, veb;
  if (!fmt_of(key_dtype, &kf, &keb) || !fmt_of(value_dtype, &vf, &veb)) return SCAN_ENOTSUP;
  auto ok32 = [](sca::Fmt f) {
    return f == sca::Fmt::I32 || f == sca::Fmt::U32 || f == sca::Fmt::F32;
  };
  if (!ok32(kf) || !ok32(vf)) return SCAN_ENOTSUP;
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  if (num_runs == nullptr || !aligned(num_runs, 4)) return SCAN_EINVAL;
  if (n > 0) {
    if (keys_in == nullptr || values_in == nullptr || keys_out == nullptr ||
        values_out == nullptr || scratch == nullptr)
      return SCAN_EINVAL;
    if (!aligned(keys_in, 4) || !aligned(values_in, 4) || !aligned(keys_out, 4) ||
        !aligned(values_out, 4) || !aligned(scratch, 16))
      return SCAN_EINVAL;
    const size_t need = reduce_by_key_scratch_bytes(n);
    if (scratch_bytes < need) return SCAN_ESCRATCH;
    const size_t bytes = (size_t)n * 4;
    // the two inputs may share memory (both are only read); nothing else may
    const void* r[6] = {keys_in, values_in, keys_out, values_out, num_runs, scratch};
    const size_t z[6] = {bytes, bytes, bytes, bytes, 4, need};
    for (int a = 0; a < 6; ++a)
      for (int b = a + 1; b < 6; ++b)
        if (!(a == 0 && b == 1) && overlap(r[a], z[a], r[b], z[b])) return SCAN_EALIAS;
  }
  if (devn) {
    const size_t bytes = (size_t)n * 4;
    const void* w[4] = {keys_out, values_out, num_runs, scratch};
    const size_t z[4] = {bytes, bytes, 4, n > 0 ? reduce_by_key_scratch_bytes(n) : 0};
    const scan_status dv = devn_check(n_dev, w, z, 4);
    if (dv != SCAN_OK) return dv;
  }
  return hip_status(sca::launch_reduce_by_key(keys_in, values_in, keys_out, values_out, num_runs,
                                              n, kf, vf, scratch, (hipStream_t)stream, n_dev));
}

scan_status reduce_by_key(const void* keys_in, const void* values_in, void* keys_out,
                          void* values_out, int32_t* num_runs, int64_t n, scan_dtype key_dtype,
                          scan_dtype value_dtype, void* scratch, size_t scratch_bytes,
                          void* stream) {
  return rbk_any(keys_in, values_in, keys_out, values_out, num_runs, n, key_dtype, value_dtype,
                 scratch, scratch_bytes, stream, false, nullptr);
}

scan_status reduce_by_key_devn(const void* keys_in, const void* values_in, void* keys_out,
                               void* values_out, int32_t* num_runs, const int32_t* n_live,
                               int64_t capacity, scan_dtype key_dtype, scan_dtype value_dtype,
                               void* scratch, size_t scratch_bytes, void* stream) {
  if (n_live == nullptr) return SCAN_EINVAL;
  return rbk_any(keys_in, values_in, keys_out, values_out, num_runs, capacity, key_dtype,
                 value_dtype, scratch, scratch_bytes, stream, true, n_live);
}

size_t radix_sort_scratch_bytes(int64_t n, scan_dtype key_dtype) {
  sca::Fmt f;
  size_t eb;
  if (!fmt_of(key_dtype, &f, &eb) || eb < 4 || n < 0) return 0;
  return round16(sca::radix_sort_scratch(n, eb));
}

static scan_status sort_any(void* keys, void* tmp_keys, void* values, void* tmp_values,
                            int64_t n, scan_dtype key_dtype, scan_dtype value_dtype, int end_bit,
                            void* scratch, size_t scratch_bytes, void* stream, bool devn,
                            const int32_t* n_dev) {
  sca::Fmt kf, vf;
  size_t keb, veb = 0;
  if (!fmt_of(key_dtype, &kf, &keb) || keb < 4) return SCAN_ENOTSUP;
  if (values != nullptr || tmp_values != nullptr) {
    if (!fmt_of(value_dtype, &vf, &veb) || veb < 4) return SCAN_ENOTSUP;
    if (values == nullptr || tmp_values == nullptr) return SCAN_EINVAL;
  }
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  if (end_bit < 8 || end_bit > (int)(8 * keb) || end_bit % 8 != 0) return SCAN_EINVAL;
  if (devn && (end_bit / 8) % 2 != 0) return SCAN_EINVAL;   // the result must land in keys
  if (devn && n_dev == nullptr) return SCAN_EINVAL;
  if (n <= 1) return SCAN_OK;
  if (keys == nullptr || tmp_keys == nullptr || scratch == nullptr) return SCAN_EINVAL;
  if (!aligned(keys, keb) || !aligned(tmp_keys, keb) || !aligned(scratch, 16)) return SCAN_EINVAL;
  if (veb && (!aligned(values, veb) || !aligned(tmp_values, veb))) return SCAN_EINVAL;
  const size_t need = radix_sort_scratch_bytes(n, key_dtype);
  if (scratch_bytes < need) return SCAN_ESCRATCH;
  const size_t kb = (size_t)n * keb, vb = (size_t)n * veb;
  const void* r[5] = {keys, tmp_keys, values, tmp_values, scratch};
  const size_t z[5] = {kb, kb, vb, vb, need};
  for (int a = 0; a < 5; ++a)
    for (int b = a + 1; b < 5; ++b)
      if (overlap(r[a], z[a], r[b], z[b])) return SCAN_EALIAS;
  if (devn) {
    const scan_status dv = devn_check(n_dev, r, z, 5);
    if (dv != SCAN_OK) return dv;
  }
  return hip_status(sca::launch_radix_sort(keys, tmp_keys, values, tmp_values, n, kf, (int)veb,
                                           end_bit, scratch, (hipStream_t)stream, n_dev));
}

scan_status radix_sort(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                       scan_dtype key_dtype, scan_dtype value_dtype, int end_bit, void* scratch,
                       size_t scratch_bytes, void* stream) {
  return sort_any(keys, tmp_keys, values, tmp_values, n, key_dtype, value_dtype, end_bit, scratch,
                  scratch_bytes, stream, false, nullptr);
}

scan_status radix_sort_devn(void* keys, void* tmp_keys, void* values, void* tmp_values,
                            const int32_t* n_live, int64_t capacity, scan_dtype key_dtype,
                            scan_dtype value_dtype, int end_bit, void* scratch,
                            size_t scratch_bytes, void* stream) {
  return sort_any(keys, tmp_keys, values, tmp_values, capacity, key_dtype, value_dtype, end_bit,
                  scratch, scratch_bytes, stream, true, n_live);
}

size_t select_compact_scratch_bytes(int64_t n) {
  if (n < 0) return 0;
  return sca::desc_scratch_bytes(sca::select_tiles(n, 16));
}

static scan_status select_any(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                              int64_t n, size_t elem_bytes, void* scratch, size_t scratch_bytes,
                              void* stream, bool devn, const int32_t* n_dev) {
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 &&
      elem_bytes != 16)
    return SCAN_ENOTSUP;
  if (n < 0 || n > kMaxN) return SCAN_EINVAL;
  if (num_out == nullptr || !aligned(num_out, 4)) return SCAN_EINVAL;
  if (n > 0) {
    if (in == nullptr || flags == nullptr || out == nullptr || scratch == nullptr)
      return SCAN_EINVAL;
    if (!aligned(in, elem_bytes) || !aligned(out, elem_bytes) || !aligned(scratch, 16))
      return SCAN_EINVAL;
    const size_t need = select_compact_scratch_bytes(n);
    if (scratch_bytes < need) return SCAN_ESCRATCH;
    const size_t bytes = (size_t)n * elem_bytes;
    const void* ranges[4] = {in, flags, num_out, scratch};
    const size_t sizes[4] = {bytes, (size_t)n, 4, need};
    for (int a = 0; a < 4; ++a)
      for (int b = a + 1; b < 4; ++b)
        if (overlap(ranges[a], sizes[a], ranges[b], sizes[b]) && !(a <= 1 && b <= 1))
          return SCAN_EALIAS;
    for (int a = 0; a < 4; ++a)
      if (overlap(out, bytes, ranges[a], sizes[a])) return SCAN_EALIAS;
  }
  if (devn) {
    const void* w[3] = {out, num_out, scratch};
    const size_t z[3] = {(size_t)n * elem_bytes, 4, n > 0 ? select_compact_scratch_bytes(n) : 0};
    const scan_status dv = devn_check(n_dev, w, z, 3);
    if (dv != SCAN_OK) return dv;
  }
  return hip_status(sca::launch_select(in, flags, out, num_out, n, elem_bytes, scratch,
                                       (hipStream_t)stream, n_dev));
}

scan_status select_compact(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                           int64_t n, size_t elem_bytes, void* scratch, size_t scratch_bytes,
                           void* stream) {
  return select_any(in, flags, out, num_out, n, elem_bytes, scratch, scratch_bytes, stream, false,
                    nullptr);
}

scan_status select_compact_devn(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                                const int32_t* n_live, int64_t capacity, size_t elem_bytes,
                                void* scratch, size_t scratch_bytes, void* stream) {
  if (n_live == nullptr) return SCAN_EINVAL;
  return select_any(in, flags, out, num_out, capacity, elem_bytes, scratch, scratch_bytes, stream,
                    true, n_live);
}

}  // extern "C"

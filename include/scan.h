/*
 * scan.h - C ABI of the stream_compaction_amd library (libscan_amd.so):
 * row-wise prefix scan, device-wide exclusive and inclusive scan, device-wide
 * reduction, reduce-by-key, radix sort and stream compaction on one AMD
 * Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer (in, out, flags, num_out, scratch) is a DEVICE pointer
 *    owned by the caller.  The library never allocates, frees or
 *    synchronizes: all work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream) and the call returns as soon as it
 *    is enqueued.  Results are visible to later work on the same stream.
 *    Nothing is read back to the host (the "Algorithms" page, Quadrants user
 *    guide, section "Key sizing parameters": no host round-trip).
 *  - Arguments are validated on the host BEFORE anything is enqueued; a
 *    non-OK status means nothing was launched and no memory was touched.
 *  - Pointers must be aligned to their element size.  Ranges of different
 *    arguments must not overlap (SCAN_EALIAS); this refines the rule that an
 *    exclusive scan's output must be a distinct buffer from its input
 *    ("Algorithms" page, section qd.algorithms.exclusive_scan_{add,min,max},
 *    its list of constraints).
 *  - Input arrays are read in whole 16-byte vectors, which may include bytes
 *    just outside an array's range but never outside the 128-byte lines that
 *    hold its first and last bytes (so never outside their pages); those
 *    bytes are ignored.  Nothing outside an output array's range is ever
 *    written.
 *  - Sizes: 0 <= n <= INT32_MAX (the pages index and count with 32-bit
 *    integers: "Algorithms" page, section "Capacity (log256_max_n)", and the
 *    i32 count of select).  n == 0 (or rows == 0) is a valid no-op ("Tile
 *    operations and reductions", section "Why not just infer it from
 *    reduce?": empty input gives empty output).
 *  - Scratch ("Algorithms" page, section "Scratch space"): caller-owned, sized
 *    with the matching *_scratch_bytes() helper (host-only integer
 *    arithmetic), needs no initialization; the library clears what it needs
 *    at the start of each call with a small fill kernel on `stream`.  Two
 *    calls that are in flight at the same time must use different scratch
 *    buffers.  Scratch must be 16-byte aligned.
 *  - Identities ("Algorithms" page, section "Common conventions", identity
 *    value): add 0; min +inf (floats) / INT32_MAX, INT64_MAX / UINT32_MAX,
 *    UINT64_MAX; max -inf (floats) / INT32_MIN, INT64_MIN / 0.  The product
 *    (row scans only) has identity 1 (metaltile-std src/mlx/scan.rs, op table
 *    of the "Multi-op scan variants" comment).
 *  - Combine order: the earlier operand is always on the left ("Tile
 *    operations and reductions", section "Why not just infer it from
 *    reduce?"); min is (a < b ? a : b) and max is (a > b ? a : b), so a tie
 *    yields the later element, as in the running-max/min kernels of
 *    metaltile-std src/mlx/scan.rs.  Integer add wraps modulo 2^w.  min/max
 *    and integer results are deterministic and exact; floating add may be
 *    regrouped, so its last bits can differ from a sequential fold ("Algorithms"
 *    page, "Common conventions", floating-point non-associativity), and for the
 *    device-wide scans and reduce-by-key also from one run to the next (the
 *    look-back combines whichever predecessor descriptors are ready).
 */
#ifndef STREAM_COMPACTION_AMD_SCAN_H
#define STREAM_COMPACTION_AMD_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SCAN_OK = 0,
    SCAN_EINVAL = 1,    /* bad size, null or misaligned pointer, bad flag value */
    SCAN_ENOTSUP = 2,   /* dtype/op combination this entry point does not implement */
    SCAN_EALIAS = 3,    /* two argument ranges overlap */
    SCAN_ESCRATCH = 4,  /* scratch smaller than *_scratch_bytes() */
    SCAN_EHIP = 5       /* the HIP runtime refused a launch; see scan_last_hip_error() */
} scan_status;

/* Element types.  Codes start at 1 so that a zeroed value is rejected. */
typedef enum {
    SCAN_F32 = 1, SCAN_F16 = 2, SCAN_BF16 = 3, SCAN_F64 = 4,
    SCAN_I32 = 5, SCAN_U32 = 6, SCAN_I64 = 7, SCAN_U64 = 8
} scan_dtype;

typedef enum { SCAN_ADD = 1, SCAN_MIN = 2, SCAN_MAX = 3, SCAN_MUL = 4 } scan_op;

/*
 * Row-wise scan along the last axis of a contiguous row-major [rows, n]
 * array (row r starts at element r*n).  Defined in the header comment of
 * metaltile-std src/mlx/scan.rs: inclusive out[r,i] = op(in[r,0..i]),
 * exclusive out[r,i] = op(in[r,0..i-1]) with out[r,0] = identity; its
 * "Multi-op scan variants" comment extends this to prod, min and max, and its
 * "Inclusive product scan" / "Exclusive product scan" sections define the
 * product forms (out[r,i] = in[r,0] * ... * in[r,i]; exclusive out[r,0] = 1).
 *
 *   in, out    device pointers, [rows, n] of `dtype`, same layout; must not
 *              overlap.
 *   dtype      SCAN_F32, SCAN_F16 or SCAN_BF16 (else SCAN_ENOTSUP).  16-bit
 *              inputs are widened exactly to float32, accumulated in float32
 *              (as the kernels of that page cast every load to f32) and each
 *              output is rounded once to `dtype`, nearest-even ("Tile
 *              operations and reductions", section "Storage and arithmetic
 *              precision").
 *   op         SCAN_ADD, SCAN_MIN, SCAN_MAX or SCAN_MUL (products are formed
 *              in float32 and rounded once per output, like sums).
 *   exclusive  0 = inclusive, 1 = exclusive (any other value: SCAN_EINVAL).
 *   rows, n    0 <= rows, n <= INT32_MAX.
 */
scan_status scan_rows(const void* in, void* out, int64_t rows, int64_t n,
                      scan_dtype dtype, scan_op op, int exclusive, void* stream);

/*
 * Device-wide EXCLUSIVE scan of a flat array ("Algorithms" page, section
 * qd.algorithms.exclusive_scan_{add,min,max}): out[i] = op(in[0..i-1]),
 * out[0] = identity(op, dtype).  One pass over the data (single-pass scan
 * with decoupled look-back between tiles, the alternative that page's
 * "Related" list names next to the grid-scope fence).
 *
 *   in, out    device pointers to n elements of `dtype`; must not overlap.
 *   dtype      SCAN_I32, SCAN_U32, SCAN_F32, SCAN_I64, SCAN_U64, SCAN_F64
 *              (the dtype set of that page's "Common conventions").
 *   op         SCAN_ADD, SCAN_MIN, SCAN_MAX (SCAN_MUL: SCAN_ENOTSUP).
 *   scratch    >= scan_device_scratch_bytes(n, dtype) bytes, 16-byte aligned,
 *              must not overlap in/out.
 */
size_t scan_device_scratch_bytes(int64_t n, scan_dtype dtype);
scan_status scan_device(const void* in, void* out, int64_t n, scan_dtype dtype, scan_op op,
                        void* scratch, size_t scratch_bytes, void* stream);

/*
 * Device-wide INCLUSIVE scan of a flat array: out[i] = op(in[0..i]).  The
 * inclusive prefix sum of the "Algorithms" page's PrefixSumExecutor section
 * (there in place, i32 and add only), here out of place with the dtypes, ops,
 * scratch and errors of scan_device (same scratch size helper); equivalently
 * the inclusive form of the row scan's definition applied to one row of n.
 */
scan_status scan_device_inclusive(const void* in, void* out, int64_t n, scan_dtype dtype,
                                  scan_op op, void* scratch, size_t scratch_bytes,
                                  void* stream);

/*
 * Device-wide reduction ("Algorithms" page, section
 * qd.algorithms.reduce_{add,min,max}): out[0] = op(in[0..n)), written on the
 * device.  n == 0 writes the identity (the seed, which "Tile operations and
 * reductions" gives as the final state of an empty fiber).  Integer and
 * min/max results equal the sequential left fold bit for bit (ties keep the
 * later element); floating add is a fixed regrouping, deterministic for a
 * given n and pointer alignment.
 *
 *   in         device pointer to n elements of `dtype`.
 *   out        device pointer to one element of `dtype`; must not overlap in or
 *              scratch.
 *   dtype      SCAN_I32, SCAN_U32, SCAN_F32, SCAN_I64, SCAN_U64, SCAN_F64.
 *   op         SCAN_ADD, SCAN_MIN, SCAN_MAX (SCAN_MUL: SCAN_ENOTSUP).
 *   scratch    >= reduce_device_scratch_bytes(n, dtype) bytes, 16-byte
 *              aligned, must not overlap in/out (may be NULL when that size is
 *              0, i.e. n == 0).  Holds per-workgroup partials; needs no
 *              initialization.
 */
size_t reduce_device_scratch_bytes(int64_t n, scan_dtype dtype);
scan_status reduce_device(const void* in, void* out, int64_t n, scan_dtype dtype, scan_op op,
                          void* scratch, size_t scratch_bytes, void* stream);

/*
 * Reduce-by-key ("Algorithms" page, section qd.algorithms.reduce_by_key_add):
 * every maximal run of consecutive equal keys becomes one pair (the run's
 * first key, the sum of its values), in input order; the number of runs r
 * is written to num_runs[0] on the device.  keys_out[0..r) and
 * values_out[0..r) receive the pairs; nothing past r is written.  Keys
 * compare with their type's == (an f32 NaN key is a run of its own; +0 and
 * -0 are equal).  Integer values wrap modulo 2^32; f32 sums are formed in
 * float32 in a fixed regrouping of each run (deterministic for a given n and
 * alignment), so their last bits may differ from a sequential sum.  One pass
 * over the input (a segmented scan with decoupled look-back; no atomics).
 *
 *   keys_in      device pointer, n elements of key_dtype.
 *   values_in    device pointer, n elements of value_dtype (may alias keys_in).
 *   keys_out     device pointer, capacity n elements of key_dtype.
 *   values_out   device pointer, capacity n elements of value_dtype.
 *   num_runs     device pointer to one int32 (0 for n == 0).
 *   key_dtype, value_dtype   each SCAN_I32, SCAN_U32 or SCAN_F32 (else
 *                SCAN_ENOTSUP).
 *   scratch      >= reduce_by_key_scratch_bytes(n) bytes, 16-byte aligned.
 * Outputs, num_runs and scratch must not overlap each other or the inputs.
 */
size_t reduce_by_key_scratch_bytes(int64_t n);
scan_status reduce_by_key(const void* keys_in, const void* values_in, void* keys_out,
                          void* values_out, int32_t* num_runs, int64_t n, scan_dtype key_dtype,
                          scan_dtype value_dtype, void* scratch, size_t scratch_bytes,
                          void* stream);

/*
 * Radix sort ("Algorithms" page, section qd.algorithms.sort): stable ascending
 * LSD radix sort, 8-bit digits, of n keys in place in `keys`, carrying
 * `values` along when given.  The order is that of each key's sortable image
 * (unsigned keys as they are; signed keys with the sign bit flipped; floats
 * with the sign bit flipped when clear and every bit flipped when set, so
 * -0 sorts before +0), restricted to its low `end_bit` bits; every NaN key
 * sorts after all other keys, in input order (the page's "NaNs land at the
 * end").  Equal images keep their input order.  Keys and values move as raw
 * bits.  Each pass is the page's tile histogram, scan of the digit-major
 * histograms (this library's device-wide scan) and scatter.
 *
 *   keys, tmp_keys       device pointers, n keys of key_dtype each, distinct;
 *                        tmp_keys holds garbage on return.
 *   values, tmp_values   both NULL (keys-only sort) or both device pointers to
 *                        n values of value_dtype each, distinct.
 *   key_dtype            SCAN_U32, SCAN_I32, SCAN_F32, SCAN_U64, SCAN_I64 or
 *                        SCAN_F64 (else SCAN_ENOTSUP).
 *   value_dtype          any of the same six (ignored for a keys-only sort).
 *   end_bit              a multiple of 8 in [8, key bits] (else SCAN_EINVAL);
 *                        end_bit / 8 digit passes.
 *   n                    0 <= n <= INT32_MAX.
 *   scratch              >= radix_sort_scratch_bytes(n, key_dtype) bytes,
 *                        16-byte aligned; needs no initialization.
 * No two of keys, tmp_keys, values, tmp_values and scratch may overlap.
 */
size_t radix_sort_scratch_bytes(int64_t n, scan_dtype key_dtype);
scan_status radix_sort(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                       scan_dtype key_dtype, scan_dtype value_dtype, int end_bit, void* scratch,
                       size_t scratch_bytes, void* stream);

/*
 * Stream compaction ("Algorithms" page, section qd.algorithms.select): every
 * in[i] whose flags[i] is nonzero is copied, in input order, into the dense
 * prefix out[0..k), and k is written to num_out[0] on the device.  The page
 * requires flags to be exactly 0/1; here any nonzero byte selects.  out must
 * hold n elements; out[k..n) is left untouched.  Elements are copied as raw
 * bytes, so any element type of 1, 2, 4, 8 or 16 bytes works (NaN payloads
 * survive; the page allows any scalar or struct element type).
 *
 *   in         device pointer, n elements of elem_bytes bytes, aligned to
 *              elem_bytes (as is out).
 *   flags      device pointer, n bytes (uint8).
 *   out        device pointer, capacity n elements; must not overlap in,
 *              flags, num_out or scratch.
 *   num_out    device pointer to one int32.
 *   elem_bytes 1, 2, 4, 8 or 16 (else SCAN_ENOTSUP).
 *   scratch    >= select_compact_scratch_bytes(n) bytes, 16-byte aligned.
 */
size_t select_compact_scratch_bytes(int64_t n);
scan_status select_compact(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                           int64_t n, size_t elem_bytes, void* scratch, size_t scratch_bytes,
                           void* stream);

/*
 * Device-count variants, for graph capture ("Algorithms" page, sections "Key
 * sizing parameters" and "Capacity (log256_max_n)": the live count is read on
 * the device and a fixed capacity sizes everything, so one captured graph
 * replays across every count up to that capacity).  Each *_devn entry point
 * does exactly what its namesake does, on n = n_live[0] elements, where that
 * count is read by the kernels when they run and clamped to [0, capacity].
 *   n_live     device pointer to one int32, 4-byte aligned; it must not
 *              overlap anything the call writes.  NULL: SCAN_EINVAL.
 *   capacity   takes the place of n in host-side validation, in the
 *              *_scratch_bytes sizing and in the launch sizes (the grids
 *              cover the capacity; work past the live count exits at once).
 * Outputs past the live count are left untouched, as past n.
 * radix_sort_devn needs an even number of digit passes (end_bit / 8 even,
 * as the page requires of its sort) so that the result lands in keys
 * without a copy sized on the host; otherwise SCAN_EINVAL.
 */
scan_status scan_device_devn(const void* in, void* out, const int32_t* n_live, int64_t capacity,
                             scan_dtype dtype, scan_op op, void* scratch, size_t scratch_bytes,
                             void* stream);
scan_status scan_device_inclusive_devn(const void* in, void* out, const int32_t* n_live,
                                       int64_t capacity, scan_dtype dtype, scan_op op,
                                       void* scratch, size_t scratch_bytes, void* stream);
scan_status reduce_device_devn(const void* in, void* out, const int32_t* n_live, int64_t capacity,
                               scan_dtype dtype, scan_op op, void* scratch, size_t scratch_bytes,
                               void* stream);
scan_status reduce_by_key_devn(const void* keys_in, const void* values_in, void* keys_out,
                               void* values_out, int32_t* num_runs, const int32_t* n_live,
                               int64_t capacity, scan_dtype key_dtype, scan_dtype value_dtype,
                               void* scratch, size_t scratch_bytes, void* stream);
scan_status radix_sort_devn(void* keys, void* tmp_keys, void* values, void* tmp_values,
                            const int32_t* n_live, int64_t capacity, scan_dtype key_dtype,
                            scan_dtype value_dtype, int end_bit, void* scratch,
                            size_t scratch_bytes, void* stream);
scan_status select_compact_devn(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                                const int32_t* n_live, int64_t capacity, size_t elem_bytes,
                                void* scratch, size_t scratch_bytes, void* stream);

/* Static string naming a status code (never NULL). */
const char* scan_status_str(scan_status s);

/* hipError_t value behind the calling thread's last SCAN_EHIP (0 if none). */
int scan_last_hip_error(void);

/*
 * scan_device without a scratch argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operation, arguments, results and
 * kernels as scan_device (exclusive scan, out[0] = identity).  It allocates
 * nothing: the tile descriptors live in a static device array of
 * SCAN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends; the array of the calling thread's current
 * device is used, so `stream` must belong to that device.  Each call clears
 * the descriptors it uses (a fill kernel on `stream`), so nothing carries
 * over from one call to the next, but every such call on one GPU shares the
 * array: two calls in flight at the same time on one GPU (other streams,
 * other threads) race and give wrong results.
 *
 *   n          0 <= n and scan_device_scratch_bytes(n, dtype) <=
 *              SCAN_NOALLOC_SCRATCH_BYTES (n <= 469,754,880; a larger n
 *              returns SCAN_ESCRATCH before anything is launched).
 *   others     as for scan_device.
 */
#define SCAN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
scan_status scan_device_noalloc(const void* in, void* out, int64_t n, scan_dtype dtype,
                                scan_op op, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_COMPACTION_AMD_SCAN_H */

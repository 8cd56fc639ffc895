/*
 * Plain sequential CPU oracle for prefix scan and stream compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source, header, table or constant with the
 * HIP library and has its own dtype/op codes; its entry points are the
 * non-static functions below (loaded through oracle/__init__.py).
 *
 * What it computes (all definitions written out, no blocking, no reordering):
 *
 *  - The left-prefix recurrence of "Tile operations and reductions"
 *    (LuisaCompute), section "Why not just infer it from reduce?":
 *    for an ordered fiber x[0..n) with seed z and combine op,
 *        p[0] = z,  p[i+1] = op(p[i], x[i]),
 *        inclusive[i] = p[i+1],  exclusive[i] = p[i].
 *    The seed is the identity of (op, dtype) from the "Algorithms" page
 *    (Quadrants user guide), section "Common conventions", paragraph on the
 *    identity value: add 0; min +inf / INT_MAX / UINT_MAX; max -inf /
 *    INT_MIN / 0.
 *  - Row-wise scans along the last axis of a contiguous [rows, n] array as
 *    defined in the header comment of metaltile-std src/mlx/scan.rs
 *    (inclusive out[i] = sum_{j<=i}, exclusive out[i] = sum_{j<i}, out[0]=0),
 *    one independent fold per row.
 *  - Stream compaction as defined on the "Algorithms" page, section
 *    qd.algorithms.select: every element whose flag is set is copied, in
 *    input order, into a dense prefix of out, and the count is returned.
 *
 * Arithmetic choices (each a reading of the pages, restated in the tests):
 *  - integer add is done in the unsigned type of the same width, so it wraps
 *    modulo 2^w (two's complement), with no signed-overflow UB;
 *  - floating add is accumulated in double, sequentially, and rounded once
 *    per output element: to float by a C cast (round to nearest even under
 *    the default FP environment), then, for bf16/f16 outputs, from that float
 *    to 16 bits by round-to-nearest-even written out below from the bit
 *    patterns ("Tile operations and reductions", section "Storage and
 *    arithmetic precision": nearest-even, signed zeros and subnormals kept,
 *    overflow to infinity, NaN quieted);
 *  - min is (a < b) ? a : b and max is (a > b) ? a : b with a the earlier
 *    operand (so a tie returns the later operand), compared in the element's
 *    own type; bf16/f16 compare their exact float32 widening;
 *  - select treats any nonzero flag byte as selected and copies bytes, so
 *    NaN payloads survive.
 *
 * Extra outputs for tolerance checks: ref[i] is the double accumulator of the
 * fold that produced out[i] (floating add only) and absref[i] is
 * sum_{j<=i} |x_j| in double.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* dtype codes of this oracle */
enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_F64 = 3,
       O_I32 = 4, O_U32 = 5, O_I64 = 6, O_U64 = 7 };
/* op codes of this oracle */
enum { O_ADD = 0, O_MIN = 1, O_MAX = 2 };

/* ---- 16-bit float conversions, from the bit patterns ---------------------- */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the top half of a float32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* float32 -> bf16, round to nearest, ties to even. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* NaN: keep sign, set quiet bit */
    uint32_t lsb = (u >> 16) & 1u;                        /* ties go to the even result */
    uint32_t r = u + 0x7fffu + lsb;                       /* overflow carries into inf */
    return (uint16_t)(r >> 16);
}

/* IEEE binary16 -> float32 (exact). */
float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int32_t e = (h >> 10) & 0x1f;
    uint32_t m = h & 0x3ffu;
    if (e == 0x1f)                                        /* inf / NaN */
        return bits_f32(sign | 0x7f800000u | (m << 13));
    if (e == 0) {
        if (m == 0) return bits_f32(sign);                /* signed zero */
        /* subnormal: value = m * 2^-24, exact in float */
        float v = (float)m * 0x1p-24f;
        return sign ? -v : v;
    }
    return bits_f32(sign | (uint32_t)(e - 15 + 127) << 23 | (m << 13));
}

/* float32 -> IEEE binary16, round to nearest, ties to even.  Worked in double,
 * where every step below is exact: the float is divided by the binary16 unit in
 * the last place of its binade (a power of two), rounded to an integer with
 * nearbyint (nearest-even in the default rounding mode), and re-encoded. */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u | ((u >> 13) & 0x3ffu));   /* quiet NaN */
    if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;                            /* signed zero */
    int e;
    frexp(a, &e);                                         /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                                        /* floor(log2 a) */
    if (E < -14) E = -14;                                 /* subnormal binade */
    double ulp = ldexp(1.0, E - 10);
    double v = nearbyint(a / ulp) * ulp;                  /* rounded magnitude */
    if (v >= 65536.0) return (uint16_t)(sign | 0x7c00u);  /* overflow to inf */
    if (v < ldexp(1.0, -14))                              /* subnormal (or zero) */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    frexp(v, &e);
    E = e - 1;
    uint32_t mant = (uint32_t)(v / ldexp(1.0, E - 10)) - 1024u;
    return (uint16_t)(sign | (uint32_t)(E + 15) << 10 | mant);
}

/* ---- element access -------------------------------------------------------- */

static int elem_size(int dt) {
    switch (dt) {
    case O_F32: case O_I32: case O_U32: return 4;
    case O_F16: case O_BF16: return 2;
    case O_F64: case O_I64: case O_U64: return 8;
    }
    return 0;
}

static int is_float(int dt) { return dt == O_F32 || dt == O_F16 || dt == O_BF16 || dt == O_F64; }

static double load_fp(const void* p, int64_t i, int dt) {
    switch (dt) {
    case O_F32: return (double)((const float*)p)[i];
    case O_F16: return (double)oracle_f16_to_f32(((const uint16_t*)p)[i]);
    case O_BF16: return (double)oracle_bf16_to_f32(((const uint16_t*)p)[i]);
    default: return ((const double*)p)[i];
    }
}

/* store a floating value already in the output's own range of values */
static void store_fp(void* p, int64_t i, int dt, double v) {
    switch (dt) {
    case O_F32: ((float*)p)[i] = (float)v; break;
    case O_F16: ((uint16_t*)p)[i] = oracle_f32_to_f16((float)v); break;
    case O_BF16: ((uint16_t*)p)[i] = oracle_f32_to_bf16((float)v); break;
    default: ((double*)p)[i] = v; break;
    }
}

/* ---- the fold ------------------------------------------------------------- */

/* Floating fold over one fiber.  add accumulates in double; min/max keep the
 * earlier-operand-left compare+select on the element values (float for the
 * 32- and 16-bit formats, double for f64). */
static void fold_fp(const void* in, void* out, int64_t base, int64_t n, int dt, int op,
                    int exclusive, double* ref, double* absref) {
    double absacc = 0.0;
    if (op == O_ADD) {
        double acc = 0.0;                                  /* identity of add */
        for (int64_t k = 0; k < n; ++k) {
            double x = load_fp(in, base + k, dt);
            absacc += fabs(x);
            if (exclusive) { store_fp(out, base + k, dt, acc); if (ref) ref[base + k] = acc; }
            acc = acc + x;
            if (!exclusive) { store_fp(out, base + k, dt, acc); if (ref) ref[base + k] = acc; }
            if (absref) absref[base + k] = absacc;
        }
        return;
    }
    if (dt == O_F64) {
        double acc = (op == O_MIN) ? INFINITY : -INFINITY;
        for (int64_t k = 0; k < n; ++k) {
            double x = ((const double*)in)[base + k];
            absacc += fabs(x);
            if (exclusive) ((double*)out)[base + k] = acc;
            acc = (op == O_MIN) ? ((acc < x) ? acc : x) : ((acc > x) ? acc : x);
            if (!exclusive) ((double*)out)[base + k] = acc;
            if (ref) ref[base + k] = exclusive ? ((double*)out)[base + k] : acc;
            if (absref) absref[base + k] = absacc;
        }
        return;
    }
    float acc = (op == O_MIN) ? INFINITY : -INFINITY;
    for (int64_t k = 0; k < n; ++k) {
        float x = (float)load_fp(in, base + k, dt);        /* exact widening */
        absacc += fabs((double)x);
        if (exclusive) store_fp(out, base + k, dt, (double)acc);
        acc = (op == O_MIN) ? ((acc < x) ? acc : x) : ((acc > x) ? acc : x);
        if (!exclusive) store_fp(out, base + k, dt, (double)acc);
        if (ref) ref[base + k] = (double)(exclusive ? (float)load_fp(out, base + k, dt) : acc);
        if (absref) absref[base + k] = absacc;
    }
}

/* Integer fold over one fiber, in the unsigned type of the element's width. */
static void fold_int(const void* in, void* out, int64_t base, int64_t n, int dt, int op,
                     int exclusive) {
    if (dt == O_I32 || dt == O_U32) {
        const uint32_t* x = (const uint32_t*)in + base;
        uint32_t* y = (uint32_t*)out + base;
        uint32_t acc;
        if (op == O_ADD) acc = 0u;
        else if (dt == O_I32) acc = (op == O_MIN) ? (uint32_t)INT32_MAX : (uint32_t)INT32_MIN;
        else acc = (op == O_MIN) ? UINT32_MAX : 0u;
        for (int64_t k = 0; k < n; ++k) {
            uint32_t v = x[k];
            if (exclusive) y[k] = acc;
            if (op == O_ADD) acc = acc + v;               /* wraps mod 2^32 */
            else if (dt == O_I32) {
                int32_t a = (int32_t)acc, b = (int32_t)v;
                acc = (uint32_t)((op == O_MIN) ? ((a < b) ? a : b) : ((a > b) ? a : b));
            } else {
                acc = (op == O_MIN) ? ((acc < v) ? acc : v) : ((acc > v) ? acc : v);
            }
            if (!exclusive) y[k] = acc;
        }
    } else {
        const uint64_t* x = (const uint64_t*)in + base;
        uint64_t* y = (uint64_t*)out + base;
        uint64_t acc;
        if (op == O_ADD) acc = 0u;
        else if (dt == O_I64) acc = (op == O_MIN) ? (uint64_t)INT64_MAX : (uint64_t)INT64_MIN;
        else acc = (op == O_MIN) ? UINT64_MAX : 0u;
        for (int64_t k = 0; k < n; ++k) {
            uint64_t v = x[k];
            if (exclusive) y[k] = acc;
            if (op == O_ADD) acc = acc + v;               /* wraps mod 2^64 */
            else if (dt == O_I64) {
                int64_t a = (int64_t)acc, b = (int64_t)v;
                acc = (uint64_t)((op == O_MIN) ? ((a < b) ? a : b) : ((a > b) ? a : b));
            } else {
                acc = (op == O_MIN) ? ((acc < v) ? acc : v) : ((acc > v) ? acc : v);
            }
            if (!exclusive) y[k] = acc;
        }
    }
}

/* Scan every row of a contiguous [rows, n] array along its last axis.
 * Returns 0 on success, -1 for an unknown dtype/op. ref/absref may be NULL. */
int oracle_scan(const void* in, void* out, int64_t rows, int64_t n, int dtype, int op,
                int exclusive, double* ref, double* absref) {
    if (elem_size(dtype) == 0 || op < O_ADD || op > O_MAX || rows < 0 || n < 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        if (is_float(dtype)) fold_fp(in, out, r * n, n, dtype, op, exclusive, ref, absref);
        else fold_int(in, out, r * n, n, dtype, op, exclusive);
    }
    return 0;
}

/* Stream compaction: copy element i (elem_bytes bytes) to out[k++] whenever
 * flags[i] != 0.  Elements of out past the count are not written.  Returns k. */
int64_t oracle_select(const void* in, const uint8_t* flags, void* out, int64_t n,
                      int64_t elem_bytes) {
    int64_t k = 0;
    const unsigned char* src = (const unsigned char*)in;
    unsigned char* dst = (unsigned char*)out;
    for (int64_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            memcpy(dst + k * elem_bytes, src + i * elem_bytes, (size_t)elem_bytes);
            ++k;
        }
    }
    return k;
}

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
 *    the running states of a sequence x[0..n) folded from seed z with op,
 *        p[0] = z,  p[i+1] = op(p[i], x[i]),
 *        inclusive[i] = p[i+1],  exclusive[i] = p[i].
 *    The seed is the identity of (op, dtype) from the "Algorithms" page
 *    (Quadrants user guide), section "Common conventions", paragraph on the
 *    identity value: add 0; min +inf / INT_MAX / UINT_MAX; max -inf /
 *    INT_MIN / 0.  The product (mul) has identity 1, per the op table of
 *    metaltile-std src/mlx/scan.rs, comment "Multi-op scan variants", and
 *    the definitions under "Inclusive product scan" / "Exclusive product
 *    scan" there (out[i] = v[0]*...*v[i]; exclusive out[0] = 1).
 *  - Row-wise scans along the last axis of a contiguous [rows, n] array as
 *    defined in the header comment of metaltile-std src/mlx/scan.rs
 *    (inclusive out[i] = sum_{j<=i}, exclusive out[i] = sum_{j<i}, out[0]=0),
 *    one independent fold per row.
 *  - Stream compaction as defined on the "Algorithms" page, section
 *    qd.algorithms.select: every element whose flag is set is copied, in
 *    input order, into a dense prefix of out, and the count is returned.
 *  - Reduce-by-key as defined on the "Algorithms" page, section
 *    qd.algorithms.reduce_by_key_add: every maximal run of consecutive equal
 *    keys becomes one output pair (key, sum of the run's values), in input
 *    order, and the number of runs is returned.  Keys compare with the
 *    key type's own ==, so a NaN key never equals anything (each NaN is a
 *    run of its own) and +0 equals -0; the run's key is its first element's
 *    key (the page's scatter leaves that choice to whichever write lands
 *    last; the first is the deterministic reading).  Sums start from 0 and
 *    fold the run in order: integer values wrap, f32 values accumulate in
 *    double and are rounded once.
 *  - Reduction as defined on the "Algorithms" page, section
 *    qd.algorithms.reduce_{add,min,max}: out[0] = op over in[0..n), here
 *    the final state p[n] of the recurrence above (p[0], the identity, for
 *    an empty input: "Tile operations and reductions" names the seed as the
 *    final state of an empty scan).
 *
 * Arithmetic choices (each a reading of the pages, restated in the tests):
 *  - integer add is done in the unsigned type of the same width, so it wraps
 *    modulo 2^w (two's complement), with no signed-overflow UB;
 *  - floating add and mul are accumulated in double, sequentially, and rounded once
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
 * fold that produced out[i] (floating add and mul) and absref[i] is
 * sum_{j<=i} |x_j| in double.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* dtype codes of this oracle */
enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_F64 = 3,
       O_I32 = 4, O_U32 = 5, O_I64 = 6, O_U64 = 7 };
/* op codes of this oracle */
enum { O_ADD = 0, O_MIN = 1, O_MAX = 2, O_MUL = 3 };

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

/* ---- the combine, per value class ------------------------------------------ */

/* a is the earlier operand.  Floating add and mul accumulate in double (the
 * caller holds the double accumulator); min/max compare+select in the
 * element's own type. */
static double comb_fp64(int op, double a, double b) {
    switch (op) {
    case O_ADD: return a + b;
    case O_MUL: return a * b;
    case O_MIN: return (a < b) ? a : b;
    default: return (a > b) ? a : b;
    }
}

static float comb_fp32_minmax(int op, float a, float b) {
    return (op == O_MIN) ? ((a < b) ? a : b) : ((a > b) ? a : b);
}

static uint32_t comb_u32(int dt, int op, uint32_t a, uint32_t b) {
    if (op == O_ADD) return a + b;                        /* wraps mod 2^32 */
    if (op == O_MUL) return a * b;                        /* wraps mod 2^32 */
    if (dt == O_I32) {
        int32_t x = (int32_t)a, y = (int32_t)b;
        return (uint32_t)((op == O_MIN) ? ((x < y) ? x : y) : ((x > y) ? x : y));
    }
    return (op == O_MIN) ? ((a < b) ? a : b) : ((a > b) ? a : b);
}

static uint64_t comb_u64(int dt, int op, uint64_t a, uint64_t b) {
    if (op == O_ADD) return a + b;                        /* wraps mod 2^64 */
    if (op == O_MUL) return a * b;                        /* wraps mod 2^64 */
    if (dt == O_I64) {
        int64_t x = (int64_t)a, y = (int64_t)b;
        return (uint64_t)((op == O_MIN) ? ((x < y) ? x : y) : ((x > y) ? x : y));
    }
    return (op == O_MIN) ? ((a < b) ? a : b) : ((a > b) ? a : b);
}

/* identities, as bit patterns of the element's width */
static double ident_fp(int op) {
    switch (op) {
    case O_ADD: return 0.0;
    case O_MUL: return 1.0;
    case O_MIN: return INFINITY;
    default: return -INFINITY;
    }
}

static uint32_t ident_u32(int dt, int op) {
    if (op == O_ADD) return 0u;
    if (op == O_MUL) return 1u;
    if (dt == O_I32) return (op == O_MIN) ? (uint32_t)INT32_MAX : (uint32_t)INT32_MIN;
    return (op == O_MIN) ? UINT32_MAX : 0u;
}

static uint64_t ident_u64(int dt, int op) {
    if (op == O_ADD) return 0u;
    if (op == O_MUL) return 1u;
    if (dt == O_I64) return (op == O_MIN) ? (uint64_t)INT64_MAX : (uint64_t)INT64_MIN;
    return (op == O_MIN) ? UINT64_MAX : 0u;
}

/* ---- the fold ------------------------------------------------------------- */

/* Floating fold over one fiber.  add and mul accumulate in double; min/max
 * keep the earlier-operand-left compare+select on the element values (float
 * for the 32- and 16-bit formats, double for f64). */
static void fold_fp(const void* in, void* out, int64_t base, int64_t n, int dt, int op,
                    int exclusive, double* ref, double* absref) {
    double absacc = 0.0;
    if (op == O_ADD || op == O_MUL || dt == O_F64) {
        double acc = ident_fp(op);
        for (int64_t k = 0; k < n; ++k) {
            double x = load_fp(in, base + k, dt);
            absacc += fabs(x);
            if (exclusive) { store_fp(out, base + k, dt, acc); if (ref) ref[base + k] = acc; }
            acc = comb_fp64(op, acc, x);
            if (!exclusive) { store_fp(out, base + k, dt, acc); if (ref) ref[base + k] = acc; }
            if (absref) absref[base + k] = absacc;
        }
        return;
    }
    float acc = (float)ident_fp(op);
    for (int64_t k = 0; k < n; ++k) {
        float x = (float)load_fp(in, base + k, dt);        /* exact widening */
        absacc += fabs((double)x);
        if (exclusive) store_fp(out, base + k, dt, (double)acc);
        acc = comb_fp32_minmax(op, acc, x);
        if (!exclusive) store_fp(out, base + k, dt, (double)acc);
        if (ref) ref[base + k] = (double)(exclusive ? (float)load_fp(out, base + k, dt) : acc);
        if (absref) absref[base + k] = absacc;
    }
}

/* Integer fold over one fiber, in the unsigned type of the element's width. */
static void fold_int(const void* in, void* out, int64_t base, int64_t n, int dt, int op,
                     int exclusive) {
    if (elem_size(dt) == 4) {
        const uint32_t* x = (const uint32_t*)in + base;
        uint32_t* y = (uint32_t*)out + base;
        uint32_t acc = ident_u32(dt, op);
        for (int64_t k = 0; k < n; ++k) {
            if (exclusive) y[k] = acc;
            acc = comb_u32(dt, op, acc, x[k]);
            if (!exclusive) y[k] = acc;
        }
    } else {
        const uint64_t* x = (const uint64_t*)in + base;
        uint64_t* y = (uint64_t*)out + base;
        uint64_t acc = ident_u64(dt, op);
        for (int64_t k = 0; k < n; ++k) {
            if (exclusive) y[k] = acc;
            acc = comb_u64(dt, op, acc, x[k]);
            if (!exclusive) y[k] = acc;
        }
    }
}

/* Scan every row of a contiguous [rows, n] array along its last axis.
 * Returns 0 on success, -1 for an unknown dtype/op. ref/absref may be NULL. */
int oracle_scan(const void* in, void* out, int64_t rows, int64_t n, int dtype, int op,
                int exclusive, double* ref, double* absref) {
    if (elem_size(dtype) == 0 || op < O_ADD || op > O_MUL || rows < 0 || n < 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        if (is_float(dtype)) fold_fp(in, out, r * n, n, dtype, op, exclusive, ref, absref);
        else fold_int(in, out, r * n, n, dtype, op, exclusive);
    }
    return 0;
}

/* Reduction of a flat array: out[0] = op-fold of in[0..n) from the identity,
 * i.e. the final state of the same recurrence (an empty input leaves the
 * identity).  ref/absref (may be NULL) receive the double accumulator
 * (floating add/mul; the value itself otherwise) and sum |x| in double.
 * Returns 0 on success, -1 for an unknown dtype/op. */
int oracle_reduce(const void* in, void* out, int64_t n, int dtype, int op, double* ref,
                  double* absref) {
    if (elem_size(dtype) == 0 || op < O_ADD || op > O_MUL || n < 0) return -1;
    double absacc = 0.0;
    if (is_float(dtype) && (op == O_ADD || op == O_MUL || dtype == O_F64)) {
        double acc = ident_fp(op);
        for (int64_t k = 0; k < n; ++k) {
            double x = load_fp(in, k, dtype);
            absacc += fabs(x);
            acc = comb_fp64(op, acc, x);
        }
        store_fp(out, 0, dtype, acc);
        if (ref) *ref = acc;
    } else if (is_float(dtype)) {
        float acc = (float)ident_fp(op);
        for (int64_t k = 0; k < n; ++k) {
            float x = (float)load_fp(in, k, dtype);
            absacc += fabs((double)x);
            acc = comb_fp32_minmax(op, acc, x);
        }
        store_fp(out, 0, dtype, (double)acc);
        if (ref) *ref = (double)acc;
    } else if (elem_size(dtype) == 4) {
        const uint32_t* x = (const uint32_t*)in;
        uint32_t acc = ident_u32(dtype, op);
        for (int64_t k = 0; k < n; ++k) acc = comb_u32(dtype, op, acc, x[k]);
        *(uint32_t*)out = acc;
        if (ref) *ref = (dtype == O_I32) ? (double)(int32_t)acc : (double)acc;
    } else {
        const uint64_t* x = (const uint64_t*)in;
        uint64_t acc = ident_u64(dtype, op);
        for (int64_t k = 0; k < n; ++k) acc = comb_u64(dtype, op, acc, x[k]);
        *(uint64_t*)out = acc;
        if (ref) *ref = (dtype == O_I64) ? (double)(int64_t)acc : (double)acc;
    }
    if (absref) *absref = absacc;
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

/* Reduce-by-key over n (key, value) pairs; keys and values are 32-bit (key
 * dtype and value dtype each O_I32, O_U32 or O_F32).  Writes the runs'
 * first keys to keys_out[0..r) and their value sums to values_out[0..r);
 * nothing past r is written.  ref/absref (may be NULL) receive, per run, the
 * double accumulator and the sum of |value| over the run.  Returns r, or -1
 * for unsupported dtypes. */
int64_t oracle_reduce_by_key(const void* keys, const void* values, int64_t n, int key_dtype,
                             int value_dtype, void* keys_out, void* values_out, double* ref,
                             double* absref) {
    if (elem_size(key_dtype) != 4 || elem_size(value_dtype) != 4 || n < 0) return -1;
    const uint32_t* kb = (const uint32_t*)keys;
    const uint32_t* vb = (const uint32_t*)values;
    uint32_t* ko = (uint32_t*)keys_out;
    uint32_t* vo = (uint32_t*)values_out;
    int64_t r = -1;                    /* index of the current run */
    double dacc = 0.0, aacc = 0.0;     /* f32 values */
    uint32_t iacc = 0u;                /* integer values, wrapping */
    for (int64_t i = 0; i < n; ++i) {
        int head;
        if (i == 0) {
            head = 1;
        } else if (key_dtype == O_F32) {
            float a, b;
            memcpy(&a, &kb[i - 1], 4);
            memcpy(&b, &kb[i], 4);
            head = !(a == b);
        } else {
            head = kb[i] != kb[i - 1];
        }
        if (head) {
            if (r >= 0) {              /* close the previous run */
                if (value_dtype == O_F32) {
                    float f = (float)dacc;
                    memcpy(&vo[r], &f, 4);
                    if (ref) ref[r] = dacc;
                    if (absref) absref[r] = aacc;
                } else {
                    vo[r] = iacc;
                }
            }
            ++r;
            ko[r] = kb[i];
            dacc = 0.0; aacc = 0.0; iacc = 0u;
        }
        if (value_dtype == O_F32) {
            float f;
            memcpy(&f, &vb[i], 4);
            dacc += (double)f;
            aacc += fabs((double)f);
        } else {
            iacc += vb[i];
        }
    }
    if (r >= 0) {
        if (value_dtype == O_F32) {
            float f = (float)dacc;
            memcpy(&vo[r], &f, 4);
            if (ref) ref[r] = dacc;
            if (absref) absref[r] = aacc;
        } else {
            vo[r] = iacc;
        }
    }
    return r + 1;
}

"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against one of: a worked example printed on the
pages (fixtures under tests/golden/, each carrying its citation), a closed
form, an invariant between separately computed results, an independent
library routine (numpy accumulate, numpy/torch float conversions, boolean
masking), or brute force on tiny inputs.  A mistake in the oracle's fold (a
dropped term, an off-by-one shift, a wrong identity, a swapped operand in
min/max, a wrong rounding, a missing wrap) fails at least one of them.
"""
import functools
import itertools
import math
import operator

import numpy as np
import pytest
import torch

import oracle
import workloads

INT_DT = {"i32": np.int32, "u32": np.uint32, "i64": np.int64, "u64": np.uint64}
ALL_DT = ("f32", "f16", "bf16", "f64", "i32", "u32", "i64", "u64")


def bits_to_f32(h, dtype):
    """16-bit patterns -> float32 through torch/numpy (independent of the oracle)."""
    h = np.asarray(h, dtype=np.uint16)
    if dtype == "bf16":
        return torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    return h.view(np.float16).astype(np.float32)


def f32_to_bits(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return workloads.to_bf16_bits(x)
    return workloads.to_f16_bits(x)


def as_float(vals, dtype):
    """Oracle output -> float64 values, decoding 16-bit formats independently."""
    if dtype in ("bf16", "f16"):
        return bits_to_f32(vals, dtype).astype(np.float64)
    return np.asarray(vals, dtype=np.float64)


def random_input(dtype, n, seed):
    rng = np.random.default_rng(seed)
    if dtype in ("f32", "f64"):
        return rng.uniform(-4, 4, size=n).astype(oracle.STORAGE[dtype])
    if dtype in ("bf16", "f16"):
        return f32_to_bits(rng.standard_normal(n).astype(np.float32), dtype)
    info = np.iinfo(INT_DT[dtype])
    return rng.integers(info.min, info.max, size=n, dtype=INT_DT[dtype], endpoint=True)


# ---- worked examples printed on the pages ----------------------------------------

def test_page_exclusive_scan_example(golden):
    g = golden("exclusive_scan_example.json")
    x = np.array(g["input"], dtype=np.int32)
    out = oracle.scan(x, "i32", "add", exclusive=True)
    assert out.tolist() == g["exclusive"]


def test_page_reduce_example(golden):
    g = golden("reduce_example.json")
    x = np.array(g["input"], dtype=np.int32)
    for op in ("add", "min", "max"):
        inc = oracle.scan(x, "i32", op, exclusive=False)
        assert int(inc[-1]) == g[op], op           # the inclusive scan ends in the reduction
        assert int(oracle.reduce(x, "i32", op)[0]) == g[op], op


def test_page_select_example(golden):
    g = golden("select_example.json")
    out, k = oracle.select(np.array(g["input"], np.int32), np.array(g["flags"], np.uint8))
    assert k == g["count"]
    assert out[:k].tolist() == g["selected"]


def test_page_order_example(golden):
    g = golden("order_example.json")
    for case in g["cases"]:
        inc = oracle.scan(np.array(case["input"], np.int32), "i32", "add")
        assert inc.tolist() == case["inclusive"]


def test_identities(golden):
    g = golden("identities.json")
    for op in ("add", "min", "max", "mul"):
        for dt in ALL_DT:
            if dt not in g[op]:
                continue
            x = random_input(dt, 3, 11)
            excl = oracle.scan(x, dt, op, exclusive=True)
            want = g[op][dt]
            if dt in oracle.FLOATS:
                got = as_float(excl[:1], dt)[0]
                want = float(want)
                assert got == want and math.copysign(1, got) == math.copysign(1, want), (op, dt)
            else:
                assert int(excl[0]) == int(want), (op, dt)
            # the identities agree with numpy's own limits, an independent source
            if dt in INT_DT and op != "add":
                info = np.iinfo(INT_DT[dt])
                assert int(want) == (info.max if op == "min" else info.min)


def test_tie_break_signed_zero(golden):
    g = golden("tie_break.json")
    for case in g["cases"]:
        x = np.array([float(v) for v in case["input"]], dtype=np.float32)
        inc = oracle.scan(x, "f32", case["op"])
        want = np.array([float(v) for v in case["inclusive"]], dtype=np.float32)
        assert inc.view(np.uint32).tolist() == want.view(np.uint32).tolist(), case


# ---- closed forms -------------------------------------------------------------------

@pytest.mark.parametrize("dt", ALL_DT)
def test_all_ones(dt):
    n = 5000
    if dt in oracle.FLOATS:
        x = np.ones(n, np.float32)
        x = f32_to_bits(x, dt) if dt in ("bf16", "f16") else x.astype(oracle.STORAGE[dt])
    else:
        x = np.ones(n, INT_DT[dt])
    inc = oracle.scan(x, dt, "add")
    exc = oracle.scan(x, dt, "add", exclusive=True)
    i = np.arange(n)
    if dt in ("bf16", "f16"):
        # exact sums i+1 / i, rounded once to the 16-bit format by torch/numpy
        assert inc.tolist() == f32_to_bits((i + 1).astype(np.float32), dt).tolist()
        assert exc.tolist() == f32_to_bits(i.astype(np.float32), dt).tolist()
    else:
        assert np.array_equal(inc.astype(np.float64), i + 1)
        assert np.array_equal(exc.astype(np.float64), i)


def test_bf16_ones_rounding_ties():
    # 257 and 259 are halfway between bf16 neighbours: ties go to even
    x = f32_to_bits(np.ones(300, np.float32), "bf16")
    inc = bits_to_f32(oracle.scan(x, "bf16", "add"), "bf16")
    assert inc[256] == 256.0 and inc[258] == 260.0 and inc[255] == 256.0 and inc[259] == 260.0


def test_arange_i32_wraps():
    n = 100_000                                    # n(n-1)/2 ~ 5e9 > 2^32: wraps
    x = np.arange(n, dtype=np.int32)
    inc = oracle.scan(x, "i32", "add")
    exc = oracle.scan(x, "i32", "add", exclusive=True)
    for i in (0, 1, 2, 65535, 65536, 92681, 92682, n - 1):
        want_inc = (i * (i + 1) // 2) % (1 << 32)
        want_exc = (i * (i - 1) // 2) % (1 << 32) if i > 0 else 0
        assert int(inc[i]) & 0xffffffff == want_inc
        assert int(exc[i]) & 0xffffffff == want_exc
    assert (inc.astype(np.int64) < 0).any()        # some prefix did wrap into the sign bit


def test_arange_f32_exact():
    n = 4096                                       # 4095*4096/2 < 2^24: every prefix is exact in f32
    x = np.arange(n, dtype=np.float32)
    inc = oracle.scan(x, "f32", "add")
    i = np.arange(n, dtype=np.float64)
    assert np.array_equal(inc.astype(np.float64), i * (i + 1) / 2)


def test_arange_minmax():
    n = 1000
    up = np.arange(n, dtype=np.int64)
    assert np.array_equal(oracle.scan(up, "i64", "max"), up)
    assert np.array_equal(oracle.scan(up, "i64", "min"), np.zeros(n, np.int64))
    down = up[::-1].copy()
    assert np.array_equal(oracle.scan(down, "i64", "min"), down)
    assert np.array_equal(oracle.scan(down, "i64", "max"), np.full(n, n - 1, np.int64))


# ---- invariants between separately computed results -----------------------------------

@pytest.mark.parametrize("dt", ALL_DT)
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_shift_invariant(dt, op):
    x = random_input(dt, 777, 3)
    inc = oracle.scan(x, dt, op)
    exc = oracle.scan(x, dt, op, exclusive=True)
    if dt in oracle.FLOATS and op == "add" and dt != "f64":
        # both are roundings of the same double accumulators: compare those
        _, ri, _ = oracle.scan(x, dt, op, want_ref=True)
        _, re, _ = oracle.scan(x, dt, op, exclusive=True, want_ref=True)
        assert re[0] == 0.0 and np.array_equal(re[1:], ri[:-1])
    assert np.array_equal(exc[1:].view(np.uint8), inc[:-1].view(np.uint8)) or \
        exc[1:].tobytes() == inc[:-1].tobytes()


@pytest.mark.parametrize("dt", ["i32", "u32", "i64", "u64"])
def test_inclusive_is_exclusive_combined_with_input(dt):
    x = random_input(dt, 1000, 5)
    for op in ("add", "min", "max"):
        inc = oracle.scan(x, dt, op)
        exc = oracle.scan(x, dt, op, exclusive=True)
        if op == "add":
            u = np.uint32 if dt in ("i32", "u32") else np.uint64
            want = (exc.view(u) + x.view(u)).view(INT_DT[dt])   # numpy wraps
        elif op == "min":
            want = np.minimum(exc, x)
        else:
            want = np.maximum(exc, x)
        assert np.array_equal(inc, want), op


def test_rows_are_independent():
    x = random_input("f32", 7 * 301, 9).reshape(7, 301)
    for op in ("add", "min", "max"):
        for ex in (False, True):
            whole = oracle.scan(x, "f32", op, exclusive=ex)
            for r in range(7):
                assert np.array_equal(whole[r], oracle.scan(x[r].copy(), "f32", op, exclusive=ex))


# ---- independent library routines ------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "f64", "bf16", "f16"])
def test_fp_add_matches_numpy_accumulate(dt):
    x = random_input(dt, 20000, 21)
    xf = as_float(x, dt)                           # decoded by torch/numpy
    acc = np.add.accumulate(xf)                    # sequential double fold
    out, ref, absref = oracle.scan(x, dt, "add", want_ref=True)
    assert np.array_equal(ref, acc)
    assert np.array_equal(absref, np.add.accumulate(np.abs(xf)))
    if dt == "f64":
        assert np.array_equal(out, acc)
    elif dt == "f32":
        assert np.array_equal(out, acc.astype(np.float32))
    else:
        assert np.array_equal(out, f32_to_bits(acc.astype(np.float32), dt))
    _, eref, _ = oracle.scan(x, dt, "add", exclusive=True, want_ref=True)
    assert eref[0] == 0.0 and np.array_equal(eref[1:], acc[:-1])


@pytest.mark.parametrize("dt", ["i32", "u32", "i64", "u64"])
def test_int_add_matches_numpy_cumsum(dt):
    x = random_input(dt, 20000, 23)
    u = np.uint32 if dt in ("i32", "u32") else np.uint64
    want = np.cumsum(x.view(u), dtype=u).view(INT_DT[dt])       # wraps mod 2^w
    assert np.array_equal(oracle.scan(x, dt, "add"), want)


@pytest.mark.parametrize("dt", ["f32", "f64", "bf16", "f16", "i32", "u32", "i64", "u64"])
def test_minmax_match_numpy_accumulate(dt):
    x = random_input(dt, 20000, 25)
    xv = as_float(x, dt) if dt in oracle.FLOATS else x
    for op, uf in (("min", np.minimum), ("max", np.maximum)):
        got = oracle.scan(x, dt, op)
        want = uf.accumulate(xv)
        gv = as_float(got, dt) if dt in oracle.FLOATS else got
        assert np.array_equal(gv, want), op


def test_bf16_rounding_matches_torch():
    specials = np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.005859375, 1.01171875, 3.4e38,
                         -3.4e38, 3.3961776e38, 1e-40, -1e-40, 1.4e-45, 65504.0, np.inf, -np.inf,
                         2.0 ** -126, 2.0 ** -133, 0.1, 1.0 / 3.0], dtype=np.float32)
    rng = np.random.default_rng(31)
    rand = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32)
    bits = rng.integers(0, 1 << 32, size=5000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    v = np.concatenate([specials, rand, bits])
    assert np.array_equal(oracle.f32_to_bf16(v), workloads.to_bf16_bits(v))
    # NaN: quiet, sign kept
    q = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (q & 0x7f80) == 0x7f80 and (q & 0x0040)
    # widening is exact
    h = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    h = h[(h & 0x7f80) != 0x7f80]
    assert np.array_equal(oracle.bf16_to_f32(h), bits_to_f32(h, "bf16"))


def test_f16_rounding_matches_numpy():
    specials = np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e6, -1e6,
                         2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
                         3.0 * 2.0 ** -25, 6.1e-5, 1.00048828125, 1.00146484375,
                         np.inf, -np.inf, 0.1, -2.0 / 3.0], dtype=np.float32)
    rng = np.random.default_rng(33)
    rand = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000))).astype(np.float32)
    bits = rng.integers(0, 1 << 32, size=5000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    v = np.concatenate([specials, rand, bits])
    assert np.array_equal(oracle.f32_to_f16(v), workloads.to_f16_bits(v))
    h = np.arange(0, 1 << 16, 3, dtype=np.uint16)
    h = h[(h & 0x7c00) != 0x7c00]
    assert np.array_equal(oracle.f16_to_f32(h), bits_to_f32(h, "f16"))


# ---- brute force on tiny inputs -----------------------------------------------------------

def _brute_prefix(vals, dt, op, upto):
    """Combine vals[0:upto] independently of the oracle."""
    seq = vals[:upto]
    if op == "add":
        if dt in oracle.FLOATS:
            return functools.reduce(operator.add, [float(v) for v in seq], 0.0)
        w = 32 if dt in ("i32", "u32") else 64
        s = sum(int(v) for v in seq) % (1 << w)
        if dt in ("i32", "i64") and s >= 1 << (w - 1):
            s -= 1 << w
        return s
    if not seq:
        return None
    return min(seq) if op == "min" else max(seq)


@pytest.mark.parametrize("dt", ALL_DT)
def test_brute_force_tiny(dt):
    for n in range(0, 11):
        x = random_input(dt, n, 100 + n)
        xv = [float(v) for v in as_float(x, dt)] if dt in oracle.FLOATS else [int(v) for v in x]
        for op in ("add", "min", "max"):
            inc = oracle.scan(x, dt, op)
            exc = oracle.scan(x, dt, op, exclusive=True)
            for i in range(n):
                wi = _brute_prefix(xv, dt, op, i + 1)
                we = _brute_prefix(xv, dt, op, i)
                gi = as_float(inc[i:i + 1], dt)[0] if dt in oracle.FLOATS else int(inc[i])
                ge = as_float(exc[i:i + 1], dt)[0] if dt in oracle.FLOATS else int(exc[i])
                if op == "add" and dt in oracle.FLOATS:
                    # one rounding of the double fold to the output format
                    wi = float(as_float(_round_to(dt, wi), dt)[0])
                    we = float(as_float(_round_to(dt, we), dt)[0])
                if we is None:                     # empty prefix: the identity
                    continue
                assert gi == wi and ge == we, (dt, op, n, i)


def _round_to(dt, v):
    if dt == "f64":
        return np.array([v], np.float64)
    f = np.array([v], np.float32)
    if dt == "f32":
        return f
    return f32_to_bits(f, dt)


def test_empty_inputs():
    for dt in ALL_DT:
        x = np.zeros(0, oracle.STORAGE[dt])
        assert oracle.scan(x, dt, "add").shape == (0,)
        assert oracle.scan(np.zeros((0, 5), oracle.STORAGE[dt]), dt, "max").shape == (0, 5)
    out, k = oracle.select(np.zeros(0, np.float32), np.zeros(0, np.uint8))
    assert k == 0 and out.shape == (0,)


# ---- select ---------------------------------------------------------------------------------

def test_select_every_flag_pattern():
    n = 10
    x = np.arange(100, 100 + n, dtype=np.int32)
    for pattern in itertools.product((0, 1), repeat=n):
        f = np.array(pattern, np.uint8)
        out, k = oracle.select(x, f)
        want = x[f.astype(bool)]
        assert k == want.size and np.array_equal(out[:k], want)
        assert not out[k:].any()                   # nothing written past the count


def test_select_nonzero_bytes_count_as_selected():
    x = np.arange(6, dtype=np.int64)
    f = np.array([0, 2, 255, 0, 1, 128], np.uint8)
    out, k = oracle.select(x, f)
    assert k == 4 and out[:k].tolist() == [1, 2, 4, 5]


@pytest.mark.parametrize("itemsize", [1, 2, 4, 8, 16])
def test_select_element_sizes_bit_copy(itemsize):
    rng = np.random.default_rng(itemsize)
    n = 3000
    raw = rng.integers(0, 256, size=n * itemsize, dtype=np.uint8)
    x = raw.view(np.dtype((np.void, itemsize)))
    f = (rng.random(n) < 0.3).astype(np.uint8)
    out, k = oracle.select(x, f)
    assert out[:k].tobytes() == x[f.astype(bool)].tobytes()


def test_select_keeps_nan_payloads():
    x = np.array([0x7fc00001, 0xffa00002, 0x3f800000], dtype=np.uint32).view(np.float32)
    out, k = oracle.select(x, np.array([1, 1, 0], np.uint8))
    assert k == 2 and out[:2].view(np.uint32).tolist() == [0x7fc00001, 0xffa00002]


# ---- product scans ("mul") ---------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "f64", "bf16", "f16"])
def test_prod_powers_of_two_exact(dt):
    """x = 2 everywhere: the inclusive prefix is 2^(i+1), the exclusive 2^i (exact)."""
    n = 15 if dt == "f16" else 100                 # stay inside each format's range
    x = np.full(n, 2.0, np.float32)
    xs = x.astype(np.float64) if dt == "f64" else (x if dt == "f32" else f32_to_bits(x, dt))
    inc = as_float(oracle.scan(xs, dt, "mul"), dt)
    exc = as_float(oracle.scan(xs, dt, "mul", exclusive=True), dt)
    assert np.array_equal(inc, 2.0 ** np.arange(1, n + 1))
    assert np.array_equal(exc, 2.0 ** np.arange(0, n))


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_prod_signs_and_alternation(dt):
    rng = np.random.default_rng(7)
    s = rng.choice([-1.0, 1.0], size=300).astype(np.float32)
    got = as_float(oracle.scan(f32_to_bits(s, dt) if dt != "f32" else s, dt, "mul"), dt)
    # the sign of a product of +-1 is (-1)^(number of negatives so far)
    want = np.where(np.cumsum(s < 0) % 2 == 1, -1.0, 1.0)
    assert np.array_equal(got, want)
    alt = np.tile(np.array([2.0, 0.5], np.float32), 50)
    got = as_float(oracle.scan(f32_to_bits(alt, dt) if dt != "f32" else alt, dt, "mul"), dt)
    assert np.array_equal(got, np.tile([2.0, 1.0], 50))


def test_prod_zero_absorbs():
    x = np.array([3.0, -2.0, 0.0, 5.0, -7.0], np.float32)
    inc = oracle.scan(x, "f32", "mul")
    assert inc[:2].tolist() == [3.0, -6.0]
    assert np.all(inc[2:] == 0.0)


@pytest.mark.parametrize("dt", ["f32", "f64", "bf16", "f16"])
def test_prod_matches_numpy_accumulate(dt):
    """Against numpy's sequential multiply.accumulate in float64, rounded once."""
    rng = np.random.default_rng(21)
    n = 4096
    v = (rng.choice([-1.0, 1.0], size=n) * (1.0 + rng.uniform(-1 / 64, 1 / 64, size=n)))
    if dt == "f64":
        x = v.astype(np.float64)
        xv = x
    elif dt == "f32":
        x = v.astype(np.float32)
        xv = x.astype(np.float64)
    else:
        x = f32_to_bits(v.astype(np.float32), dt)
        xv = bits_to_f32(x, dt).astype(np.float64)
    acc = np.multiply.accumulate(xv)
    got, ref, _ = oracle.scan(x, dt, "mul", want_ref=True)
    assert np.array_equal(ref, acc)
    if dt == "f64":
        assert np.array_equal(got, acc)
    elif dt == "f32":
        assert np.array_equal(got, acc.astype(np.float32))
    else:
        assert np.array_equal(got, f32_to_bits(acc.astype(np.float32), dt))


@pytest.mark.parametrize("dt", ["i32", "u32", "i64", "u64"])
def test_int_prod_wraps_like_numpy(dt):
    rng = np.random.default_rng(5)
    x = rng.integers(-50 if dt[0] == "i" else 0, 50, size=500).astype(INT_DT[dt])
    with np.errstate(over="ignore"):
        want = np.multiply.accumulate(x, dtype=INT_DT[dt])
    assert np.array_equal(oracle.scan(x, dt, "mul"), want)


@pytest.mark.parametrize("dt", ["f32", "f64", "bf16", "f16"])
def test_prod_brute_force_tiny(dt):
    """Each prefix recomputed with math.prod (sequential double products), rounded once."""
    for n in range(0, 9):
        x = random_input(dt, n, 300 + n)
        xv = [float(v) for v in as_float(x, dt)]
        inc = as_float(oracle.scan(x, dt, "mul"), dt)
        exc = as_float(oracle.scan(x, dt, "mul", exclusive=True), dt)
        for i in range(n):
            wi = float(as_float(_round_to(dt, math.prod(xv[:i + 1])), dt)[0])
            we = float(as_float(_round_to(dt, math.prod(xv[:i])), dt)[0])
            assert inc[i] == wi and exc[i] == we, (dt, n, i)


# ---- reduce -----------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ALL_DT)
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_reduce_is_last_inclusive_prefix(dt, op):
    """Two separately written loops of the oracle agree: reduce == inclusive[-1]."""
    for n in (1, 2, 17, 1000):
        x = random_input(dt, n, 40 + n)
        red = oracle.reduce(x, dt, op)
        inc = oracle.scan(x, dt, op)
        assert red.tobytes() == inc[-1:].tobytes(), (dt, op, n)


@pytest.mark.parametrize("dt", ALL_DT)
def test_reduce_empty_is_identity(dt, golden):
    g = golden("identities.json")
    for op in ("add", "min", "max"):
        red = oracle.reduce(np.zeros(0, oracle.STORAGE[dt]), dt, op)
        want = g[op][dt]
        if dt in oracle.FLOATS:
            assert as_float(red, dt)[0] == float(want), (dt, op)
        else:
            assert int(red[0]) == int(want), (dt, op)


@pytest.mark.parametrize("dt", ["i32", "u32", "i64", "u64"])
def test_reduce_int_matches_numpy(dt):
    x = random_input(dt, 100000, 9)
    with np.errstate(over="ignore"):
        assert oracle.reduce(x, dt, "add")[0] == np.add.reduce(x, dtype=INT_DT[dt])
    assert oracle.reduce(x, dt, "min")[0] == x.min()
    assert oracle.reduce(x, dt, "max")[0] == x.max()


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_reduce_fp_add_near_exact_sum(dt):
    """The double fold is within n * 2^-53 * sum|x| of math.fsum's exact sum."""
    x = random_input(dt, 200000, 13)
    red, ref, absref = oracle.reduce(x, dt, "add", want_ref=True)
    exact = math.fsum(float(v) for v in x)
    assert abs(ref - exact) <= x.size * 2.0 ** -53 * absref
    assert abs(absref - math.fsum(abs(float(v)) for v in x)) <= x.size * 2.0 ** -53 * absref
    if dt == "f32":
        assert red[0] == np.float32(ref)


def test_reduce_minmax_signed_zero_takes_later(golden):
    g = golden("tie_break.json")
    for case in g["cases"]:
        x = np.array([float(v) for v in case["input"]], dtype=np.float32)
        red = oracle.reduce(x, "f32", case["op"])
        want = np.array([float(case["inclusive"][-1])], dtype=np.float32)
        assert red.view(np.uint32).tolist() == want.view(np.uint32).tolist(), case


# ---- reduce-by-key -------------------------------------------------------------------------------

def test_page_reduce_by_key_example(golden):
    g = golden("reduce_by_key_example.json")
    ko, vo, r = oracle.reduce_by_key(np.array(g["keys"], np.int32), np.array(g["values"], np.int32),
                                     "i32", "i32")
    assert r == g["num_runs"]
    assert ko[:r].tolist() == g["keys_out"] and vo[:r].tolist() == g["values_out"]
    assert not ko[r:].any() and not vo[r:].any()          # nothing written past the count


def _groupby_runs(keys, values, key_is_float):
    """Independent run split: a new run wherever the key differs from its predecessor."""
    runs = []
    for i, (k, v) in enumerate(zip(keys, values)):
        same = i > 0 and ((keys[i - 1] == k) if not key_is_float else
                          (float(keys[i - 1]) == float(k)))
        if same:
            runs[-1][1].append(v)
        else:
            runs.append((k, [v]))
    return runs


@pytest.mark.parametrize("kd", ["i32", "u32", "f32"])
@pytest.mark.parametrize("vd", ["i32", "u32", "f32"])
def test_reduce_by_key_brute_force(kd, vd):
    rng = np.random.default_rng(100 * ["i32", "u32", "f32"].index(kd) + ["i32", "u32", "f32"].index(vd))
    for n in (0, 1, 2, 3, 7, 50, 500):
        keys = rng.integers(0, 3, size=n).astype(oracle.STORAGE[kd])    # short random runs
        if vd == "f32":
            values = rng.uniform(-2, 2, size=n).astype(np.float32)
        else:
            values = rng.integers(np.iinfo(oracle.STORAGE[vd]).min, np.iinfo(oracle.STORAGE[vd]).max,
                                  size=n, endpoint=True).astype(oracle.STORAGE[vd])
        ko, vo, r = oracle.reduce_by_key(keys, values, kd, vd)
        runs = _groupby_runs(keys.tolist(), values.tolist(), kd == "f32")
        assert r == len(runs), (kd, vd, n)
        for j, (k, vs) in enumerate(runs):
            assert ko[j] == k
            if vd == "f32":
                assert vo[j] == np.float32(math.fsum(vs)) or \
                    abs(float(vo[j]) - math.fsum(vs)) <= 2 ** -24 * abs(math.fsum(vs)) + 1e-30
            else:
                w = sum(int(v) for v in vs) % (1 << 32)
                assert int(np.array([vo[j]]).view(np.uint32)[0]) == w


def test_reduce_by_key_invariants():
    rng = np.random.default_rng(31)
    n = 200_000
    lengths = rng.geometric(1 / 8, size=n)
    keys = np.repeat(rng.integers(0, 1 << 20, size=lengths.size), lengths)[:n].astype(np.int32)
    values = rng.integers(-1000, 1000, size=n).astype(np.int32)
    ko, vo, r = oracle.reduce_by_key(keys, values, "i32", "i32")
    heads = np.flatnonzero(np.r_[True, keys[1:] != keys[:-1]])
    assert r == heads.size
    assert np.array_equal(ko[:r], keys[heads])                        # the runs' first keys
    assert np.array_equal(vo[:r], np.add.reduceat(values, heads))     # numpy's segment sums
    assert vo[:r].sum(dtype=np.int64) == values.sum(dtype=np.int64)


def test_reduce_by_key_float_keys_nan_and_signed_zero():
    nan = np.float32("nan")
    keys = np.array([1.0, nan, nan, 0.0, -0.0, 0.0, 2.0, 2.0], np.float32)
    values = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.int32)
    ko, vo, r = oracle.reduce_by_key(keys, values, "f32", "i32")
    # each NaN is its own run; +0 and -0 compare equal, and the run keeps its first key (+0)
    assert r == 5
    assert vo[:r].tolist() == [1, 2, 3, 15, 15]
    assert np.isnan(ko[1]) and np.isnan(ko[2])
    assert ko[3] == 0.0 and math.copysign(1.0, float(ko[3])) == 1.0


def test_reduce_by_key_f32_values_double_sum():
    rng = np.random.default_rng(33)
    keys = np.repeat(np.arange(50, dtype=np.int32), 1000)
    values = rng.uniform(-1, 1, size=keys.size).astype(np.float32)
    ko, vo, r, ref, absref = oracle.reduce_by_key(keys, values, "i32", "f32", want_ref=True)
    assert r == 50
    for j in range(r):
        seg = values[j * 1000:(j + 1) * 1000].astype(np.float64)
        exact = math.fsum(seg)
        assert abs(ref[j] - exact) <= 1000 * 2.0 ** -53 * absref[j]
        assert vo[j] == np.float32(ref[j])


# ---- radix-sort order ----------------------------------------------------------------------------

def test_page_sort_example(golden):
    g = golden("sort_example.json")
    k, v = oracle.sort(np.array(g["keys"], np.int32), "i32", np.array(g["values"], np.int32))
    assert k.tolist() == g["sorted_keys"] and v.tolist() == g["sorted_values"]


@pytest.mark.parametrize("dt", ["i32", "u32", "i64", "u64"])
def test_sort_ints_match_numpy_stable(dt):
    rng = np.random.default_rng(51)
    t = INT_DT[dt]
    info = np.iinfo(t)
    for n, hi in ((10000, None), (10000, 7)):           # full range, and many duplicates
        x = (rng.integers(info.min, info.max, size=n, endpoint=True, dtype=t) if hi is None else
             rng.integers(0, hi, size=n).astype(t))
        idx = np.arange(n, dtype=np.int64)
        k, v = oracle.sort(x, dt, idx)
        want = np.argsort(x, kind="stable")                # numpy compares the native integers
        assert np.array_equal(v, want) and np.array_equal(k, x[want])


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_sort_floats_match_numpy_without_nan_or_zero(dt):
    rng = np.random.default_rng(52)
    f = np.float32 if dt == "f32" else np.float64
    x = rng.choice(rng.standard_normal(300).astype(f), size=20000)        # duplicates, no zeros
    x[::97] = np.inf
    x[::89] = -np.inf
    idx = np.arange(x.size)
    k, v = oracle.sort(x, dt, idx)
    want = np.argsort(x, kind="stable")
    assert np.array_equal(v, want)


def _brute_sort_key(x):
    """An independent statement of the order: NaNs last; otherwise by value,
    with -0 before +0."""
    xf = float(x)
    if math.isnan(xf):
        return (1, 0.0, 0)
    return (0, xf, 0 if (xf == 0.0 and math.copysign(1.0, xf) < 0) else 1)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_sort_floats_brute_force_specials(dt):
    f = np.float32 if dt == "f32" else np.float64
    alphabet = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 1.5, -1.5, 3.0], f)
    rng = np.random.default_rng(53)
    for n in range(0, 40):
        x = alphabet[rng.integers(0, alphabet.size, size=n)]
        idx = np.arange(n)
        k, v = oracle.sort(x, dt, idx)
        want = sorted(range(n), key=lambda i: _brute_sort_key(x[i]))    # Python's sort is stable
        assert v.tolist() == want, (n, x)
        assert k.view(np.uint8).tobytes() == x[want].view(np.uint8).tobytes()   # bits moved intact


def test_sort_signed_zero_and_nan_order():
    nan_p = np.float32(np.nan)
    nan_n = np.array([0xffc00001], np.uint32).view(np.float32)[0]
    x = np.array([0.0, -0.0, nan_n, 1.0, nan_p, -0.0, -np.inf, 0.0], np.float32)
    k, v = oracle.sort(x, "f32", np.arange(8))
    assert v.tolist() == [6, 1, 5, 0, 7, 3, 2, 4]


def test_sort_end_bit_uses_low_bits_only():
    rng = np.random.default_rng(54)
    x = rng.integers(0, 1 << 32, size=5000, dtype=np.uint64).astype(np.uint32)
    for end_bit in (8, 16, 24):
        k, v = oracle.sort(x, "u32", np.arange(x.size), end_bit=end_bit)
        want = np.argsort(x & np.uint32((1 << end_bit) - 1), kind="stable")
        assert np.array_equal(v, want)
    # i32 with end_bit 32 is the full signed order; with fewer bits the sign flip is masked away
    y = rng.integers(-1000, 1000, size=3000).astype(np.int32)
    _, v = oracle.sort(y, "i32", np.arange(y.size), end_bit=16)
    want = np.argsort((y.view(np.uint32) ^ np.uint32(1 << 31)) & np.uint32(0xffff), kind="stable")
    assert np.array_equal(v, want)


@pytest.mark.parametrize("dt", ["u32", "i32", "f32", "u64", "i64", "f64"])
def test_sort_output_is_sorted_permutation(dt):
    rng = np.random.default_rng(55)
    raw = rng.integers(0, 256, size=8 * 5000, dtype=np.uint8)
    x = raw.view(oracle.STORAGE[dt])[:5000].copy()        # arbitrary bit patterns, NaNs included
    k, v = oracle.sort(x, dt, np.arange(x.size))
    img = oracle.sort_image(k, dt)
    assert (np.diff(img.astype(object) if img.dtype == np.uint64 else img.astype(np.int64)) >= 0).all()
    assert sorted(v.tolist()) == list(range(x.size))
    assert np.array_equal(k.view(np.uint8), x[v].view(np.uint8))
    # stability: equal images keep increasing original positions
    same = img[1:] == img[:-1]
    assert (v[1:][same] > v[:-1][same]).all()

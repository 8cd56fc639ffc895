"""GPU parity of the operations beyond the five workloads' own: row-wise
product scans, the device-wide inclusive scan and the device-wide reduction,
each through the C ABI against the CPU oracle.

* products: within the float32 product bound of tests/parity.py
  (check_fp_mul), plus closed forms that must be exact;
* inclusive device scans: bit-exact for integers and min/max, the float-add
  tolerance otherwise (as for the exclusive scan);
* reductions: bit-exact for integers and min/max (signed zeros included),
  and the float-add tolerance at the last prefix for floating add.
"""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from parity import FP_ABS, FP_REL, check_exact, check_fp_add, check_fp_mul
from gpu_util import DEV_SIZES, ROW_SHAPES, STORE_T, from_dev, note, rand_input, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# row-wise product scans
# ---------------------------------------------------------------------------

def prod_input(dt, shape, seed):
    f = workloads.near_one_f32(shape, seed)
    if dt == "f32":
        return f
    if dt == "bf16":
        return workloads.to_bf16_bits(f)
    return workloads.to_f16_bits(f)


def compare_prod(gpu, x, dt, excl, label):
    _, ref, _ = oracle.scan(x, dt, "mul", exclusive=excl, want_ref=True)
    n = x.shape[-1]
    m = np.arange(n) + (0 if excl else 1)           # factors behind each output
    return check_fp_mul(gpu, ref, np.broadcast_to(m, x.shape), dt, label)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("excl", [False, True], ids=["incl", "excl"])
def test_rows_prod_shapes(dt, excl):
    for i, (rows, n) in enumerate(ROW_SHAPES):
        label = f"scan_rows {dt} mul excl={excl} [{rows},{n}]"
        x = prod_input(dt, (rows, n), 6000 + i)
        out = sc.scan_rows(to_dev(x, dt), op="mul", exclusive=excl)
        torch.cuda.synchronize()
        compare_prod(from_dev(out, dt), x, dt, excl, label)


@pytest.mark.parametrize("which", ["f32", "bf16", "bf16_ragged"])
@pytest.mark.parametrize("excl", [False, True], ids=["incl", "excl"])
def test_rows_prod_full(which, excl):
    if which == "f32":
        rows, n = workloads.FULL["rows_f32"]
        x, dt = workloads.prod_rows_f32(rows, n), "f32"
    else:
        rows, n = workloads.FULL["rows_bf16" if which == "bf16" else "rows_bf16_ragged"]
        x, dt = workloads.prod_rows_bf16(rows, n), "bf16"
    label = f"scan_rows {dt} mul excl={excl} [{rows},{n}]"
    note(label)
    out = sc.scan_rows(to_dev(x, dt), op="mul", exclusive=excl)
    torch.cuda.synchronize()
    r = compare_prod(from_dev(out, dt), x, dt, excl, label)
    note(f"  max err/bound {r:.3g}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rows_prod_powers_of_two_exact(dt):
    # 2^(i+1) (inclusive) and 2^i (exclusive) are exact in both formats up to 2^127
    rows, n = 40, 126
    x = torch.full((rows, n), 2.0, dtype=STORE_T[dt], device="cuda")
    for excl in (False, True):
        out = sc.scan_rows(x, op="mul", exclusive=excl).float().cpu()
        want = 2.0 ** (torch.arange(n, dtype=torch.float64) + (0 if excl else 1))
        assert torch.equal(out.double(), want.expand(rows, n)), (dt, excl)


def test_rows_prod_signs_exact():
    # products of +-1 are exactly +-1 with the parity of the negatives so far
    rng = np.random.default_rng(17)
    s = rng.choice(np.array([-1.0, 1.0], np.float32), size=(9, 20000))
    out = from_dev(sc.scan_rows(to_dev(s, "f32"), op="mul"), "f32")
    want = np.where(np.cumsum(s < 0, axis=1) % 2 == 1, -1.0, 1.0).astype(np.float32)
    assert np.array_equal(out, want)


# ---------------------------------------------------------------------------
# device-wide inclusive scan
# ---------------------------------------------------------------------------

def compare_incl(gpu, x, dt, op, label):
    if op == "add" and dt in oracle.FLOATS:
        ora, ref, absref = oracle.scan(x, dt, op, exclusive=False, want_ref=True)
        return check_fp_add(gpu, ora, ref, absref, dt, label)
    check_exact(gpu, oracle.scan(x, dt, op, exclusive=False), label)
    return None


@pytest.mark.parametrize("dt", ["i32", "u32", "f32", "i64", "u64", "f64"])
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_device_inclusive_sizes(dt, op):
    for i, n in enumerate(DEV_SIZES):
        label = f"scan_device_inclusive {dt} {op} n={n}"
        x = rand_input(dt, n, 7000 + i)
        out = sc.scan_device_inclusive(to_dev(x, dt), op=op, dtype=dt)
        torch.cuda.synchronize()
        compare_incl(from_dev(out, dt), x, dt, op, label)


def test_device_inclusive_i32_full():
    x = workloads.dev_i32()
    label = f"scan_device_inclusive i32 add n={x.size}"
    note(label)
    out = sc.scan_device_inclusive(to_dev(x, "i32"), op="add")
    torch.cuda.synchronize()
    compare_incl(from_dev(out, "i32"), x, "i32", "add", label)


@pytest.mark.parametrize("which", ["f32", "i64"])
@pytest.mark.parametrize("op", ["min", "max"])
def test_device_inclusive_minmax_full(which, op):
    x = workloads.dev_f32() if which == "f32" else workloads.dev_i64()
    label = f"scan_device_inclusive {which} {op} n={x.size}"
    note(label)
    out = sc.scan_device_inclusive(to_dev(x, which), op=op)
    torch.cuda.synchronize()
    compare_incl(from_dev(out, which), x, which, op, label)


def test_device_inclusive_misaligned_views():
    for dt in ("i32", "i64", "f32"):
        for off_in, off_out in ((1, 1), (1, 0), (0, 3), (9, 9)):
            n = 100_003
            x = rand_input(dt, n, 98)
            big_in = torch.zeros(n + 16, dtype=STORE_T[dt], device="cuda")
            big_out = torch.zeros(n + 16, dtype=STORE_T[dt], device="cuda")
            xin = big_in[off_in:off_in + n]
            xin.copy_(to_dev(x, dt))
            yout = big_out[off_out:off_out + n]
            for op in ("add", "max"):
                sc.scan_device_inclusive(xin, op=op, out=yout)
                torch.cuda.synchronize()
                compare_incl(from_dev(yout, dt), x, dt, op,
                             f"misaligned inclusive {dt} {op} in+{off_in} out+{off_out}")
            assert not big_out[:off_out].any() and not big_out[off_out + n:].any()


def test_device_inclusive_signed_zero():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 2.0, -2.0], np.float32)
    x = vals[np.random.default_rng(16).integers(0, len(vals), size=200_000)]
    for op in ("min", "max"):
        out = sc.scan_device_inclusive(to_dev(x, "f32"), op=op)
        compare_incl(from_dev(out, "f32"), x, "f32", op, f"inclusive signed zeros {op}")


# ---------------------------------------------------------------------------
# device-wide reduction
# ---------------------------------------------------------------------------

# around the run (512 vectors) and workgroup (4 runs) boundaries of the first
# launch for 4- and 8-byte elements, and past 8192 runs, where waves take
# several runs each
RED_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 2049, 4096, 8191, 8192,
             8193, 100_003, 1_000_003, 9_000_001, 20_000_003]


def compare_reduce(gpu, x, dt, op, label):
    if op == "add" and dt in oracle.FLOATS:
        ora, ref, absref = oracle.reduce(x, dt, op, want_ref=True)
        g = float(np.asarray(gpu, np.float64)[0])
        if dt == "f64":
            bound = 1e-12 * absref + 1e-300
        else:
            bound = FP_REL * absref + FP_ABS
        assert abs(g - ref) <= bound, f"{label}: gpu={g!r} ref={ref!r} bound={bound!r}"
        return abs(g - ref) / bound
    check_exact(np.asarray(gpu), oracle.reduce(x, dt, op), label)
    return None


@pytest.mark.parametrize("dt", ["i32", "u32", "f32", "i64", "u64", "f64"])
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_reduce_sizes(dt, op):
    for i, n in enumerate(RED_SIZES):
        label = f"reduce_device {dt} {op} n={n}"
        x = rand_input(dt, n, 8000 + i)
        out = sc.reduce_device(to_dev(x, dt), op=op, dtype=dt)
        torch.cuda.synchronize()
        compare_reduce(from_dev(out, dt), x, dt, op, label)


@pytest.mark.parametrize("dt", ["i32", "f32", "i64", "f64"])
def test_reduce_empty_is_identity(dt):
    for op in ("add", "min", "max"):
        x = torch.zeros(0, dtype=STORE_T[dt], device="cuda")
        out = torch.full((1,), 77, dtype=STORE_T[dt], device="cuda")
        sc.reduce_device(x, op=op, out=out)
        got = from_dev(out, dt)
        want = oracle.reduce(np.zeros(0, oracle.STORAGE[dt]), dt, op)
        check_exact(got, want, f"reduce empty {dt} {op}")


def test_reduce_i32_full():
    x = workloads.dev_i32()
    for op in ("add", "min", "max"):
        label = f"reduce_device i32 {op} n={x.size}"
        note(label)
        out = sc.reduce_device(to_dev(x, "i32"), op=op)
        compare_reduce(from_dev(out, "i32"), x, "i32", op, label)


def test_reduce_i32_wraps_full():
    # closed form: sum of 0..n-1 = n(n-1)/2 mod 2^32
    n = workloads.FULL["dev_i32"]
    out = sc.reduce_device(torch.arange(n, dtype=torch.int32, device="cuda"), op="add")
    want = (n * (n - 1) // 2) % (1 << 32)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == want


@pytest.mark.parametrize("which", ["f32", "i64"])
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_reduce_workload4_full(which, op):
    x = workloads.dev_f32() if which == "f32" else workloads.dev_i64()
    label = f"reduce_device {which} {op} n={x.size}"
    note(label)
    out = sc.reduce_device(to_dev(x, which), op=op)
    r = compare_reduce(from_dev(out, which), x, which, op, label)
    if r is not None:
        note(f"  err/bound {r:.3g}")


def test_reduce_misaligned_views():
    for dt in ("i32", "i64", "f32", "f64"):
        for off in (1, 2, 3, 7, 15):
            n = 1_000_003
            x = rand_input(dt, n, 97)
            big = torch.zeros(n + 16, dtype=STORE_T[dt], device="cuda")
            xin = big[off:off + n]
            xin.copy_(to_dev(x, dt))
            for op in ("add", "min", "max"):
                out = sc.reduce_device(xin, op=op)
                compare_reduce(from_dev(out, dt), x, dt, op, f"misaligned reduce {dt} {op} +{off}")


def test_reduce_signed_zero_ties():
    # the later of +0 / -0 wins a tie, exactly as in the sequential fold
    rng = np.random.default_rng(15)
    for i, n in enumerate((5, 1000, 70_001, 3_000_017)):
        for dt in ("f32", "f64"):
            x = rng.choice(np.array([0.0, -0.0, 1.0, 2.0], oracle.STORAGE[dt]), size=n)
            x[-1] = -0.0 if i % 2 else 0.0
            y = rng.choice(np.array([0.0, -0.0, -1.0, -2.0], oracle.STORAGE[dt]), size=n)
            y[-1] = 0.0 if i % 2 else -0.0
            for op, v in (("min", x), ("max", y)):
                out = sc.reduce_device(to_dev(v, dt), op=op)
                compare_reduce(from_dev(out, dt), v, dt, op, f"reduce ties {dt} {op} n={n}")


def test_reduce_scratch_reuse():
    rng = np.random.default_rng(14)
    nmax = 5_000_000
    scratch = torch.full((sc.reduce_device_scratch_bytes(nmax, "i64"),), 0xCD, dtype=torch.uint8,
                         device="cuda")
    out = torch.empty(1, dtype=torch.int64, device="cuda")
    for it in range(8):
        n = int(rng.integers(1, nmax))
        x = rand_input("i64", n, 900 + it)
        sc.reduce_device(to_dev(x, "i64"), op=("add", "min", "max")[it % 3], out=out,
                         scratch=scratch)
        compare_reduce(from_dev(out, "i64"), x, "i64", ("add", "min", "max")[it % 3],
                       f"reduce reuse {it} n={n}")


# ---------------------------------------------------------------------------
# look-back recovery build, inclusive form
# ---------------------------------------------------------------------------

def test_lookback_recovery_build_inclusive():
    from stream_compaction_amd import build as b
    L = sc.load(b.FALLBACK_LIB_PATH)
    stream = torch.cuda.current_stream().cuda_stream
    for i, (dt, op, n) in enumerate([("i32", "add", 3_000_001), ("f32", "max", 1_000_003),
                                     ("i64", "min", 700_001)]):
        x = rand_input(dt, n, 5100 + i)
        xd = to_dev(x, dt)
        yd = torch.empty_like(xd)
        code = sc.DTYPE_CODES[dt]
        need = L.scan_device_scratch_bytes(n, code)
        scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
        sc.check(L.scan_device_inclusive(xd.data_ptr(), yd.data_ptr(), n, code,
                                         sc.OP_CODES[op], scratch.data_ptr(), need, stream))
        torch.cuda.synchronize()
        compare_incl(from_dev(yd, dt), x, dt, op, f"fallback build inclusive {dt} {op} n={n}")


# ---------------------------------------------------------------------------
# reduce-by-key
# ---------------------------------------------------------------------------

def run_lengths_keys(n, mean_run, seed, dt="i32"):
    """Keys in runs of geometric length (mean `mean_run`), each run a random key."""
    rng = np.random.default_rng(seed)
    lengths = rng.geometric(1.0 / mean_run, size=n // max(1, int(mean_run)) + 16)
    while lengths.sum() < n:
        lengths = np.r_[lengths, rng.geometric(1.0 / mean_run, size=lengths.size)]
    keys = np.repeat(rng.integers(0, 8, size=lengths.size), lengths)[:n]
    if dt == "f32":
        return keys.astype(np.float32)
    return keys.astype(oracle.STORAGE[dt])


def rbk_values(n, vd, seed):
    rng = np.random.default_rng(seed)
    if vd == "f32":
        return rng.uniform(-1, 1, size=n).astype(np.float32)
    info = np.iinfo(oracle.STORAGE[vd])
    return rng.integers(info.min, info.max, size=n, endpoint=True).astype(oracle.STORAGE[vd])


def check_rbk(keys, values, kd, vd, label, key_out=None, val_out=None):
    n = keys.size
    kdev, vdev = to_dev(keys, kd), to_dev(values, vd)
    ko = to_dev(np.full(n, 0x5A5A5A5A, np.uint32).view(oracle.STORAGE[kd]), kd) \
        if key_out is None else key_out
    vo = to_dev(np.full(n, 0x5A5A5A5A, np.uint32).view(oracle.STORAGE[vd]), vd) \
        if val_out is None else val_out
    _, _, nr = sc.reduce_by_key(kdev, vdev, ko, vo, key_dtype=kd, value_dtype=vd)
    r = int(nr.item())
    oko, ovo, orr, ref, absref = oracle.reduce_by_key(keys, values, kd, vd, want_ref=True)
    assert r == orr, f"{label}: {r} runs, oracle {orr}"
    gk, gv = from_dev(ko, kd), from_dev(vo, vd)
    check_exact(gk[:r], oko[:r], label + " keys")
    if vd == "f32":
        bound = FP_REL * absref[:r] + FP_ABS
        err = np.abs(gv[:r].astype(np.float64) - ref[:r])
        assert (err <= bound).all(), f"{label}: value out of tolerance at run {np.argmax(err > bound)}"
    else:
        check_exact(gv[:r], ovo[:r], label + " values")
    assert (gk[r:].view(np.uint32) == 0x5A5A5A5A).all(), f"{label}: keys tail written"
    assert (gv[r:].view(np.uint32) == 0x5A5A5A5A).all(), f"{label}: values tail written"
    return r


RBK_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 28671, 28672,
             28673, 100_003, 1_000_003, 3_000_017]


@pytest.mark.parametrize("kd,vd", [("i32", "i32"), ("i32", "f32"), ("u32", "u32"),
                                   ("f32", "f32"), ("f32", "i32")])
@pytest.mark.parametrize("mean_run", [1, 3, 40])
def test_reduce_by_key_sizes(kd, vd, mean_run):
    for i, n in enumerate(RBK_SIZES):
        keys = run_lengths_keys(n, mean_run, 9000 + i, kd)
        values = rbk_values(n, vd, 9100 + i)
        check_rbk(keys, values, kd, vd, f"reduce_by_key {kd}/{vd} mean run {mean_run} n={n}")


def test_reduce_by_key_single_run_and_all_unique():
    n = 2_000_003
    check_rbk(np.zeros(n, np.int32), rbk_values(n, "i32", 1), "i32", "i32", "one run")
    check_rbk(np.arange(n, dtype=np.int32), rbk_values(n, "i32", 2), "i32", "i32", "all unique")


def test_reduce_by_key_float_keys_nan_and_zeros():
    rng = np.random.default_rng(12)
    vals = np.array([np.nan, 0.0, -0.0, 1.0, -1.0], np.float32)
    keys = vals[rng.integers(0, len(vals), size=300_001)]
    check_rbk(keys, rbk_values(keys.size, "i32", 3), "f32", "i32", "nan and signed-zero keys")


def test_reduce_by_key_misaligned_and_aliased():
    n = 200_003
    keys = run_lengths_keys(n, 5, 77)
    values = rbk_values(n, "i32", 78)
    for off_k, off_v in ((1, 1), (0, 3), (2, 1), (21, 21), (21, 5)):
        bk = torch.zeros(n + 32, dtype=torch.int32, device="cuda")
        bv = torch.zeros(n + 32, dtype=torch.int32, device="cuda")
        kin, vin = bk[off_k:off_k + n], bv[off_v:off_v + n]
        kin.copy_(torch.from_numpy(keys).cuda())
        vin.copy_(torch.from_numpy(values).cuda())
        ko, vo, nr = sc.reduce_by_key(kin, vin)
        r = int(nr.item())
        oko, ovo, orr = oracle.reduce_by_key(keys, values, "i32", "i32")
        assert r == orr
        check_exact(ko.cpu().numpy()[:r], oko[:r], f"misaligned keys {off_k},{off_v}")
        check_exact(vo.cpu().numpy()[:r], ovo[:r], f"misaligned values {off_k},{off_v}")
    # keys and values the same array: a run's value is its key times its length
    kd = to_dev(keys, "i32")
    ko, vo, nr = sc.reduce_by_key(kd, kd)
    r = int(nr.item())
    oko, ovo, orr = oracle.reduce_by_key(keys, keys, "i32", "i32")
    assert r == orr
    check_exact(vo.cpu().numpy()[:r], ovo[:r], "aliased inputs")


def test_reduce_by_key_empty():
    k = torch.zeros(0, dtype=torch.int32, device="cuda")
    nr = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    sc.reduce_by_key(k, k.clone(), num_runs=nr)
    assert int(nr.item()) == 0


def test_reduce_by_key_full():
    n = workloads.FULL["rbk"]
    keys, values = workloads.rbk_inputs(n)
    label = f"reduce_by_key i32/f32 n={n} mean run {workloads.RBK_MEAN_RUN}"
    note(label)
    r = check_rbk(keys, values, "i32", "f32", label)
    note(f"  runs {r}")


def test_lookback_recovery_build_reduce_by_key():
    from stream_compaction_amd import build as b
    L = sc.load(b.FALLBACK_LIB_PATH)
    stream = torch.cuda.current_stream().cuda_stream
    n = 2_000_003
    keys = run_lengths_keys(n, 6, 321)
    values = rbk_values(n, "i32", 322)
    kd, vd = to_dev(keys, "i32"), to_dev(values, "i32")
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    nr = torch.empty(1, dtype=torch.int32, device="cuda")
    need = L.reduce_by_key_scratch_bytes(n)
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    sc.check(L.reduce_by_key(kd.data_ptr(), vd.data_ptr(), ko.data_ptr(), vo.data_ptr(),
                             nr.data_ptr(), n, sc.DTYPE_CODES["i32"], sc.DTYPE_CODES["i32"],
                             scratch.data_ptr(), need, stream))
    r = int(nr.item())
    oko, ovo, orr = oracle.reduce_by_key(keys, values, "i32", "i32")
    assert r == orr
    check_exact(ko.cpu().numpy()[:r], oko[:r], "fallback build keys")
    check_exact(vo.cpu().numpy()[:r], ovo[:r], "fallback build values")

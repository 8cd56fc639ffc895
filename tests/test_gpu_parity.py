"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case draws seeded inputs from workloads.py, runs the library on the GPU
and the oracle on the host, and compares element by element: bit-exact for
integer and min/max scans and for select (count, prefix and untouched tail),
within the float-add tolerance of tests/parity.py otherwise.  The full-size
cases are the five workloads at their stated sizes, in the same launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from gpu_util import DEV_SIZES, ROW_SHAPES, STORE_T, from_dev, note, rand_input, to_dev
from parity import check_exact, check_fp_add, decode16

pytestmark = pytest.mark.gpu


def compare_scan(gpu, x, dt, op, exclusive, label):
    if op == "add" and dt in oracle.FLOATS:
        ora, ref, absref = oracle.scan(x, dt, op, exclusive=exclusive, want_ref=True)
        return check_fp_add(gpu, ora, ref, absref, dt, label)
    ora = oracle.scan(x, dt, op, exclusive=exclusive)
    check_exact(gpu, ora, label)
    return None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# row-wise scans
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["add", "min", "max"])
@pytest.mark.parametrize("excl", [False, True], ids=["incl", "excl"])
def test_rows_shapes(dt, op, excl):
    for i, (rows, n) in enumerate(ROW_SHAPES):
        label = f"scan_rows {dt} {op} excl={excl} [{rows},{n}]"
        x = rand_input(dt, (rows, n), 1000 + i)
        out = sc.scan_rows(to_dev(x, dt), op=op, exclusive=excl)
        torch.cuda.synchronize()
        compare_scan(from_dev(out, dt), x, dt, op, excl, label)


@pytest.mark.parametrize("rows,n", [(1 << 20, 1), (1 << 20, 3), (65_537, 2)])
def test_rows_many_tiny_rows(rows, n):
    # about a million one-wave workgroups, each row within one partial vector
    for dt in ("f32", "bf16"):
        x = rand_input(dt, (rows, n), 1500 + n)
        for op, excl in (("add", True), ("max", False), ("min", True)):
            out = sc.scan_rows(to_dev(x, dt), op=op, exclusive=excl)
            torch.cuda.synchronize()
            compare_scan(from_dev(out, dt), x, dt, op, excl,
                         f"scan_rows {dt} {op} excl={excl} [{rows},{n}]")


def test_rows_workload1_full():
    rows, n = workloads.FULL["rows_f32"]
    x = workloads.rows_f32(rows, n)
    xd = to_dev(x, "f32")
    for excl in (False, True):
        label = f"scan_rows f32 add excl={excl} [{rows},{n}]"
        note(label)
        out = sc.scan_rows(xd, op="add", exclusive=excl)
        torch.cuda.synchronize()
        err, ratio = compare_scan(from_dev(out, "f32"), x, "f32", "add", excl, label)
        note(f"  max abs err {err:.3g}, max err/bound {ratio:.3g}")


@pytest.mark.parametrize("shape", [workloads.FULL["rows_bf16"], workloads.FULL["rows_bf16_ragged"]],
                         ids=["8192x8192", "8192x8191"])
def test_rows_workload2_full(shape):
    rows, n = shape
    x = workloads.rows_bf16(rows, n)
    label = f"scan_rows bf16 add excl [{rows},{n}]"
    note(label)
    out = sc.scan_rows(to_dev(x, "bf16"), op="add", exclusive=True)
    torch.cuda.synchronize()
    err, ratio = compare_scan(from_dev(out, "bf16"), x, "bf16", "add", True, label)
    note(f"  max abs err {err:.3g}, max err/bound {ratio:.3g}")


@pytest.mark.parametrize("excl", [False, True], ids=["incl", "excl"])
def test_rows_bf16_ones_closed_form_full(excl):
    # float32 sums of ones are exact (< 2^24): each output is the bf16 rounding
    # of its index (+1), ties to even (257 -> 256, 259 -> 260), bit for bit.
    rows, n = workloads.FULL["rows_bf16"]
    x = torch.ones((rows, n), dtype=torch.bfloat16, device="cuda")
    out = sc.scan_rows(x, op="add", exclusive=excl)
    i = torch.arange(n, dtype=torch.float32) + (0 if excl else 1)
    want = i.to(torch.bfloat16).view(torch.int16)
    got = out.view(torch.int16).cpu()
    assert torch.equal(got, want.expand(rows, n))


def test_rows_misaligned_views():
    # element offsets move the arrays off 16-byte alignment, with equal and unequal phases
    for dt in ("f32", "bf16"):
        for off_in, off_out in ((1, 1), (3, 3), (1, 2), (0, 3), (5, 0)):
            rows, n = 5, 1234
            x = rand_input(dt, (rows * n,), 77)
            big_in = torch.zeros(rows * n + 8, dtype=STORE_T[dt], device="cuda")
            big_out = torch.zeros(rows * n + 8, dtype=STORE_T[dt], device="cuda")
            xin = big_in[off_in:off_in + rows * n]
            xin.copy_(to_dev(x, dt))
            yout = big_out[off_out:off_out + rows * n]
            for op in ("add", "max"):
                for excl in (False, True):
                    sc.scan_rows(xin.view(rows, n), op=op, exclusive=excl, out=yout.view(rows, n))
                    torch.cuda.synchronize()
                    compare_scan(from_dev(yout, dt).reshape(rows, n), x.reshape(rows, n), dt, op,
                                 excl, f"misaligned {dt} {op} in+{off_in} out+{off_out}")
            # nothing outside the output view was written
            assert not big_out[:off_out].any() and not big_out[off_out + rows * n:].any()


@pytest.mark.parametrize("n", [3000, 8191, 16383])
def test_rows_misaligned_long_rows(n):
    # long rows whose windows start on the 128-byte line before each row:
    # equal phases (16-byte vectors) and unequal ones (one element per vector)
    for dt in ("f32", "bf16"):
        rows = 7
        x = rand_input(dt, (rows * n,), 78 + n)
        for off_in, off_out in ((0, 0), (1, 1), (5, 5), (13, 13), (1, 2), (0, 3)):
            big_in = torch.zeros(rows * n + 16, dtype=STORE_T[dt], device="cuda")
            big_out = torch.zeros(rows * n + 16, dtype=STORE_T[dt], device="cuda")
            xin = big_in[off_in:off_in + rows * n]
            xin.copy_(to_dev(x, dt))
            yout = big_out[off_out:off_out + rows * n]
            for op, excl in (("add", True), ("max", False)):
                sc.scan_rows(xin.view(rows, n), op=op, exclusive=excl, out=yout.view(rows, n))
                torch.cuda.synchronize()
                compare_scan(from_dev(yout, dt).reshape(rows, n), x.reshape(rows, n), dt, op, excl,
                             f"long rows {dt} [{rows},{n}] {op} in+{off_in} out+{off_out}")
            assert not big_out[:off_out].any() and not big_out[off_out + rows * n:].any()


def test_rows_signed_zero_and_inf():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0], np.float32)
    rng = np.random.default_rng(5)
    x = vals[rng.integers(0, len(vals), size=(4, 3000))]
    for op in ("min", "max"):
        for excl in (False, True):
            out = sc.scan_rows(to_dev(x, "f32"), op=op, exclusive=excl)
            compare_scan(from_dev(out, "f32"), x, "f32", op, excl, f"signed zeros {op}")


def test_rows_empty():
    for shape in ((0, 5), (5, 0), (0, 0)):
        x = torch.zeros(shape, dtype=torch.float32, device="cuda")
        out = sc.scan_rows(x)
        assert out.shape == shape


# ---------------------------------------------------------------------------
# device-wide exclusive scan
# ---------------------------------------------------------------------------



@pytest.mark.parametrize("dt", ["i32", "u32", "f32", "i64", "u64", "f64"])
@pytest.mark.parametrize("op", ["add", "min", "max"])
def test_device_sizes(dt, op):
    for i, n in enumerate(DEV_SIZES):
        label = f"scan_device {dt} {op} n={n}"
        x = rand_input(dt, n, 2000 + i)
        out = sc.scan_device(to_dev(x, dt), op=op, dtype=dt)
        torch.cuda.synchronize()
        compare_scan(from_dev(out, dt), x, dt, op, True, label)


@pytest.mark.parametrize("n", [workloads.FULL["dev_i32"], workloads.FULL["dev_i32_odd"]],
                         ids=["2^28", "2^28-37"])
def test_device_workload3_full(n):
    x = workloads.dev_i32()[:n]
    label = f"scan_device i32 add n={n}"
    note(label)
    out = sc.scan_device(to_dev(x, "i32"), op="add")
    torch.cuda.synchronize()
    compare_scan(from_dev(out, "i32"), x, "i32", "add", True, label)


def test_device_arange_wraps_full():
    # closed form: exclusive sum of 0..i-1 = i(i-1)/2, reduced mod 2^32
    n = workloads.FULL["dev_i32"]
    x = torch.arange(n, dtype=torch.int32, device="cuda")
    out = sc.scan_device(x, op="add").cpu().numpy().view(np.uint32)
    i = np.arange(n, dtype=np.uint64)
    want = ((i * (i - np.uint64(1))) // np.uint64(2)) & np.uint64(0xffffffff)
    want[0] = 0
    assert np.array_equal(out.astype(np.uint64), want)


def test_device_ones_full():
    n = workloads.FULL["dev_i32"]
    out = sc.scan_device(torch.ones(n, dtype=torch.int32, device="cuda"), op="add")
    assert torch.equal(out.cpu(), torch.arange(n, dtype=torch.int32))


@pytest.mark.parametrize("which", ["f32", "i64"])
@pytest.mark.parametrize("op", ["min", "max"])
def test_device_workload4_full(which, op):
    x = workloads.dev_f32() if which == "f32" else workloads.dev_i64()
    label = f"scan_device {which} {op} n={x.size}"
    note(label)
    out = sc.scan_device(to_dev(x, which), op=op)
    torch.cuda.synchronize()
    compare_scan(from_dev(out, which), x, which, op, True, label)


def test_device_misaligned_views():
    for dt in ("i32", "i64", "f32"):
        for off_in, off_out in ((1, 1), (1, 0), (0, 3), (2, 2), (13, 13), (13, 5), (31, 31)):
            n = 100_003
            x = rand_input(dt, n, 99)
            big_in = torch.zeros(n + 40, dtype=STORE_T[dt], device="cuda")
            big_out = torch.zeros(n + 40, dtype=STORE_T[dt], device="cuda")
            xin = big_in[off_in:off_in + n]
            xin.copy_(to_dev(x, dt))
            yout = big_out[off_out:off_out + n]
            for op in ("add", "min"):
                sc.scan_device(xin, op=op, out=yout)
                torch.cuda.synchronize()
                compare_scan(from_dev(yout, dt), x, dt, op, True,
                             f"misaligned scan_device {dt} {op} in+{off_in} out+{off_out}")
            assert not big_out[:off_out].any() and not big_out[off_out + n:].any()


def test_device_repeated_calls_reuse_scratch():
    rng = np.random.default_rng(7)
    nmax = 3_000_000
    scratch = torch.empty(sc.scan_device_scratch_bytes(nmax, "i32"), dtype=torch.uint8,
                          device="cuda")
    scratch.fill_(0xAB)                     # no initialization is required of the caller
    for it in range(12):
        n = int(rng.integers(1, nmax))
        x = workloads.uniform_ints(n, 0, 15, 300 + it)
        out = sc.scan_device(to_dev(x, "i32"), op="add", scratch=scratch)
        torch.cuda.synchronize()
        compare_scan(from_dev(out, "i32"), x, "i32", "add", True, f"repeat {it} n={n}")


def test_device_two_streams():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    n = 2_000_000
    xa = workloads.uniform_ints(n, 0, 15, 41)
    xb = workloads.uniform_ints(n, 0, 15, 42)
    da, db = to_dev(xa, "i32"), to_dev(xb, "i32")
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        oa = sc.scan_device(da, op="add")
    with torch.cuda.stream(s2):
        ob = sc.scan_device(db, op="add")
    torch.cuda.synchronize()
    compare_scan(from_dev(oa, "i32"), xa, "i32", "add", True, "stream 1")
    compare_scan(from_dev(ob, "i32"), xb, "i32", "add", True, "stream 2")


def test_device_signed_zero_and_inf():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 2.0, -2.0], np.float32)
    x = vals[np.random.default_rng(6).integers(0, len(vals), size=200_000)]
    for op in ("min", "max"):
        out = sc.scan_device(to_dev(x, "f32"), op=op)
        compare_scan(from_dev(out, "f32"), x, "f32", op, True, f"scan_device signed zeros {op}")


# ---------------------------------------------------------------------------
# select
# ---------------------------------------------------------------------------

SEL_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 8191, 8192, 8193,
             20_000, 1_000_003]
SENTINEL_BYTE = 0x5A
# torch dtypes that carry elements of each width bit for bit (16 bytes: complex128)
SEL_NP = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64, 16: np.complex128}
SEL_EB = [1, 2, 4, 8, 16]


def run_select(x, flags, eb, label):
    """x: numpy array of n elements of eb bytes (any dtype of that width).
    Compares bytes with the oracle and checks that nothing past the count was
    written."""
    n = x.shape[0]
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(n, eb)
    xd = torch.from_numpy(xb.reshape(-1).view(SEL_NP[eb]).copy()).cuda()
    fd = torch.from_numpy(flags.copy()).cuda()
    out = torch.from_numpy(np.full(n * eb, SENTINEL_BYTE, np.uint8).view(SEL_NP[eb])).cuda()
    out, num = sc.select_compact(xd, fd, out=out)
    torch.cuda.synchronize()
    k = int(num.item())
    ora, ko = oracle.select(xb.reshape(-1).view(np.dtype((np.void, eb))), flags)
    assert k == ko, f"{label}: count {k} != {ko}"
    got = out.cpu().numpy().view(np.uint8).reshape(n, eb)
    want = np.ascontiguousarray(ora).view(np.uint8).reshape(n, eb)
    check_exact(got[:k].reshape(-1), want[:k].reshape(-1), label)
    assert (got[k:] == SENTINEL_BYTE).all(), f"{label}: tail written"
    return k


def sel_payload(n, eb, seed):
    """n elements of eb random bytes each (uint8 matrix viewed as one row per element)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n, eb), dtype=np.uint8).reshape(-1).view(
        np.dtype((np.void, eb)))


@pytest.mark.parametrize("eb", SEL_EB)
@pytest.mark.parametrize("p", [0.0, 0.01, 0.5, 0.99, 1.0])
def test_select_sizes(eb, p):
    for i, n in enumerate(SEL_SIZES):
        x = sel_payload(n, eb, 3000 + i)
        flags = workloads.bernoulli_flags(n, p, 4000 + i)
        run_select(x, flags, eb, f"select eb={eb} p={p} n={n}")


@pytest.mark.parametrize("eb", [1, 2, 8, 16])
def test_select_misaligned_views_all_widths(eb):
    # element offsets move payload, flags and output off their vector
    # alignment (4, 8 or 16 bytes), with equal and unequal phases
    n = 30_011
    xb = np.ascontiguousarray(sel_payload(n, eb, 11)).view(np.uint8).reshape(n, eb)
    flags = workloads.bernoulli_flags(n, 0.5, 12)
    ora, ko = oracle.select(xb.reshape(-1).view(np.dtype((np.void, eb))), flags)
    want = np.ascontiguousarray(ora).view(np.uint8).reshape(n, eb)
    dt = SEL_NP[eb]
    for off_in, off_f, off_out in ((1, 1, 1), (1, 0, 3), (0, 3, 2), (3, 2, 0), (2, 5, 1),
                                    (17, 17, 17), (17, 3, 5), (31, 30, 31), (9, 40, 2)):
        big_in = torch.zeros(n + 48, dtype=torch.from_numpy(np.zeros(1, dt)).dtype, device="cuda")
        big_f = torch.zeros(n + 48, dtype=torch.uint8, device="cuda")
        fill = np.full((n + 48) * eb, 7, np.uint8).view(dt)
        big_out = torch.from_numpy(fill).cuda()
        big_in[off_in:off_in + n].copy_(torch.from_numpy(xb.reshape(-1).view(dt).copy()).cuda())
        big_f[off_f:off_f + n].copy_(torch.from_numpy(flags).cuda())
        _, num = sc.select_compact(big_in[off_in:off_in + n], big_f[off_f:off_f + n],
                                   out=big_out[off_out:off_out + n])
        k = int(num.item())
        assert k == ko
        got = big_out.cpu().numpy().view(np.uint8).reshape(n + 48, eb)
        label = f"select eb={eb} offsets {off_in},{off_f},{off_out}"
        check_exact(got[off_out:off_out + k].reshape(-1), want[:k].reshape(-1), label)
        assert (got[:off_out] == 7).all() and (got[off_out + k:] == 7).all(), label


@pytest.mark.parametrize("p", workloads.SELECT_P)
def test_select_workload5_full(p):
    payload, flags = workloads.sel_inputs(workloads.FULL["sel"], p)
    label = f"select f32 n={payload.size} p={p}"
    note(label)
    k = run_select(payload, flags, 4, label)
    note(f"  kept {k}")


def test_select_nonbinary_flags_and_nan_payloads():
    n = 50_000
    rng = np.random.default_rng(8)
    flags = rng.integers(0, 256, size=n, dtype=np.uint8)
    flags[rng.random(n) < 0.5] = 0
    x = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    x[::7] = 0x7fc00001                      # NaN with a payload
    run_select(x, flags, 4, "select nonbinary flags")


def test_select_misaligned_views():
    n = 100_003
    rng = np.random.default_rng(9)
    x = rng.integers(0, 1 << 31, size=n, dtype=np.int64).astype(np.int32)
    flags = workloads.bernoulli_flags(n, 0.5, 10)
    ora, ko = oracle.select(x, flags)
    for off_in, off_f, off_out in ((1, 1, 1), (1, 0, 3), (0, 3, 2), (3, 2, 0), (2, 5, 1),
                                    (17, 17, 17), (17, 3, 5), (31, 30, 31), (9, 40, 2)):
        big_in = torch.zeros(n + 48, dtype=torch.int32, device="cuda")
        big_f = torch.zeros(n + 48, dtype=torch.uint8, device="cuda")
        big_out = torch.full((n + 48,), 7, dtype=torch.int32, device="cuda")
        xin = big_in[off_in:off_in + n]
        xin.copy_(torch.from_numpy(x).cuda())
        fin = big_f[off_f:off_f + n]
        fin.copy_(torch.from_numpy(flags).cuda())
        yout = big_out[off_out:off_out + n]
        _, num = sc.select_compact(xin, fin, out=yout)
        k = int(num.item())
        assert k == ko
        got = big_out.cpu().numpy()
        check_exact(got[off_out:off_out + k], ora[:k], f"select offsets {off_in},{off_f},{off_out}")
        assert (got[:off_out] == 7).all() and (got[off_out + k:] == 7).all()


def test_select_empty():
    x = torch.zeros(0, dtype=torch.float32, device="cuda")
    f = torch.zeros(0, dtype=torch.uint8, device="cuda")
    num = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    sc.select_compact(x, f, num_out=num)
    assert int(num.item()) == 0


# ---------------------------------------------------------------------------
# look-back recovery: a test-only build whose look-back never waits, so every
# predecessor descriptor that is not yet published is recomputed from the
# input by the waiting tile.  Results must be identical.
# ---------------------------------------------------------------------------

def _ptr(t):
    return t.data_ptr()


def test_lookback_recovery_build_device_scan():
    from stream_compaction_amd import build as b
    L = sc.load(b.FALLBACK_LIB_PATH)
    stream = torch.cuda.current_stream().cuda_stream
    for i, (dt, op, n) in enumerate([("i32", "add", 3_000_001), ("f32", "min", 1_000_003),
                                     ("i64", "max", 700_001), ("u64", "add", 500_000),
                                     ("f64", "add", 400_003), ("u32", "max", 2_000_000)]):
        x = rand_input(dt, n, 5000 + i)
        xd = to_dev(x, dt)
        yd = torch.empty_like(xd)
        code = sc.DTYPE_CODES[dt]
        need = L.scan_device_scratch_bytes(n, code)
        scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
        sc.check(L.scan_device(_ptr(xd), _ptr(yd), n, code, sc.OP_CODES[op], _ptr(scratch), need,
                               stream))
        torch.cuda.synchronize()
        compare_scan(from_dev(yd, dt), x, dt, op, True, f"recovery build scan_device {dt} {op}")


def test_lookback_recovery_build_select():
    from stream_compaction_amd import build as b
    L = sc.load(b.FALLBACK_LIB_PATH)
    stream = torch.cuda.current_stream().cuda_stream
    for eb, n, p in ((4, 2_000_003, 0.5), (8, 1_000_001, 0.3)):
        rng = np.random.default_rng(eb)
        x = rng.integers(0, 1 << 62, size=n, dtype=np.int64)
        x = x.astype(np.uint32) if eb == 4 else x.astype(np.uint64)
        flags = workloads.bernoulli_flags(n, p, 60 + eb)
        xd = torch.from_numpy(x.view(np.int32 if eb == 4 else np.int64).copy()).cuda()
        fd = torch.from_numpy(flags).cuda()
        out = torch.zeros_like(xd)
        num = torch.zeros(1, dtype=torch.int32, device="cuda")
        need = L.select_compact_scratch_bytes(n)
        scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
        sc.check(L.select_compact(_ptr(xd), _ptr(fd), _ptr(out), _ptr(num), n, eb, _ptr(scratch),
                                  need, stream))
        k = int(num.item())
        ora, ko = oracle.select(x, flags)
        assert k == ko
        check_exact(out.cpu().numpy().view(x.dtype)[:k], ora[:k], f"recovery build select eb={eb}")

"""GPU parity of the device-count (*_devn) entry points: each is captured
once into a HIP graph with a buffer capacity, then replayed for several live
counts written to the device between replays (with the program's own eager
work and synchronizations in between).  Every replay is checked against the
oracle on the live prefix, and outputs past it must be untouched.  Counts
beyond the capacity or below zero are clamped."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
from gpu_util import from_dev, rand_input, to_dev
from parity import FP_ABS, FP_REL, check_exact, check_fp_add

pytestmark = pytest.mark.gpu

CAP = 1_000_003
COUNTS = [CAP, 1, 0, 77_777, CAP - 37, 5, CAP + 500, -3, 300_001]
SENT = 0x5A5A5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()


def live(c):
    return max(0, min(CAP, c))


def replay_each(capture, check, reset=None):
    """Capture `capture()` once; for every count, reset the outputs (eagerly),
    set the count, replay, check."""
    n_live = torch.full((1,), CAP, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture(n_live)                          # eager warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture(n_live)
    for c in COUNTS:
        if reset is not None:
            reset()
        n_live.fill_(c)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(live(c), c)


@pytest.mark.parametrize("dt,op,incl", [("i32", "add", False), ("f32", "max", False),
                                        ("i64", "min", True), ("f64", "add", True)])
def test_scan_device_devn(dt, op, incl):
    x = rand_input(dt, CAP, 21)
    xd = to_dev(x, dt)
    out = to_dev(np.full(CAP, SENT, np.uint32).astype(np.uint64).view(np.int64).astype(oracle.STORAGE[dt])
                 if dt in ("i64", "f64") else np.full(CAP, SENT, np.uint32).view(oracle.STORAGE[dt]),
                 dt)
    sent = from_dev(out, dt).copy()
    sent_dev = out.clone()
    scratch = torch.empty(sc.scan_device_scratch_bytes(CAP, dt), dtype=torch.uint8, device="cuda")
    fn = sc.scan_device_inclusive if incl else sc.scan_device

    def capture(n_live):
        fn(xd, op, out=out, scratch=scratch, n_live=n_live)

    def check(n, c):
        got = from_dev(out, dt)
        label = f"{fn.__name__}_devn {dt} {op} count {c}"
        if n:
            if op == "add" and dt in oracle.FLOATS:
                o, ref, ab = oracle.scan(x[:n], dt, op, exclusive=not incl, want_ref=True)
                check_fp_add(got[:n], o, ref, ab, dt, label)
            else:
                check_exact(got[:n], oracle.scan(x[:n], dt, op, exclusive=not incl), label)
        if n < CAP:
            check_exact(got[n:], sent[n:], label + " tail")
    replay_each(capture, check, reset=lambda: out.copy_(sent_dev))


@pytest.mark.parametrize("dt,op", [("i32", "add"), ("f32", "min"), ("i64", "max"),
                                   ("f32", "add")])
def test_reduce_devn(dt, op):
    x = rand_input(dt, CAP, 22)
    xd = to_dev(x, dt)
    out = torch.empty(1, dtype=xd.dtype, device="cuda")
    scratch = torch.empty(sc.reduce_device_scratch_bytes(CAP, dt), dtype=torch.uint8,
                          device="cuda")

    def capture(n_live):
        sc.reduce_device(xd, op, out=out, scratch=scratch, n_live=n_live)

    def check(n, c):
        got = from_dev(out, dt)
        label = f"reduce_device_devn {dt} {op} count {c}"
        if op == "add" and dt in oracle.FLOATS:
            o, ref, ab = oracle.reduce(x[:n], dt, op, want_ref=True)
            assert abs(float(got[0]) - ref) <= FP_REL * ab + FP_ABS, label
        else:
            check_exact(got, oracle.reduce(x[:n], dt, op), label)
    replay_each(capture, check)


def test_select_devn():
    rng = np.random.default_rng(23)
    x = rng.integers(0, 1 << 31, size=CAP, dtype=np.int64).astype(np.int32)
    f = (rng.random(CAP) < 0.4).astype(np.uint8)
    xd, fd = torch.from_numpy(x).cuda(), torch.from_numpy(f).cuda()
    out = torch.full((CAP,), 7, dtype=torch.int32, device="cuda")
    num = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(sc.select_compact_scratch_bytes(CAP), dtype=torch.uint8, device="cuda")

    def capture(n_live):
        sc.select_compact(xd, fd, out=out, num_out=num, scratch=scratch, n_live=n_live)

    def check(n, c):
        o, k = oracle.select(x[:n], f[:n])
        assert int(num.item()) == k, (c, k)
        got = out.cpu().numpy()
        check_exact(got[:k], o[:k], f"select_devn count {c}")
    replay_each(capture, check)


@pytest.mark.parametrize("eb,tdt", [(1, torch.uint8), (2, torch.int16), (16, torch.complex128)])
def test_select_devn_widths(eb, tdt):
    # elements of 1, 2 and 16 bytes; compared byte for byte, tail untouched
    rng = np.random.default_rng(25 + eb)
    xb = rng.integers(0, 256, size=(CAP, eb), dtype=np.uint8)
    f = (rng.random(CAP) < 0.4).astype(np.uint8)
    npdt = {1: np.uint8, 2: np.int16, 16: np.complex128}[eb]
    xd = torch.from_numpy(xb.reshape(-1).view(npdt).copy()).cuda()
    fd = torch.from_numpy(f).cuda()
    out = torch.from_numpy(np.full(CAP * eb, 7, np.uint8).view(npdt)).cuda()
    assert xd.dtype == tdt
    num = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(sc.select_compact_scratch_bytes(CAP), dtype=torch.uint8, device="cuda")
    xv = xb.reshape(-1).view(np.dtype((np.void, eb)))

    def capture(n_live):
        sc.select_compact(xd, fd, out=out, num_out=num, scratch=scratch, n_live=n_live)

    def check(n, c):
        o, k = oracle.select(xv[:n], f[:n])
        assert int(num.item()) == k, (c, k)
        got = out.cpu().numpy().view(np.uint8).reshape(CAP, eb)
        want = np.ascontiguousarray(o).view(np.uint8).reshape(n, eb)
        check_exact(got[:k].reshape(-1), want[:k].reshape(-1), f"select_devn eb={eb} count {c}")
    replay_each(capture, check)


def test_reduce_by_key_devn():
    rng = np.random.default_rng(24)
    keys = np.repeat(rng.integers(0, 5, size=CAP), rng.geometric(0.2, size=CAP))[:CAP]
    keys = keys.astype(np.int32)
    vals = rng.integers(-100, 100, size=CAP).astype(np.int32)
    kd, vd = torch.from_numpy(keys).cuda(), torch.from_numpy(vals).cuda()
    ko = torch.full((CAP,), 7, dtype=torch.int32, device="cuda")
    vo = torch.full((CAP,), 7, dtype=torch.int32, device="cuda")
    nr = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(sc.reduce_by_key_scratch_bytes(CAP), dtype=torch.uint8, device="cuda")

    def capture(n_live):
        sc.reduce_by_key(kd, vd, ko, vo, nr, scratch, n_live=n_live)

    def check(n, c):
        oko, ovo, r = oracle.reduce_by_key(keys[:n], vals[:n], "i32", "i32")
        assert int(nr.item()) == r, (c, r)
        check_exact(ko.cpu().numpy()[:r], oko[:r], f"reduce_by_key_devn keys count {c}")
        check_exact(vo.cpu().numpy()[:r], ovo[:r], f"reduce_by_key_devn values count {c}")
    replay_each(capture, check)


def test_radix_sort_devn():
    rng = np.random.default_rng(25)
    keys0 = rng.integers(0, 1 << 32, size=CAP, dtype=np.uint64).astype(np.uint32)
    kd = torch.from_numpy(keys0.view(np.int32).copy()).cuda()
    vd = torch.arange(CAP, dtype=torch.int32, device="cuda")
    tk, tv = torch.empty_like(kd), torch.empty_like(vd)
    k_init, v_init = kd.clone(), vd.clone()
    scratch = torch.empty(sc.radix_sort_scratch_bytes(CAP, "u32"), dtype=torch.uint8,
                          device="cuda")

    def capture(n_live):
        sc.radix_sort(kd, vd, tk, tv, 32, scratch, key_dtype="u32", value_dtype="i32",
                      n_live=n_live)

    def check(n, c):
        got_k = kd.cpu().numpy().view(np.uint32)
        got_v = vd.cpu().numpy()
        ok, ov = oracle.sort(keys0[:n], "u32", np.arange(n, dtype=np.int32))
        check_exact(got_k[:n], ok, f"radix_sort_devn keys count {c}")
        check_exact(got_v[:n], ov, f"radix_sort_devn values count {c}")
        check_exact(got_k[n:], keys0[n:], f"radix_sort_devn tail count {c}")
        kd.copy_(k_init)                         # the sort works in place: restore the input
        vd.copy_(v_init)
        torch.cuda.synchronize()
    replay_each(capture, check)

"""The allocation-free device scan (scan_device_noalloc, static per-GPU
scratch) against the existing entry point it varies (scan_device, caller
scratch), called through the C ABI: the same exclusive scans, bit for bit,
on two calls in a row with the second input smaller, for several dtypes and
ops, including the 2^28-element i32 workload, arrays at element offsets, and
the largest count the static scratch admits; each result is also checked
against the oracle.  Collected last, so that a failure here cannot hide the
other tests."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from gpu_util import from_dev, note, rand_input, to_dev
from parity import check_exact

pytestmark = pytest.mark.gpu


def noalloc(x, dt, op, out=None):
    """One scan_device_noalloc call through the C ABI into a sentinel-filled
    output (a new tensor, or the given view)."""
    L = sc.lib()
    out = torch.full_like(x, -7) if out is None else out.fill_(-7)
    st = L.scan_device_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                               x.numel(), sc.DTYPE_CODES[dt], sc.OP_CODES[op],
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    sc.check(st)
    return out


def existing(x, dt, op, out=None):
    L = sc.lib()
    n = x.numel()
    out = torch.full_like(x, -7) if out is None else out.fill_(-7)
    need = L.scan_device_scratch_bytes(n, sc.DTYPE_CODES[dt])
    scratch = torch.empty(need, dtype=torch.uint8, device=x.device)
    sc.check(L.scan_device(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), n,
                           sc.DTYPE_CODES[dt], sc.OP_CODES[op], ctypes.c_void_p(scratch.data_ptr()),
                           need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return out


@pytest.mark.parametrize("dt,op", [("i32", "add"), ("u32", "max"), ("f32", "min"),
                                   ("i64", "add"), ("u64", "min"), ("f64", "max")])
def test_noalloc_matches_scan_device_two_calls(dt, op):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    for i, n in enumerate((3_000_017, 100_003)):       # the second call is smaller
        note(f"scan_device_noalloc {dt} {op} n={n}")
        x = rand_input(dt, n, 96_000 + i)
        xd = to_dev(x, dt)
        got = noalloc(xd, dt, op)
        want = existing(xd, dt, op)
        torch.cuda.synchronize()
        g = from_dev(got, dt)
        check_exact(g, from_dev(want, dt), f"noalloc vs scan_device {dt} {op} n={n}")
        check_exact(g, oracle.scan(x, dt, op, exclusive=True), f"noalloc vs oracle {dt} {op} n={n}")


def test_noalloc_full_workload_then_smaller():
    x = workloads.dev_i32()
    xd = to_dev(x, "i32")
    want_all = oracle.scan(x, "i32", "add", exclusive=True)
    for n in (x.size, workloads.FULL["dev_i32_odd"] - 1_000_000):
        note(f"scan_device_noalloc i32 add n={n}")
        got = noalloc(xd[:n], "i32", "add")
        ref = existing(xd[:n], "i32", "add")
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"noalloc vs scan_device n={n}"
        check_exact(got.cpu().numpy(), want_all[:n], f"noalloc vs oracle n={n}")


def test_noalloc_offset_views():
    # input and output at the same element offset, within and past the first
    # 16-byte vector: the window then starts on the 128-byte line of the first
    # element; then at different offsets (one element per vector); the second
    # and later calls are smaller than the first
    x = rand_input("i32", 3_000_017, 96_500)
    for off_in, off_out, n in ((3, 3, 3_000_017), (17, 17, 2_000_003), (5, 0, 1_000_001)):
        note(f"scan_device_noalloc i32 add n={n} offsets {off_in}/{off_out}")
        big_in = torch.zeros(n + 32, dtype=torch.int32, device="cuda")
        big_a = torch.zeros(n + 32, dtype=torch.int32, device="cuda")
        big_b = torch.zeros(n + 32, dtype=torch.int32, device="cuda")
        xd = big_in[off_in:off_in + n]
        xd.copy_(to_dev(x[:n], "i32"))
        got = noalloc(xd, "i32", "add", out=big_a[off_out:off_out + n])
        want = existing(xd, "i32", "add", out=big_b[off_out:off_out + n])
        torch.cuda.synchronize()
        label = f"offsets {off_in}/{off_out} n={n}"
        assert torch.equal(got, want), "noalloc vs scan_device " + label
        check_exact(got.cpu().numpy(), oracle.scan(x[:n], "i32", "add", exclusive=True),
                    "noalloc vs oracle " + label)
        assert not big_a[:off_out].any() and not big_a[off_out + n:].any(), \
            "noalloc wrote outside its output " + label


def test_noalloc_largest_count():
    # the largest count the static scratch admits, in its most-tiled form:
    # input and output at different phases, so one element per vector
    n = 65_535 * 7_168
    x = workloads.uniform_ints(n, 0, 15, 96_700)
    note(f"scan_device_noalloc i32 add n={n} offsets 1/0")
    big = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    xd = big[1:]
    xd.copy_(to_dev(x, "i32"))
    got = noalloc(xd, "i32", "add", out=torch.empty(n, dtype=torch.int32, device="cuda"))
    want = existing(xd, "i32", "add", out=torch.empty(n, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(got, want), "noalloc vs scan_device at the largest count"
    check_exact(got.cpu().numpy(), oracle.scan(x, "i32", "add", exclusive=True),
                "noalloc vs oracle at the largest count")
    del big, xd, got, want
    torch.cuda.empty_cache()


def test_noalloc_rejects_more_than_its_scratch_holds():
    L = sc.lib()
    n_max = 65_535 * 7_168        # tiles the 8 MiB static scratch holds descriptors for
    x = torch.zeros(8, dtype=torch.int32, device="cuda")
    # rejected on the host before the arrays are touched, so small buffers do
    for n in (n_max + 1, (1 << 31) - 1):
        st = L.scan_device_noalloc(ctypes.c_void_p(x.data_ptr()),
                                   ctypes.c_void_p(x.data_ptr() + 4096), n,
                                   sc.DTYPE_CODES["i32"], sc.OP_CODES["add"], None)
        assert st == 4, st      # SCAN_ESCRATCH
    with pytest.raises(ValueError):
        sc.check(4)

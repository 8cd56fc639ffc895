"""Soak of the decoupled look-back kernels: many calls in a row on one scratch
buffer, each compared with the oracle bit for bit, stopping at the first
mismatch.

A single-pass scan's result depends on tiles publishing and reading each
other's descriptors while they run, so a fault in that protocol (a torn or
stale descriptor, a store that lands late) shows up only now and then.  Each
test below draws at least 100 counts log-uniformly from [1, 2^26] (plus a few
full-size calls), runs them back to back with one scratch buffer that is never
cleared by the caller, and checks every output against the oracle.  Inputs are
slices of one seeded pool at random element offsets (up to 40, past a
128-byte line for 4-byte elements), and outputs alternate between the same
offset and offset 0, so every window phase, windows on lines, and both the
vector and the one-element-per-vector paths come up.  The
64-bit-descriptor path (i64 values, reduce-by-key's pairs) is covered too.
"""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from gpu_util import note, to_dev
from parity import check_exact

pytestmark = pytest.mark.gpu

ITERS = 100
NMAX = 1 << 26


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def draws(seed, iters=ITERS, nmax=NMAX):
    """(n, offset) pairs: n log-uniform in [1, nmax], offset in [0, 40)."""
    rng = np.random.default_rng(seed)
    ns = np.exp(rng.uniform(0, np.log(nmax), size=iters)).astype(np.int64)
    return [(int(max(1, n)), int(o)) for n, o in zip(ns, rng.integers(0, 40, size=iters))]


@pytest.mark.parametrize("dt,op", [("i32", "add"), ("i64", "min")])
def test_soak_scan_device(dt, op):
    pool_n = NMAX + 40
    pool = workloads.uniform_ints(pool_n, 0, 15, 90_001) if dt == "i32" else \
        np.random.default_rng(90_002).integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max,
                                               size=pool_n, dtype=np.int64, endpoint=True)
    pd = to_dev(pool, dt)
    out = torch.empty_like(pd)
    scratch = torch.empty(sc.scan_device_scratch_bytes(pool_n, dt), dtype=torch.uint8,
                          device="cuda").fill_(0xA5)
    for it, (n, off) in enumerate(draws(91_000 + len(dt))):
        if it % 20 == 0:
            note(f"soak scan_device {dt} {op}: call {it}, n={n}, offset {off}")
        # even calls: output at the input's offset (windows on lines), odd: at 0
        o = out[off:off + n] if it % 2 == 0 else out[:n]
        sc.scan_device(pd[off:off + n], op=op, out=o, scratch=scratch, dtype=dt)
        got = o.cpu().numpy()
        check_exact(got, oracle.scan(pool[off:off + n], dt, op, exclusive=True),
                    f"soak scan_device {dt} {op} call {it} n={n} offset {off}")
    del pd, out
    # full size, twice in a row on the same scratch
    if dt == "i32":
        x = workloads.dev_i32()
        n_full = (workloads.FULL["dev_i32"], workloads.FULL["dev_i32_odd"])
    else:
        x = workloads.dev_i64()
        n_full = (x.size, x.size - 3)
    xd = to_dev(x, dt)
    big = torch.empty(sc.scan_device_scratch_bytes(x.size, dt), dtype=torch.uint8, device="cuda")
    want = oracle.scan(x, dt, op, exclusive=True)
    for n in n_full:
        note(f"soak scan_device {dt} {op}: full size n={n}")
        got = sc.scan_device(xd[:n], op=op, scratch=big, dtype=dt).cpu().numpy()
        check_exact(got, want[:n], f"soak scan_device {dt} {op} full n={n}")


def test_soak_select():
    pool_n = NMAX + 40
    payload = np.random.default_rng(92_001).integers(0, 1 << 32, size=pool_n,
                                                     dtype=np.uint64).astype(np.uint32)
    level = np.random.default_rng(92_002).integers(0, 256, size=pool_n, dtype=np.uint8)
    pd = torch.from_numpy(payload.view(np.int32)).cuda()
    ld = torch.from_numpy(level).cuda()
    out = torch.empty_like(pd)
    num = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(sc.select_compact_scratch_bytes(pool_n), dtype=torch.uint8,
                          device="cuda").fill_(0x3C)
    thresholds = np.random.default_rng(92_003).integers(0, 257, size=ITERS)
    for it, (n, off) in enumerate(draws(93_000)):
        thr = int(thresholds[it])
        if it % 20 == 0:
            note(f"soak select: call {it}, n={n}, offset {off}, threshold {thr}")
        # even calls: flags a slice of a pool-sized array at the payload's offset
        # (so the payload window can start on its line) and output at that
        # offset too; odd calls: fresh flags and output at 0
        if it % 2 == 0:
            fd = (ld < thr).to(torch.uint8)[off:off + n]
            o = out[off:off + n]
        else:
            fd = (ld[off:off + n] < thr).to(torch.uint8)
            o = out[:n]
        sc.select_compact(pd[off:off + n], fd, out=o, num_out=num, scratch=scratch)
        k = int(num.item())
        fl = (level[off:off + n] < thr).astype(np.uint8)
        want, kw = oracle.select(payload[off:off + n], fl)
        assert k == kw, f"soak select call {it} n={n}: count {k} != {kw}"
        check_exact(o[:k].cpu().numpy().view(np.uint32), want[:k],
                    f"soak select call {it} n={n} offset {off}")
    del pd, ld, out
    p, f = workloads.sel_inputs(workloads.FULL["sel"], 0.5)
    xd, fd = torch.from_numpy(p).cuda(), torch.from_numpy(f).cuda()
    want, kw = oracle.select(p, f)
    big = torch.empty(sc.select_compact_scratch_bytes(p.size), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        note(f"soak select: full size, call {rep}")
        o, nm = sc.select_compact(xd, fd, scratch=big)
        k = int(nm.item())
        assert k == kw
        check_exact(o[:k].cpu().numpy().view(np.uint32), want[:k].view(np.uint32),
                    f"soak select full size call {rep}")


def test_soak_reduce_by_key():
    pool_n = NMAX + 40
    rng = np.random.default_rng(94_001)
    lengths = rng.geometric(1.0 / 8, size=pool_n // 4)
    keys = np.repeat(rng.integers(0, 1 << 20, size=lengths.size), lengths)[:pool_n].astype(np.int32)
    values = rng.integers(-(1 << 20), 1 << 20, size=pool_n).astype(np.int32)
    kd, vd = torch.from_numpy(keys).cuda(), torch.from_numpy(values).cuda()
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    nr = torch.empty(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(sc.reduce_by_key_scratch_bytes(pool_n), dtype=torch.uint8,
                          device="cuda").fill_(0x77)
    for it, (n, off) in enumerate(draws(95_000)):
        if it % 20 == 0:
            note(f"soak reduce_by_key: call {it}, n={n}, offset {off}")
        sc.reduce_by_key(kd[off:off + n], vd[off:off + n], ko, vo, nr, scratch)
        r = int(nr.item())
        oko, ovo, orr = oracle.reduce_by_key(keys[off:off + n], values[off:off + n], "i32", "i32")
        assert r == orr, f"soak reduce_by_key call {it} n={n}: {r} runs, oracle {orr}"
        check_exact(ko[:r].cpu().numpy(), oko[:r], f"soak reduce_by_key call {it} keys")
        check_exact(vo[:r].cpu().numpy(), ovo[:r], f"soak reduce_by_key call {it} values")
    del kd, vd, ko, vo
    n = workloads.FULL["rbk"]
    k2, v2 = workloads.rbk_inputs(n)
    v2i = (v2 * 1000).astype(np.int32)        # integer sums: exact comparison
    kd, vd = torch.from_numpy(k2).cuda(), torch.from_numpy(v2i).cuda()
    oko, ovo, orr = oracle.reduce_by_key(k2, v2i, "i32", "i32")
    big = torch.empty(sc.reduce_by_key_scratch_bytes(n), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        note(f"soak reduce_by_key: full size, call {rep}")
        ko, vo, nr = sc.reduce_by_key(kd, vd, scratch=big)
        r = int(nr.item())
        assert r == orr
        check_exact(ko[:r].cpu().numpy(), oko[:r], "soak reduce_by_key full keys")
        check_exact(vo[:r].cpu().numpy(), ovo[:r], "soak reduce_by_key full values")

"""GPU parity of the radix sort (through the C ABI) against the oracle's
stable sort order: keys bit for bit, and values (each key's original index)
bit for bit, which checks stability exactly."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from gpu_util import from_dev, note, to_dev
from parity import check_exact, check_stable_by_image

pytestmark = pytest.mark.gpu

KEY_DT = ["u32", "i32", "f32", "u64", "i64", "f64"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()


def sort_keys(dt, n, seed, kind):
    """Keys of dtype `dt`: arbitrary bit patterns ("bits", NaNs included for
    floats), few distinct values ("dups"), or float specials ("specials")."""
    rng = np.random.default_rng(seed)
    st = oracle.STORAGE[dt]
    if kind == "bits":
        raw = rng.integers(0, 256, size=n * np.dtype(st).itemsize, dtype=np.uint8)
        return raw.view(st).copy()
    if kind == "dups":
        vals = rng.integers(0, 1 << 62, size=5, dtype=np.int64)
        return vals.astype(np.uint64).view(np.int64).astype(st)[rng.integers(0, 5, size=n)] \
            if dt[0] != "f" else rng.choice(np.array([1.5, -2.0, 0.0, 7.0, -0.0], st), size=n)
    alphabet = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 2.5, -1e30], st)
    return alphabet[rng.integers(0, alphabet.size, size=n)]


def run_sort(keys, dt, values=None, vdt=None, end_bit=None, label=""):
    kd = to_dev(keys, dt)
    vd = to_dev(values, vdt) if values is not None else None
    sc.radix_sort(kd, vd, end_bit=end_bit, key_dtype=dt, value_dtype=vdt)
    torch.cuda.synchronize()
    ok, ov = oracle.sort(keys, dt, values, end_bit=end_bit)
    check_exact(from_dev(kd, dt), ok, label + " keys")
    if values is not None:
        check_exact(from_dev(vd, vdt), ov, label + " values")


SIZES = [1, 2, 3, 64, 1000, 4095, 4096, 4097, 8191, 8192, 8193, 100_003, 1_000_003]


@pytest.mark.parametrize("dt", KEY_DT)
def test_sort_sizes_key_value(dt):
    for i, n in enumerate(SIZES):
        keys = sort_keys(dt, n, 10_000 + i, "bits")
        run_sort(keys, dt, np.arange(n, dtype=np.int32), "i32", label=f"sort {dt} n={n}")


EDGE_SIZES = [8191, 8192, 8193, 16383, 16384, 16385, 32769, 40_961]


@pytest.mark.parametrize("dt,vdt", [("u32", "i64"), ("f32", "f64"), ("u64", "i32"),
                                    ("i64", "i64"), ("f64", "u64"), ("u32", "i32"),
                                    ("i32", "f32"), ("f32", "u32")])
def test_sort_tile_edges_wide_values(dt, vdt):
    # 32-bit keys with 8-byte values and 64-bit keys with values run on tiles
    # of 8,192 keys (16 waves of 8), 32-bit keys with 4-byte values on 16,384
    # (16 waves of 16): counts on both sides of one and two tiles of either
    # size, and ragged multiples
    for i, n in enumerate(EDGE_SIZES):
        keys = sort_keys(dt, n, 16_000 + i, "bits")
        vals = np.arange(n, dtype=np.int64).astype(oracle.STORAGE[vdt]) if vdt in ("i32", "i64") \
            else np.random.default_rng(16_100 + i).integers(
                0, 256, size=n * np.dtype(oracle.STORAGE[vdt]).itemsize, dtype=np.uint8) \
            .view(oracle.STORAGE[vdt]).copy()
        run_sort(keys, dt, vals, vdt, label=f"sort {dt} + {vdt} n={n}")


@pytest.mark.parametrize("dt,kind", [(d, "dups") for d in KEY_DT] +
                         [("f32", "specials"), ("f64", "specials")])
def test_sort_duplicates_and_specials_stable(dt, kind):
    for n in (5000, 300_001):
        keys = sort_keys(dt, n, 11_000 + n, kind)
        run_sort(keys, dt, np.arange(n, dtype=np.int64), "i64", label=f"sort {dt} {kind} n={n}")


@pytest.mark.parametrize("dt", KEY_DT)
def test_sort_keys_only(dt):
    keys = sort_keys(dt, 777_777, 12_000, "bits")
    run_sort(keys, dt, label=f"sort keys only {dt}")


@pytest.mark.parametrize("vdt", ["u32", "f32", "u64", "f64"])
def test_sort_value_types(vdt):
    n = 200_003
    keys = sort_keys("u32", n, 13_000, "dups")
    rng = np.random.default_rng(13_001)
    raw = rng.integers(0, 256, size=n * np.dtype(oracle.STORAGE[vdt]).itemsize, dtype=np.uint8)
    values = raw.view(oracle.STORAGE[vdt]).copy()            # arbitrary bits, NaNs included
    run_sort(keys, "u32", values, vdt, label=f"sort values {vdt}")


@pytest.mark.parametrize("dt,end_bit", [("u32", 8), ("u32", 16), ("u32", 24), ("i32", 16),
                                        ("f32", 24), ("u64", 40), ("i64", 8), ("u64", 56)])
def test_sort_end_bit(dt, end_bit):
    n = 300_007
    keys = sort_keys(dt, n, 14_000 + end_bit, "bits")
    run_sort(keys, dt, np.arange(n, dtype=np.int32), "i32", end_bit=end_bit,
             label=f"sort {dt} end_bit={end_bit}")


def test_sort_page_example():
    keys = np.array([3, 1, 4, 1, 5, 9, 2, 6], np.int32)
    run_sort(keys, "i32", np.arange(8, dtype=np.int32), "i32", label="page example")


def test_sort_empty_and_single():
    for n in (0, 1):
        k = torch.full((n,), 5, dtype=torch.int32, device="cuda")
        sc.radix_sort(k)
        assert k.tolist() == [5] * n


def test_sort_full_u32_key_value():
    n = workloads.FULL["sort"]
    keys = workloads.sort_keys_u32(n)
    label = f"sort u32 + i32 index n={n}"
    note(label)
    run_sort(keys, "u32", np.arange(n, dtype=np.int32), "i32", label=label)


def test_lookback_recovery_build_sort():
    from stream_compaction_amd import build as b
    L = sc.load(b.FALLBACK_LIB_PATH)
    n = 100_003
    keys = sort_keys("u32", n, 15_000, "bits")
    kd, tk = to_dev(keys, "u32"), torch.empty(n, dtype=torch.int32, device="cuda")
    vd = torch.arange(n, dtype=torch.int32, device="cuda")
    tv = torch.empty_like(vd)
    need = L.radix_sort_scratch_bytes(n, sc.DTYPE_CODES["u32"])
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    sc.check(L.radix_sort(kd.data_ptr(), tk.data_ptr(), vd.data_ptr(), tv.data_ptr(), n,
                          sc.DTYPE_CODES["u32"], sc.DTYPE_CODES["i32"], 32, scratch.data_ptr(),
                          need, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ok, ov = oracle.sort(keys, "u32", np.arange(n, dtype=np.int32))
    check_exact(from_dev(kd, "u32"), ok, "fallback build keys")
    check_exact(vd.cpu().numpy(), ov, "fallback build values")


def test_sort_keys_only_past_4gib():
    """u64 keys only, n = 2^29 + 7 (4 GiB): the scatter's 64-bit-address stores
    (below 4 GiB it uses 32-bit buffer offsets).  Keys come from 997 distinct
    bit patterns; the output must be the input's multiset in the oracle's image
    order (non-decreasing images; equal keys are indistinguishable, so this is
    the stable order)."""
    g = torch.Generator(device="cuda").manual_seed(20_000)
    n = (1 << 29) + 7
    note(f"sort u64 keys only n={n}")
    alphabet = torch.randint(-(1 << 63), (1 << 63) - 1, (997,), generator=g, device="cuda",
                             dtype=torch.int64)
    sym = torch.randint(0, 997, (n,), generator=g, device="cuda")
    keys = alphabet[sym]
    counts_in = torch.bincount(sym, minlength=997).cpu().numpy()
    del sym
    sc.radix_sort(keys, key_dtype="u64")
    torch.cuda.synchronize()
    out = keys.cpu().numpy().view(np.uint64)
    del keys
    note("  checking on the host")
    al = alphabet.cpu().numpy().view(np.uint64)
    img = oracle.sort_image(out, "u64")
    assert not (img[1:] < img[:-1]).any(), "u64 keys past 4 GiB: out of order"
    del img
    order = np.argsort(al)
    pos = np.searchsorted(al[order], out)
    assert np.array_equal(al[order][pos], out), "u64 keys past 4 GiB: a key not in the input"
    assert np.array_equal(np.bincount(order[pos], minlength=997), counts_in), \
        "u64 keys past 4 GiB: multiset changed"


@pytest.mark.parametrize("kdt", ["u32", "u64"])
def test_sort_key_value_past_4gib(kdt):
    """u32 or u64 keys with i64 values (each key's original index), n = 2^29 + 3:
    the values array passes 4 GiB, so the scatter takes its 64-bit-address
    stores.  Keys come from 1,009 distinct bit patterns (long runs of equal
    keys, so stability matters); checked against the oracle's order."""
    g = torch.Generator(device="cuda").manual_seed(20_001 if kdt == "u32" else 20_002)
    n = (1 << 29) + 3
    note(f"sort {kdt} keys + i64 values n={n}")
    tdt = torch.int32 if kdt == "u32" else torch.int64
    lo, hi = (-(1 << 31), (1 << 31) - 1) if kdt == "u32" else (-(1 << 63), (1 << 63) - 1)
    alpha = torch.randint(lo, hi, (1009,), generator=g, device="cuda", dtype=tdt)
    keys = alpha[torch.randint(0, 1009, (n,), generator=g, device="cuda")]
    keys_in = keys.cpu().numpy().view(np.uint32 if kdt == "u32" else np.uint64)
    vals = torch.arange(n, dtype=torch.int64, device="cuda")
    sc.radix_sort(keys, vals, key_dtype=kdt, value_dtype="i64")
    torch.cuda.synchronize()
    keys_out = keys.cpu().numpy().view(keys_in.dtype)
    idx = vals.cpu().numpy()
    del keys, vals
    note("  checking on the host")
    check_stable_by_image(keys_in, keys_out, idx, kdt, f"{kdt} keys + i64 values past 4 GiB")

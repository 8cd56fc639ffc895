"""Every entry point at the largest count the C ABI accepts, n = 2^31 - 1,
and a row scan whose rows together pass 2^31 elements.

At this size the checks are closed forms of the inputs, evaluated with torch
on the GPU (no call into this library), chunk by chunk:
  - x[i] = (i mod 7) - 3 sums to zero over every period of seven, so its
    exclusive prefix at i is f(i mod 7) with f(r) = r(r-1)/2 - 3r, and its
    total is f(n mod 7);
  - a row of alternating +1, -1 has the exclusive prefix i mod 2, exact in
    any order of float32 additions;
  - keeping i where i mod 3 = 0 gives out[j] = 3j and ceil(n/3) elements;
  - keys i div 8 with unit values give runs r with sum 8 (the last one
    n - 8(R-1)), R = ceil(n/8);
  - 2^31 - 1 is prime, so keys (i * 48271) mod n are a permutation of
    [0, n): sorted they are 0..n-1, and the value carried from index i sits at
    key (i * 48271) mod n, i.e. position j holds j * 48271^-1 mod n.
"""
import pytest
import torch

import stream_compaction_amd as sc
from gpu_util import note

pytestmark = pytest.mark.gpu

N = (1 << 31) - 1          # the largest element count the C ABI accepts
CH = 1 << 28               # chunk of the closed-form checks


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def chunks(n):
    for a in range(0, n, CH):
        yield a, min(n, a + CH)


def mod7_input(n):
    x = torch.arange(n, dtype=torch.int32, device="cuda")
    x.remainder_(7).sub_(3)
    return x


def mod7_prefix(r):
    return r * (r - 1) // 2 - 3 * r


def test_scan_device_max_count():
    note(f"scan_device i32 add n={N}")
    x = mod7_input(N)
    out = sc.scan_device(x, op="add")
    torch.cuda.synchronize()
    for a, b in chunks(N):
        r = torch.arange(a, b, dtype=torch.int64, device="cuda").remainder_(7)
        assert torch.equal(out[a:b].to(torch.int64), mod7_prefix(r)), f"elements [{a}, {b})"


def test_reduce_device_max_count():
    note(f"reduce_device i32 add n={N}")
    x = mod7_input(N)
    got = int(sc.reduce_device(x, op="add").item())
    assert got == mod7_prefix(N % 7)


def test_select_max_count():
    note(f"select_compact 4-byte n={N}")
    x = torch.arange(N, dtype=torch.int32, device="cuda")
    flags = (x % 3 == 0).to(torch.uint8)
    out, num = sc.select_compact(x, flags)
    k = int(num.item())
    assert k == (N + 2) // 3
    del flags
    for a, b in chunks(k):
        want = torch.arange(a, b, dtype=torch.int64, device="cuda").mul_(3)
        assert torch.equal(out[a:b].to(torch.int64), want), f"outputs [{a}, {b})"


def test_scan_rows_one_max_row():
    note(f"scan_rows bf16 [1, {N}] exclusive add")
    i = torch.arange(N, dtype=torch.int32, device="cuda")
    x = (1 - 2 * (i % 2)).to(torch.bfloat16).view(1, N)
    del i
    out = sc.scan_rows(x, op="add", exclusive=True)
    torch.cuda.synchronize()
    for a, b in chunks(N):
        want = (torch.arange(a, b, dtype=torch.int32, device="cuda") % 2).to(torch.bfloat16)
        assert torch.equal(out[0, a:b], want), f"elements [{a}, {b})"


def test_scan_rows_past_2_31_elements():
    # 65,537 rows of 32,771 elements: 2^31 + 2^16 + ... elements in all, so row
    # offsets pass 32 bits; rows of odd length start inside 16-byte vectors
    rows, n = 65_537, 32_771
    note(f"scan_rows bf16 [{rows}, {n}] exclusive add")
    i = torch.arange(n, dtype=torch.int32, device="cuda")
    row = (1 - 2 * (i % 2)).to(torch.bfloat16)
    x = row.expand(rows, n).contiguous()
    out = sc.scan_rows(x, op="add", exclusive=True)
    torch.cuda.synchronize()
    want = (i % 2).to(torch.bfloat16)
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        assert torch.equal(out[r0:r1], want.expand(r1 - r0, n)), f"rows [{r0}, {r1})"


def test_reduce_by_key_max_count():
    note(f"reduce_by_key i32/i32 n={N}")
    keys = torch.arange(N, dtype=torch.int32, device="cuda").div_(8, rounding_mode="floor")
    vals = torch.ones(N, dtype=torch.int32, device="cuda")
    ko, vo, nr = sc.reduce_by_key(keys, vals)
    runs = (N + 7) // 8
    assert int(nr.item()) == runs
    del keys, vals
    for a, b in chunks(runs):
        assert torch.equal(ko[a:b], torch.arange(a, b, dtype=torch.int32, device="cuda")), \
            f"keys [{a}, {b})"
        want = torch.full((b - a,), 8, dtype=torch.int32, device="cuda")
        if b == runs:
            want[-1] = N - 8 * (runs - 1)
        assert torch.equal(vo[a:b], want), f"sums [{a}, {b})"


def test_radix_sort_max_count_key_value():
    note(f"radix_sort u32 keys + i32 values n={N}")
    a_mul = 48271
    a_inv = pow(a_mul, N - 2, N)
    keys = torch.empty(N, dtype=torch.int32, device="cuda")
    for a, b in chunks(N):
        keys[a:b] = torch.arange(a, b, dtype=torch.int64, device="cuda").mul_(a_mul) \
            .remainder_(N).to(torch.int32)
    vals = torch.arange(N, dtype=torch.int32, device="cuda")
    sc.radix_sort(keys, vals, key_dtype="u32", value_dtype="i32")
    torch.cuda.synchronize()
    for a, b in chunks(N):
        j = torch.arange(a, b, dtype=torch.int64, device="cuda")
        assert torch.equal(keys[a:b].to(torch.int64), j), f"keys [{a}, {b})"
        assert torch.equal(vals[a:b].to(torch.int64), j.mul_(a_inv).remainder_(N)), \
            f"values [{a}, {b})"


@pytest.mark.parametrize("rows", [(1 << 26) + 1, N], ids=["2^26+1", "2^31-1"])
def test_scan_rows_many_one_element_rows(rows):
    # more rows than one dispatch can hold (its work-items are counted in 32
    # bits), so the rows go out in several launches.  With one element per row,
    # each row's inclusive prefix is its element and its exclusive prefix the
    # identity: here x[r] = (r mod 7) - 3 in bf16 (exact), identity 0 for add
    # and -inf for max.
    note(f"scan_rows bf16 [{rows}, 1] add/max")
    x = mod7_input(rows).to(torch.bfloat16).view(rows, 1)
    for op, excl in (("add", False), ("add", True), ("max", True)):
        out = sc.scan_rows(x, op=op, exclusive=excl)
        torch.cuda.synchronize()
        for a, b in chunks(rows):
            if not excl:
                want = x[a:b]
            else:
                want = torch.full((b - a, 1), 0.0 if op == "add" else float("-inf"),
                                  dtype=torch.bfloat16, device="cuda")
            assert torch.equal(out[a:b], want), f"{op} excl={excl} rows [{a}, {b})"
        del out


def test_scan_rows_many_three_element_rows():
    # rows [1, -1, r mod 5] (f32): exclusive [0, 1, 0], inclusive [1, 0, r mod 5],
    # over 2^26 + 1 rows (several launches; rows straddle 16-byte vectors)
    rows = (1 << 26) + 1
    note(f"scan_rows f32 [{rows}, 3] add")
    x = torch.empty((rows, 3), dtype=torch.float32, device="cuda")
    x[:, 0] = 1.0
    x[:, 1] = -1.0
    x[:, 2] = torch.arange(rows, dtype=torch.int32, device="cuda").remainder_(5).float()
    for excl in (False, True):
        out = sc.scan_rows(x, op="add", exclusive=excl)
        torch.cuda.synchronize()
        for a, b in chunks(rows):
            if excl:
                want = torch.tensor([0.0, 1.0, 0.0], device="cuda").expand(b - a, 3)
            else:
                want = torch.stack([torch.ones(b - a, device="cuda"),
                                    torch.zeros(b - a, device="cuda"), x[a:b, 2]], dim=1)
            assert torch.equal(out[a:b], want), f"excl={excl} rows [{a}, {b})"
        del out

"""CPU-side checks of the C ABI: the library loads, exports every entry point
that include/scan.h declares, and rejects bad arguments on the host before
anything touches a GPU (so these run without one).  The pointers below are
fake addresses: every call here returns from host validation."""
import ctypes
import os
import re

import pytest

import stream_compaction_amd as sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "scan.h")

OK, EINVAL, ENOTSUP, EALIAS, ESCRATCH = 0, 1, 2, 3, 4
D = sc.DTYPE_CODES
OP = sc.OP_CODES
A = 0x10000000            # fake, 256-byte aligned "device" addresses
B = 0x20000000
S = 0x30000000


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_]+)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(sc.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sc.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_enum_codes_match_header():
    text = open(HDR).read()
    for name, code in D.items():
        assert re.search(rf"SCAN_{name.upper()} = {code}\b", text), name
    for name, code in OP.items():
        assert re.search(rf"SCAN_{name.upper()} = {code}\b", text), name


def test_status_strings():
    L = sc.lib()
    for s in range(6):
        assert L.scan_status_str(s)
    assert L.scan_status_str(99) == b"unknown status"
    assert L.scan_last_hip_error() == 0


def rows(*args):
    return sc.lib().scan_rows(*args)


def test_scan_rows_validation():
    f32 = D["f32"]
    add = OP["add"]
    assert rows(A, B, 4, 16, D["i32"], add, 0, None) == ENOTSUP     # row scan is float-only
    assert rows(A, B, 4, 16, 0, add, 0, None) == ENOTSUP            # zeroed dtype code
    assert rows(A, B, 4, 16, f32, 0, 0, None) == ENOTSUP            # zeroed op code
    assert rows(A, B, 4, 16, f32, add, 2, None) == EINVAL           # exclusive must be 0/1
    assert rows(A, B, -1, 16, f32, add, 0, None) == EINVAL
    assert rows(A, B, 4, -16, f32, add, 0, None) == EINVAL
    assert rows(A, B, 4, 1 << 31, f32, add, 0, None) == EINVAL      # n > INT32_MAX
    assert rows(None, B, 4, 16, f32, add, 0, None) == EINVAL
    assert rows(A + 2, B, 4, 16, f32, add, 0, None) == EINVAL       # not element aligned
    assert rows(A, B + 1, 4, 16, D["bf16"], add, 0, None) == EINVAL
    assert rows(A, A + 64, 4, 16, f32, add, 0, None) == EALIAS      # 256 B ranges overlap
    assert rows(A, A, 1, 1, f32, add, 0, None) == EALIAS            # in place
    # empty shapes are no-ops that never launch (no GPU needed)
    assert rows(A, B, 0, 16, f32, add, 0, None) == OK
    assert rows(A, B, 4, 0, f32, add, 0, None) == OK
    assert rows(None, None, 0, 0, f32, add, 1, None) == OK


def test_scan_device_validation():
    L = sc.lib()
    i32 = D["i32"]
    add = OP["add"]
    need = L.scan_device_scratch_bytes(1000, i32)
    assert need >= 16 and need % 16 == 0
    assert L.scan_device_scratch_bytes(-1, i32) == 0
    assert L.scan_device(A, B, 1000, D["bf16"], add, S, need, None) == ENOTSUP
    assert L.scan_device(A, B, 1000, i32, 7, S, need, None) == ENOTSUP
    assert L.scan_device(A, B, -1, i32, add, S, need, None) == EINVAL
    assert L.scan_device(A, B, 1 << 31, i32, add, S, need, None) == EINVAL
    assert L.scan_device(A, B, 1000, i32, add, None, need, None) == EINVAL
    assert L.scan_device(A, B, 1000, i32, add, S + 8, need, None) == EINVAL   # scratch alignment
    assert L.scan_device(A, B + 2, 1000, i32, add, S, need, None) == EINVAL
    assert L.scan_device(A, B, 1000, i32, add, S, need - 1, None) == ESCRATCH
    assert L.scan_device(A, A + 3996, 1000, i32, add, S, need, None) == EALIAS
    assert L.scan_device(A, B, 1000, i32, add, A + 256, need, None) == EALIAS  # scratch in `in`
    assert L.scan_device(A, B, 0, i32, add, None, 0, None) == OK
    # scratch grows with n and is sized for every dtype and alignment
    for name in ("i32", "u32", "f32", "i64", "u64", "f64"):
        small = L.scan_device_scratch_bytes(1 << 20, D[name])
        big = L.scan_device_scratch_bytes(1 << 28, D[name])
        assert big > small > 0
        eb = 8 if name in ("i64", "u64", "f64") else 4
        assert big < (1 << 28) * eb // 100           # under 1% of the input bytes


def test_scan_device_inclusive_validation():
    L = sc.lib()
    i32 = D["i32"]
    need = L.scan_device_scratch_bytes(1000, i32)
    assert L.scan_device_inclusive(A, B, 1000, i32, OP["mul"], S, need, None) == ENOTSUP
    assert L.scan_device(A, B, 1000, i32, OP["mul"], S, need, None) == ENOTSUP
    assert L.scan_device_inclusive(A, B, 1000, D["f16"], OP["add"], S, need, None) == ENOTSUP
    assert L.scan_device_inclusive(A, B, 1000, i32, OP["add"], S, need - 1, None) == ESCRATCH
    assert L.scan_device_inclusive(A, A + 3996, 1000, i32, OP["add"], S, need, None) == EALIAS
    assert L.scan_device_inclusive(A, B, -3, i32, OP["add"], S, need, None) == EINVAL
    assert L.scan_device_inclusive(A, B, 0, i32, OP["add"], None, 0, None) == OK


def test_scan_rows_accepts_mul():
    # validation passes for the product on every row dtype (empty shape: no launch)
    for name in ("f32", "f16", "bf16"):
        assert rows(A, B, 0, 16, D[name], OP["mul"], 0, None) == OK
        assert rows(A, B, 4, 16, D[name], OP["mul"], 3, None) == EINVAL


def test_reduce_validation():
    L = sc.lib()
    i32, f64 = D["i32"], D["f64"]
    add = OP["add"]
    need = L.reduce_device_scratch_bytes(1 << 20, i32)
    assert need >= 16 and need % 16 == 0
    assert L.reduce_device_scratch_bytes(0, i32) == 0
    assert L.reduce_device_scratch_bytes(-1, i32) == 0
    # at most one 8-byte partial per workgroup, and never more than 2048 of them
    assert L.reduce_device_scratch_bytes(1 << 30, i32) <= 2048 * 8
    assert L.reduce_device_scratch_bytes(1 << 30, f64) <= 2048 * 8
    n = 1 << 20
    assert L.reduce_device(A, B, n, D["bf16"], add, S, need, None) == ENOTSUP
    assert L.reduce_device(A, B, n, i32, OP["mul"], S, need, None) == ENOTSUP
    assert L.reduce_device(A, B, n, i32, 0, S, need, None) == ENOTSUP
    assert L.reduce_device(A, B, -1, i32, add, S, need, None) == EINVAL
    assert L.reduce_device(A, B, 1 << 31, i32, add, S, need, None) == EINVAL
    assert L.reduce_device(A, None, n, i32, add, S, need, None) == EINVAL
    assert L.reduce_device(A, B + 2, n, i32, add, S, need, None) == EINVAL     # out alignment
    assert L.reduce_device(None, B, n, i32, add, S, need, None) == EINVAL
    assert L.reduce_device(A, B, n, i32, add, None, need, None) == EINVAL
    assert L.reduce_device(A, B, n, i32, add, S + 8, need, None) == EINVAL     # scratch alignment
    assert L.reduce_device(A, B, n, i32, add, S, need - 16, None) == ESCRATCH
    assert L.reduce_device(A, A + 4 * 100, n, i32, add, S, need, None) == EALIAS   # out in `in`
    assert L.reduce_device(A, B, n, i32, add, A + 4096, need, None) == EALIAS      # scratch in `in`
    assert L.reduce_device(A, S + 8, n, i32, add, S, need, None) == EALIAS         # out in scratch


def test_select_validation():
    L = sc.lib()
    need = L.select_compact_scratch_bytes(1000)
    N = B + 0x100000
    for eb in (0, 3, 5, 12, 32):                     # element widths other than 1/2/4/8/16
        assert L.select_compact(A, S + 0x1000, B, N, 1000, eb, S, need, None) == ENOTSUP
    assert L.select_compact(A + 1, S + 0x1000, B, N, 1000, 2, S, need, None) == EINVAL   # in alignment
    assert L.select_compact(A, S + 0x1000, B + 8, N, 1000, 16, S, need, None) == EINVAL  # out alignment
    assert L.select_compact(A, S + 0x1000, B, None, 1000, 4, S, need, None) == EINVAL
    assert L.select_compact(A, S + 0x1000, B, N + 2, 1000, 4, S, need, None) == EINVAL
    assert L.select_compact(A, S + 0x10000, B, N, -5, 4, S, need, None) == EINVAL
    assert L.select_compact(None, S + 0x10000, B, N, 1000, 4, S, need, None) == EINVAL
    assert L.select_compact(A, S + 0x10000, B, N, 1000, 4, S, need - 16, None) == ESCRATCH
    assert L.select_compact(A, S + 0x10000, A + 100, N, 1000, 4, S, need, None) == EALIAS
    assert L.select_compact(A, S + 0x10000, B, B + 40, 1000, 4, S, need, None) == EALIAS
    assert L.select_compact(A, S + 8, B, N, 1000, 4, S, need, None) == EALIAS    # flags in scratch


def test_binding_maps_status_to_exceptions():
    with pytest.raises(ValueError):
        sc.check(EINVAL)
    with pytest.raises(NotImplementedError):
        sc.check(ENOTSUP)
    with pytest.raises(ValueError):
        sc.check(EALIAS)
    with pytest.raises(sc.ScanError):
        sc.check(5)
    sc.check(OK)


def test_reduce_by_key_validation():
    L = sc.lib()
    n = 1000
    need = L.reduce_by_key_scratch_bytes(n)
    assert need >= 32 and need % 16 == 0
    assert L.reduce_by_key_scratch_bytes(-1) == 0
    i32, f32 = D["i32"], D["f32"]
    K, V, KO, VO, NR = A, A + 0x10000, B, B + 0x10000, B + 0x20000

    def call(*, k=K, v=V, ko=KO, vo=VO, nr=NR, nn=n, kd=i32, vd=f32, s=S, sb=need):
        return L.reduce_by_key(k, v, ko, vo, nr, nn, kd, vd, s, sb, None)
    assert call(kd=D["i64"]) == ENOTSUP
    assert call(vd=D["f64"]) == ENOTSUP
    assert call(kd=D["bf16"]) == ENOTSUP
    assert call(nn=-1) == EINVAL
    assert call(nn=1 << 31) == EINVAL
    assert call(nr=None) == EINVAL
    assert call(nr=NR + 2) == EINVAL
    assert call(k=None) == EINVAL
    assert call(vo=VO + 2) == EINVAL
    assert call(s=S + 8) == EINVAL
    assert call(sb=need - 16) == ESCRATCH
    assert call(ko=K + 400) == EALIAS                 # keys_out over keys_in
    assert call(vo=KO + 400) == EALIAS                # the two outputs overlap
    assert call(nr=VO + 40) == EALIAS                 # num_runs inside values_out
    assert call(s=V + 64) == EALIAS                   # scratch inside values_in
    # (calls that pass validation would launch on these fake addresses, so the
    # accepted cases, aliased inputs and n == 0 included, run in the GPU tests)


def test_radix_sort_validation():
    L = sc.lib()
    n = 100_000
    u32, u64 = D["u32"], D["u64"]
    need = L.radix_sort_scratch_bytes(n, u32)
    assert need > 0 and need % 16 == 0
    assert L.radix_sort_scratch_bytes(n, D["bf16"]) == 0
    KEY, TK, V, TV = A, A + 0x100000, B, B + 0x100000

    def call(*, k=KEY, tk=TK, v=V, tv=TV, nn=n, kd=u32, vd=u32, eb=32, s=S, sb=need):
        return L.radix_sort(k, tk, v, tv, nn, kd, vd, eb, s, sb, None)
    assert call(kd=D["f16"]) == ENOTSUP
    assert call(vd=D["bf16"]) == ENOTSUP
    assert call(nn=-1) == EINVAL
    assert call(nn=1 << 31) == EINVAL
    assert call(eb=12) == EINVAL
    assert call(eb=0) == EINVAL
    assert call(eb=40) == EINVAL                      # beyond a 32-bit key
    assert call(v=None) == EINVAL                     # values without temporaries
    assert call(k=None) == EINVAL
    assert call(k=KEY + 2) == EINVAL
    assert call(s=S + 8) == EINVAL
    assert call(sb=need - 16) == ESCRATCH
    assert call(tk=KEY + 400) == EALIAS
    assert call(tv=V + 4) == EALIAS
    assert call(s=TK + 64) == EALIAS
    assert call(kd=u64, tk=KEY + 8 * n - 8, sb=L.radix_sort_scratch_bytes(n, u64)) == EALIAS
    # 64-bit keys take 8 passes and have their own tile size
    assert L.radix_sort_scratch_bytes(n, u64) > 0


def test_devn_validation():
    L = sc.lib()
    i32, u32 = D["i32"], D["u32"]
    cap = 1000
    need = L.scan_device_scratch_bytes(cap, i32)
    NL = B + 0x100000                                  # the device count, away from everything
    assert L.scan_device_devn(A, B, None, cap, i32, OP["add"], S, need, None) == EINVAL
    assert L.scan_device_devn(A, B, NL + 2, cap, i32, OP["add"], S, need, None) == EINVAL
    assert L.scan_device_devn(A, B, B + 40, cap, i32, OP["add"], S, need, None) == EALIAS  # in out
    assert L.scan_device_devn(A, B, S + 64, cap, i32, OP["add"], S, need, None) == EALIAS  # in scratch
    assert L.scan_device_inclusive_devn(A, B, B + 8, cap, i32, OP["max"], S, need, None) == EALIAS
    assert L.scan_device_devn(A, B, NL, cap, i32, OP["add"], S, need - 1, None) == ESCRATCH
    rneed = L.reduce_device_scratch_bytes(cap, i32)
    assert L.reduce_device_devn(A, B, None, cap, i32, OP["add"], S, rneed, None) == EINVAL
    assert L.reduce_device_devn(A, B, B, cap, i32, OP["add"], S, rneed, None) == EALIAS   # in out
    kneed = L.reduce_by_key_scratch_bytes(cap)
    assert L.reduce_by_key_devn(A, A + 0x10000, B, B + 0x10000, B + 0x20000, None, cap, i32, i32,
                                S, kneed, None) == EINVAL
    assert L.reduce_by_key_devn(A, A + 0x10000, B, B + 0x10000, B + 0x20000, B + 0x20000, cap,
                                i32, i32, S, kneed, None) == EALIAS      # the count is num_runs
    sneed = L.radix_sort_scratch_bytes(cap, u32)
    assert L.radix_sort_devn(A, A + 0x100000, None, None, NL, cap, u32, 0, 24, S, sneed,
                             None) == EINVAL                            # odd pass count
    assert L.radix_sort_devn(A, A + 0x100000, None, None, None, cap, u32, 0, 32, S, sneed,
                             None) == EINVAL
    assert L.radix_sort_devn(A, A + 0x100000, None, None, A + 8, cap, u32, 0, 32, S, sneed,
                             None) == EALIAS                            # the count is a key
    cneed = L.select_compact_scratch_bytes(cap)
    assert L.select_compact_devn(A, S + 0x10000, B, B + 0x10000, None, cap, 4, S, cneed,
                                 None) == EINVAL
    assert L.select_compact_devn(A, S + 0x10000, B, B + 0x10000, B + 0x10000, cap, 4, S, cneed,
                                 None) == EALIAS                        # the count is num_out


def test_scan_device_noalloc_validation():
    # every case is rejected on the host, before the static scratch is looked up
    L = sc.lib()
    assert L.scan_device_noalloc(A, B, 100, D["f16"], OP["add"], None) == ENOTSUP
    assert L.scan_device_noalloc(A, B, 100, D["i32"], OP["mul"], None) == ENOTSUP
    assert L.scan_device_noalloc(A, B, -1, D["i32"], OP["add"], None) == EINVAL
    assert L.scan_device_noalloc(A, B, 0, D["i32"], OP["add"], None) == OK
    assert L.scan_device_noalloc(0, B, 100, D["i32"], OP["add"], None) == EINVAL
    assert L.scan_device_noalloc(A + 2, B, 100, D["i32"], OP["add"], None) == EINVAL
    assert L.scan_device_noalloc(A, A + 8, 100, D["i32"], OP["add"], None) == EALIAS
    # the static scratch holds the descriptors of at most 65,535 tiles of 7,168 elements
    n_max = 65_535 * 7_168
    assert L.scan_device_scratch_bytes(n_max, D["i32"]) <= 8 << 20
    assert L.scan_device_scratch_bytes(n_max + 1, D["i32"]) > 8 << 20
    for dt in ("i32", "f64"):
        assert L.scan_device_noalloc(A, B, n_max + 1, D[dt], OP["add"], None) == ESCRATCH
        assert L.scan_device_noalloc(A, B, (1 << 31) - 1, D[dt], OP["min"], None) == ESCRATCH

"""GPU parity at the tile boundaries of the look-back kernels.

The device-wide scans, select and reduce-by-key cut their input into tiles of
a fixed number of 16-byte vectors (one workgroup each), so an array that ends
one element before, exactly at, or one element after a tile boundary takes a
different path through the kernel: a last tile with a single element, a last
tile whose every vector is full (the fast store path, no partial tile), or a
second tile holding one element.  The sizes below are derived from the launch
shapes (data waves x loads per lane x 64 lanes = vectors per tile, times the
elements per vector), and every case is compared with the oracle: bit for bit
for integers, min/max and select, within the float-add tolerance otherwise.

Arrays that start inside a 16-byte vector are addressed through an aligned
window that begins `ph` elements before the array, so their boundaries move to
k*T - ph; each size list is repeated for in-phase offsets of 1-3 elements.  The
device scans start their window on the 128-byte line that holds the first
element when input and output share their place in it, so for them ph is the
element offset within the line, and offsets past the first vector are tested
too.
Arrays whose input and output phases differ run with one element per vector,
so their tiles are as many elements as vectors.
"""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_amd as sc
import workloads
from gpu_util import STORE_T, from_dev, rand_input, to_dev
from parity import FP_ABS, FP_REL, check_exact, check_fp_add

pytestmark = pytest.mark.gpu

# launch shapes (vectors per tile)
DEV_ADD_TILE_VECS = 8 * 16 * 64  # device add scans: 8 side-by-side data waves x 16 loads
DEV_RUNS_TILE_VECS = 11 * 12 * 64  # device min/max scans: 11 data waves x 12 loads each
SEL_TILE_VECS = 8 * 8 * 4 * 64   # select: 8 data waves x 8 chunks x 4 loads
RBK_TILE_VECS = 11 * 6 * 64      # reduce-by-key: 11 data waves x 6 loads


def edge_sizes(t, ph=0):
    """Counts around one, two and three tiles of t elements for a window phase ph."""
    return [t - ph - 1, t - ph, t - ph + 1, 2 * t - ph + 37, 3 * t - ph]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.lib()
    yield
    torch.cuda.synchronize()


def views(n, dt, off_in, off_out):
    """Zeroed device buffers of n + 40 elements and the n-element views at the offsets."""
    big_in = torch.zeros(n + 40, dtype=STORE_T[dt], device="cuda")
    big_out = torch.zeros(n + 40, dtype=STORE_T[dt], device="cuda")
    return big_in, big_out, big_in[off_in:off_in + n], big_out[off_out:off_out + n]


def dev_tile_vecs(op):
    return DEV_ADD_TILE_VECS if op == "add" else DEV_RUNS_TILE_VECS


def compare(gpu, x, dt, op, inclusive, label):
    if op == "add" and dt in oracle.FLOATS:
        ora, ref, absref = oracle.scan(x, dt, op, exclusive=not inclusive, want_ref=True)
        check_fp_add(gpu, ora, ref, absref, dt, label)
    else:
        check_exact(gpu, oracle.scan(x, dt, op, exclusive=not inclusive), label)


# ---------------------------------------------------------------------------
# device-wide scans (exclusive and inclusive), every element width
# ---------------------------------------------------------------------------

DEV_CASES = [("i32", "add"), ("u32", "max"), ("i32", "min"), ("f32", "min"), ("f32", "add"),
             ("i64", "add"), ("u64", "min"), ("f64", "max"), ("f64", "add")]


@pytest.mark.parametrize("dt,op", DEV_CASES)
@pytest.mark.parametrize("inclusive", [False, True], ids=["excl", "incl"])
def test_device_scan_tile_edges(dt, op, inclusive):
    e = 16 // np.dtype(oracle.STORAGE[dt]).itemsize
    t = dev_tile_vecs(op) * e
    fn = sc.scan_device_inclusive if inclusive else sc.scan_device
    seed = 0
    # offsets within the first vector, then past it (up to the end of a line)
    offs = [0, 1, 2, 3, 5, 17, 31] if e == 4 else [0, 1, 3, 9, 15]
    for off in offs:
        ph = off                        # the window phase: the offset within the 128-byte line
        for n in edge_sizes(t, ph):
            seed += 1
            x = rand_input(dt, n, 70_000 + seed)
            big_in, big_out, xin, yout = views(n, dt, off, off)
            xin.copy_(to_dev(x, dt))
            fn(xin, op=op, out=yout, dtype=dt)
            torch.cuda.synchronize()
            label = f"scan_device {dt} {op} incl={inclusive} n={n} offset {off}"
            compare(from_dev(yout, dt), x, dt, op, inclusive, label)
            assert not big_out[:off].any() and not big_out[off + n:].any(), label + ": outside written"


@pytest.mark.parametrize("dt,op", [("i32", "add"), ("i64", "max"), ("f64", "add")])
def test_device_scan_tile_edges_one_element_vectors(dt, op):
    # input and output phases differ: one element per vector, tiles of as many elements
    t = dev_tile_vecs(op)
    for i, n in enumerate(edge_sizes(t)):
        x = rand_input(dt, n, 71_000 + i)
        for inclusive in (False, True):
            big_in, big_out, xin, yout = views(n, dt, 1, 0)
            xin.copy_(to_dev(x, dt))
            (sc.scan_device_inclusive if inclusive else sc.scan_device)(xin, op=op, out=yout,
                                                                         dtype=dt)
            torch.cuda.synchronize()
            compare(from_dev(yout, dt), x, dt, op, inclusive,
                    f"scan_device {dt} {op} incl={inclusive} n={n} phases 1/0")


# ---------------------------------------------------------------------------
# select: every element width, p in {0, 0.5, 1}
# ---------------------------------------------------------------------------

SENTINEL = 0x5A
SEL_NP = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64, 16: np.complex128}


def sel_elems(eb):
    """Elements per payload vector: 4 for 1-, 2- and 4-byte elements, 2 for 8, 1 for 16."""
    return 4 if eb <= 4 else 16 // eb


def run_select_view(xb, flags, eb, off, label):
    """xb: uint8 [n, eb]; payload, flags and output all at element offset `off`."""
    n = xb.shape[0]
    tdt = torch.from_numpy(np.zeros(1, SEL_NP[eb])).dtype
    big_in = torch.zeros(n + 128, dtype=tdt, device="cuda")
    big_f = torch.zeros(n + 136, dtype=torch.uint8, device="cuda")
    big_out = torch.from_numpy(np.full((n + 128) * eb, SENTINEL, np.uint8).view(SEL_NP[eb])).cuda()
    big_in[off:off + n].copy_(torch.from_numpy(xb.reshape(-1).view(SEL_NP[eb]).copy()).cuda())
    big_f[off:off + n].copy_(torch.from_numpy(flags).cuda())
    _, num = sc.select_compact(big_in[off:off + n], big_f[off:off + n], out=big_out[off:off + n])
    k = int(num.item())
    ora, ko = oracle.select(xb.reshape(-1).view(np.dtype((np.void, eb))), flags)
    assert k == ko, f"{label}: count {k} != {ko}"
    got = big_out.cpu().numpy().view(np.uint8).reshape(n + 128, eb)
    want = np.ascontiguousarray(ora).view(np.uint8).reshape(n, eb)
    check_exact(got[off:off + k].reshape(-1), want[:k].reshape(-1), label)
    assert (got[:off] == SENTINEL).all() and (got[off + k:] == SENTINEL).all(), \
        f"{label}: written outside the kept prefix"


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("p", [0.0, 0.5, 1.0])
def test_select_tile_edges(eb, p):
    e = sel_elems(eb)
    t = SEL_TILE_VECS * e
    seed = 0
    # offsets within the first payload vector, then past it: the window then
    # starts on the payload's 128-byte line, ph elements before the array
    line = 128 // eb
    for off in sorted({0, 1, 2, 3, line // 4 + 1, line - 1} if e > 1 else {0, 3, line - 1}):
        ph = off % line
        for n in edge_sizes(t, ph):
            seed += 1
            rng = np.random.default_rng(72_000 + seed)
            xb = rng.integers(0, 256, size=(n, eb), dtype=np.uint8)
            flags = workloads.bernoulli_flags(n, p, 73_000 + seed)
            run_select_view(xb, flags, eb, off, f"select eb={eb} p={p} n={n} offset {off}")


# ---------------------------------------------------------------------------
# reduce-by-key
# ---------------------------------------------------------------------------

def rbk_case(n, mean_run, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.geometric(1.0 / mean_run, size=n + 16)
    keys = np.repeat(rng.integers(0, 8, size=lengths.size), lengths)[:n].astype(np.int32)
    values = rng.integers(-1000, 1000, size=n).astype(np.int32)
    return keys, values


def run_rbk_view(keys, values, off_k, off_v, vd, label):
    n = keys.size
    bk = torch.zeros(n + 40, dtype=torch.int32, device="cuda")
    bv = torch.zeros(n + 40, dtype=STORE_T[vd], device="cuda")
    bk[off_k:off_k + n].copy_(torch.from_numpy(keys).cuda())
    bv[off_v:off_v + n].copy_(to_dev(values, vd))
    ko = torch.full((n,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    vo = torch.from_numpy(np.full(n, 0x5A5A5A5A, np.uint32).view(oracle.STORAGE[vd]).copy()).cuda()
    _, _, nr = sc.reduce_by_key(bk[off_k:off_k + n], bv[off_v:off_v + n], ko, vo,
                                key_dtype="i32", value_dtype=vd)
    r = int(nr.item())
    oko, ovo, orr, ref, absref = oracle.reduce_by_key(keys, values, "i32", vd, want_ref=True)
    assert r == orr, f"{label}: {r} runs, oracle {orr}"
    check_exact(ko.cpu().numpy()[:r], oko[:r], label + " keys")
    gv = from_dev(vo, vd)
    if vd == "f32":
        err = np.abs(gv[:r].astype(np.float64) - ref[:r])
        assert (err <= FP_REL * absref[:r] + FP_ABS).all(), f"{label}: value out of tolerance"
    else:
        check_exact(gv[:r], ovo[:r], label + " values")
    assert (ko.cpu().numpy()[r:].view(np.uint32) == 0x5A5A5A5A).all(), f"{label}: keys tail written"
    assert (gv[r:].view(np.uint32) == 0x5A5A5A5A).all(), f"{label}: values tail written"


@pytest.mark.parametrize("mean_run", [1, 6, 5000])
def test_reduce_by_key_tile_edges(mean_run):
    t = RBK_TILE_VECS * 4
    seed = 0
    # offsets within the first vector, then past it (the window starts on the
    # keys' 128-byte line when the values share it)
    for ph in (0, 1, 2, 3, 9, 31):
        for n in edge_sizes(t, ph):
            seed += 1
            keys, values = rbk_case(n, mean_run, 74_000 + seed + 100 * mean_run)
            run_rbk_view(keys, values, ph, ph, "i32",
                         f"reduce_by_key mean run {mean_run} n={n} offset {ph}")


def test_reduce_by_key_tile_edges_float_values_and_one_element_vectors():
    t = RBK_TILE_VECS * 4
    for i, n in enumerate(edge_sizes(t)):
        keys, _ = rbk_case(n, 7, 75_000 + i)
        values = np.random.default_rng(75_100 + i).uniform(-1, 1, size=n).astype(np.float32)
        run_rbk_view(keys, values, 0, 0, "f32", f"reduce_by_key f32 values n={n}")
    # keys and values at different phases: one element per vector
    for i, n in enumerate(edge_sizes(RBK_TILE_VECS)):
        keys, values = rbk_case(n, 3, 75_200 + i)
        run_rbk_view(keys, values, 1, 0, "i32", f"reduce_by_key phases 1/0 n={n}")

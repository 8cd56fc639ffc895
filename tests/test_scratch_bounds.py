"""Host logic: the scratch each look-back kernel and the reduction ask for
covers every tile (or partial) any of their launches can use.

The launches cut the input into tiles of a fixed number of vectors, counted
over a window that starts up to one 128-byte line before the array (a window
phase `ph` of up to 128 / element-size - 1 elements) or, when input and output
phases differ, over one element per vector.  The scratch-size functions of the
C ABI are pure host arithmetic, so this runs without a GPU: for many counts n
and every phase and element width, the descriptors (one 128-byte line per tile,
plus one line of alignment slack) or reduction partials (8 bytes per workgroup
of the first launch) a launch needs must fit in what the function returns.

The launch shapes below are the kernels' (vectors per tile); a change of shape
must be reflected here.
"""
import numpy as np

import stream_compaction_amd as sc

LINE = 128
DEV_TILES_VECS = (8 * 16 * 64, 11 * 12 * 64)    # device scan: side by side (add), runs (min/max)
SEL_TILE_VECS = 8 * 8 * 4 * 64                   # select, every element width
RBK_TILE_VECS = 11 * 6 * 64                      # reduce-by-key
RED_WAVES, RED_MAX_BLOCKS = 4, 2048              # reduction: waves per workgroup, workgroup cap
RED_LOADS = (8, 16)                              # loads per lane per run (float min/max, others)


def counts():
    """Counts around every tile boundary that matters, small ones, and a spread of large ones."""
    ns = set(range(1, 600))
    for t in (7168, 8192, 8448, 16384, 4224, 65536, 33792, 16896, 32768):
        for m in (1, 2, 3, 7, 64, 1000):
            for d in range(-40, 41):
                ns.add(t * m + d)
    rng = np.random.default_rng(7)
    ns.update(int(x) for x in rng.integers(1, 2**31 - 1, size=400))
    ns.update((2**31 - 1, 2**31 - 2, 2**30, 2**28, 2**28 - 37))
    return sorted(n for n in ns if 1 <= n <= 2**31 - 1)


def tiles(n, ph, e, tv):
    """Tiles of tv vectors of e elements over window elements [ph, n + ph)."""
    return ((n + ph - 1) // e) // tv + 1


def desc_bytes(ntiles):
    return ntiles * LINE + LINE


def test_scan_device_scratch_covers_every_launch():
    L = sc.lib()
    for name, size in (("i32", 4), ("u32", 4), ("f32", 4), ("i64", 8), ("u64", 8), ("f64", 8)):
        e = 16 // size
        code = sc.DTYPE_CODES[name]
        for n in counts():
            have = L.scan_device_scratch_bytes(n, code)
            for tv in DEV_TILES_VECS:
                need = desc_bytes(tiles(n, 0, 1, tv))          # one element per vector
                for ph in range(LINE // size):                # windows on a line
                    need = max(need, desc_bytes(tiles(n, ph, e, tv)))
                assert have >= need, f"scan_device {name} n={n}: {have} < {need}"


def test_select_scratch_covers_every_launch():
    L = sc.lib()
    for n in counts():
        have = L.select_compact_scratch_bytes(n)
        for eb in (1, 2, 4, 8, 16):
            e = 4 if eb <= 4 else 16 // eb
            need = max(desc_bytes(tiles(n, ph, e, SEL_TILE_VECS)) for ph in range(LINE // eb))
            assert have >= need, f"select eb={eb} n={n}: {have} < {need}"


def test_reduce_by_key_scratch_covers_every_launch():
    L = sc.lib()
    for n in counts():
        have = L.reduce_by_key_scratch_bytes(n)
        need = desc_bytes(tiles(n, 0, 1, RBK_TILE_VECS))
        need = max([need] + [desc_bytes(tiles(n, ph, 4, RBK_TILE_VECS)) for ph in range(LINE // 4)])
        assert have >= need, f"reduce_by_key n={n}: {have} < {need}"


def red_blocks(n, e, ph, run_vecs):
    """Workgroups of the reduction's first launch: runs of run_vecs vectors spread over at
    most RED_MAX_BLOCKS workgroups of RED_WAVES waves, none left without a run."""
    runs = ((n + ph - 1) // e) // run_vecs + 1
    blocks = min(-(-runs // RED_WAVES), RED_MAX_BLOCKS)
    per_wave = -(-runs // (blocks * RED_WAVES))
    waves_used = -(-runs // per_wave)
    return -(-waves_used // RED_WAVES)


def test_reduce_scratch_covers_every_launch():
    L = sc.lib()
    for name, size in (("i32", 4), ("f32", 4), ("i64", 8), ("f64", 8)):
        e = 16 // size
        code = sc.DTYPE_CODES[name]
        for n in counts():
            have = L.reduce_device_scratch_bytes(n, code)
            need = max(8 * red_blocks(n, e, ph, 64 * loads)
                       for loads in RED_LOADS for ph in range(LINE // size))
            assert have >= need, f"reduce {name} n={n}: {have} < {need}"


def test_noalloc_limit_matches_its_scratch():
    # the allocation-free scan takes n up to the largest count whose scratch
    # fits its static array
    L = sc.lib()
    limit = 469_754_880
    for name in ("i32", "f64"):
        code = sc.DTYPE_CODES[name]
        assert L.scan_device_scratch_bytes(limit, code) <= 8 << 20
        assert L.scan_device_scratch_bytes(limit + 1, code) > 8 << 20

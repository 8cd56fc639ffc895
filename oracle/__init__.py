"""Plain sequential CPU oracle for row-wise scan, device-wide scan and select.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product library
(``stream_compaction_amd``) never imports, links or calls it, and this module
imports nothing from the product.

The arithmetic lives in ``oracle/oracle.c`` (compiled by gcc into
``oracle/liboracle.so``); this file only marshals numpy arrays.  What it
computes, with the passages it follows:

* ``scan``: the left-prefix recurrence from "Tile operations and reductions"
  (section "Why not just infer it from reduce?"): ``p[0] = identity``,
  ``p[i+1] = op(p[i], x[i])``, inclusive ``out[i] = p[i+1]``, exclusive
  ``out[i] = p[i]``, applied to every row of a ``[rows, n]`` array (the row
  definitions of metaltile-std ``src/mlx/scan.rs``, header comment).  The
  identities are those of the "Algorithms" page, "Common conventions".
* ``scan`` with ``op="mul"``: the product scans of metaltile-std
  ``src/mlx/scan.rs`` ("Inclusive product scan", "Exclusive product scan";
  identity 1 from its "Multi-op scan variants" table), accumulated in double.
* ``reduce``: ``out[0] = op(x[0..n))`` per the "Algorithms" page, section
  ``qd.algorithms.reduce_{add,min,max}``: the final state of the same
  recurrence, the identity for an empty input.
* ``reduce_by_key``: runs of equal consecutive keys collapsed into (first key,
  sum of values) per the "Algorithms" page, section
  ``qd.algorithms.reduce_by_key_add``.
* ``sort`` / ``sort_image``: stable ascending radix-sort order per the
  "Algorithms" page, section ``qd.algorithms.sort`` (sortable-key transform
  written out; numpy's stable argsort orders the transformed keys).
* ``select``: stream compaction per the "Algorithms" page, section
  ``qd.algorithms.select`` (stable, dense prefix, count).
* ``f32_to_bf16`` / ``f32_to_f16`` and the widenings: round-to-nearest-even per
  "Tile operations and reductions", section "Storage and arithmetic precision".

Every function here is pinned in ``tests/test_oracle.py`` against page
examples, closed forms, invariants, brute force and independent library
routines.  Floating add beyond those pins is "parity unpinned" (only the
tolerance against the double fold applies).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

# the oracle's own codes (see oracle.c); the product library has separate ones
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3, "i32": 4, "u32": 5, "i64": 6, "u64": 7}
OPS = {"add": 0, "min": 1, "max": 2, "mul": 3}
# numpy storage type of each dtype (bf16 and f16 travel as raw uint16 bits)
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64,
           "i32": np.int32, "u32": np.uint32, "i64": np.int64, "u64": np.uint64}
FLOATS = ("f32", "f16", "bf16", "f64")

_lib = None


def build_cmd():
    """The gcc command that builds liboracle.so (used by __graft_entry__.build)."""
    return ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
            SRC_PATH, "-o", LIB_PATH, "-lm"]


def build():
    import subprocess
    subprocess.check_call(build_cmd())


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_scan.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp]
        L.oracle_scan.restype = i32
        L.oracle_reduce.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.oracle_reduce.restype = i32
        L.oracle_reduce_by_key.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp]
        L.oracle_reduce_by_key.restype = i64
        L.oracle_select.argtypes = [vp, vp, vp, i64, i64]
        L.oracle_select.restype = i64
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def scan(x, dtype, op="add", exclusive=False, want_ref=False):
    """Scan every row of ``x`` (shape ``[rows, n]`` or ``[n]``) along its last axis.

    ``x`` holds the storage type of ``dtype`` (``STORAGE``).  Returns ``out``
    with the same shape and storage type; with ``want_ref`` also returns
    ``(ref, absref)`` as float64 arrays: ``ref`` is the double accumulator
    behind each output (floating add) and ``absref[i] = sum_{j<=i}|x_j|``.
    """
    x = np.ascontiguousarray(x, dtype=STORAGE[dtype])
    shape = x.shape
    if x.ndim == 1:
        rows, n = 1, x.shape[0]
    else:
        rows, n = int(np.prod(shape[:-1])), shape[-1]
    out = np.empty_like(x)
    ref = absref = None
    if want_ref:
        ref = np.zeros(shape, dtype=np.float64)
        absref = np.zeros(shape, dtype=np.float64)
    rc = lib().oracle_scan(_ptr(x), _ptr(out), rows, n, DTYPES[dtype], OPS[op],
                           1 if exclusive else 0, _ptr(ref), _ptr(absref))
    if rc != 0:
        raise ValueError("oracle_scan rejected its arguments")
    if want_ref:
        return out, ref, absref
    return out


def reduce(x, dtype, op="add", want_ref=False):
    """Fold all of the 1-D ``x`` (storage type of ``dtype``) from the identity.

    Returns a one-element array of the storage type; with ``want_ref`` also
    ``(ref, absref)`` as Python floats: the double accumulator (floating add
    and mul; the value itself otherwise) and ``sum |x_j|``.
    """
    x = np.ascontiguousarray(x, dtype=STORAGE[dtype]).ravel()
    out = np.zeros(1, dtype=STORAGE[dtype])
    ref = np.zeros(1, dtype=np.float64)
    absref = np.zeros(1, dtype=np.float64)
    rc = lib().oracle_reduce(_ptr(x), _ptr(out), x.shape[0], DTYPES[dtype], OPS[op],
                             _ptr(ref), _ptr(absref))
    if rc != 0:
        raise ValueError("oracle_reduce rejected its arguments")
    if want_ref:
        return out, float(ref[0]), float(absref[0])
    return out


def reduce_by_key(keys, values, key_dtype, value_dtype, want_ref=False):
    """Collapse runs of equal consecutive keys into (first key, sum of values).

    ``keys`` / ``values`` hold the storage types of ``key_dtype`` /
    ``value_dtype`` (each "i32", "u32" or "f32").  Returns ``(keys_out,
    values_out, r)`` with ``len(keys)`` slots each (zero past ``r``); with
    ``want_ref`` also per-run ``(ref, absref)`` float64 arrays (f32 values).
    """
    keys = np.ascontiguousarray(keys, dtype=STORAGE[key_dtype]).ravel()
    values = np.ascontiguousarray(values, dtype=STORAGE[value_dtype]).ravel()
    if keys.shape != values.shape:
        raise ValueError("keys and values differ in length")
    n = keys.shape[0]
    ko = np.zeros(n, dtype=STORAGE[key_dtype])
    vo = np.zeros(n, dtype=STORAGE[value_dtype])
    ref = np.zeros(n, dtype=np.float64)
    absref = np.zeros(n, dtype=np.float64)
    r = lib().oracle_reduce_by_key(_ptr(keys), _ptr(values), n, DTYPES[key_dtype],
                                   DTYPES[value_dtype], _ptr(ko), _ptr(vo), _ptr(ref),
                                   _ptr(absref))
    if r < 0:
        raise ValueError("oracle_reduce_by_key rejected its arguments")
    if want_ref:
        return ko, vo, int(r), ref, absref
    return ko, vo, int(r)


_SORT_UNSIGNED = {"u32": np.uint32, "i32": np.uint32, "f32": np.uint32,
                  "u64": np.uint64, "i64": np.uint64, "f64": np.uint64}


def sort_image(keys, key_dtype, end_bit=None):
    """The unsigned integer each key sorts by (ascending), restricted to its
    low ``end_bit`` bits.

    Written from the "Algorithms" page, section qd.algorithms.sort (Under the
    hood): unsigned keys sort as they are; signed keys with their sign bit
    flipped; floats with the sign bit flipped when it is clear and every bit
    flipped when it is set (the standard sortable-key transform), so -0 sorts
    just before +0.  The page also states that NaNs land at the end, as in
    numpy.sort: every NaN (either sign) takes the largest image, so NaNs go
    last and keep their input order.
    """
    u_t = _SORT_UNSIGNED[key_dtype]
    bits = 32 if u_t is np.uint32 else 64
    u = np.ascontiguousarray(keys).view(u_t).copy()
    top = u_t(1) << u_t(bits - 1)
    if key_dtype in ("i32", "i64"):
        u ^= top
    elif key_dtype in ("f32", "f64"):
        neg = (u & top) != 0
        u = np.where(neg, ~u, u | top).astype(u_t)
        f = np.ascontiguousarray(keys).view(np.float32 if bits == 32 else np.float64)
        u[np.isnan(f)] = np.iinfo(u_t).max
    if end_bit is not None and end_bit < bits:
        u &= u_t((1 << end_bit) - 1)
    return u


def sort(keys, key_dtype, values=None, end_bit=None):
    """Stable ascending sort of 1-D ``keys`` by their sort image (see
    ``sort_image``); ``values`` (any 1-D array of the same length) are
    permuted alongside.  The "Algorithms" page, section qd.algorithms.sort:
    ascending, stable (equal images keep their input order).  Returns
    ``(sorted_keys, sorted_values or None)``; the keys' bits are moved, not
    transformed.  The ordering step is numpy's stable argsort of the images.
    """
    keys = np.ascontiguousarray(keys)
    order = np.argsort(sort_image(keys, key_dtype, end_bit), kind="stable")
    return keys[order], (None if values is None else np.ascontiguousarray(values)[order])


def select(x, flags):
    """Stable compaction of ``x`` (1-D, any fixed-size dtype) by nonzero ``flags`` (u8).

    Returns ``(out, k)`` where ``out`` has ``len(x)`` slots, zero-filled past ``k``.
    """
    x = np.ascontiguousarray(x)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    if x.shape[0] != flags.shape[0]:
        raise ValueError("x and flags differ in length")
    out = np.zeros_like(x)
    k = lib().oracle_select(_ptr(x), _ptr(flags), _ptr(out), x.shape[0], x.dtype.itemsize)
    return out, int(k)


def f32_to_bf16(v):
    return np.array([lib().oracle_f32_to_bf16(float(f)) for f in np.asarray(v, np.float32).ravel()],
                    dtype=np.uint16)


def f32_to_f16(v):
    return np.array([lib().oracle_f32_to_f16(float(f)) for f in np.asarray(v, np.float32).ravel()],
                    dtype=np.uint16)


def bf16_to_f32(h):
    return np.array([lib().oracle_bf16_to_f32(int(b)) for b in np.asarray(h, np.uint16).ravel()],
                    dtype=np.float32)


def f16_to_f32(h):
    return np.array([lib().oracle_f16_to_f32(int(b)) for b in np.asarray(h, np.uint16).ravel()],
                    dtype=np.float32)

"""stream_compaction_amd: prefix scan and stream compaction on an MI355X (gfx950).

Thin Python binding over the C ABI of ``libscan_amd.so`` (declared in
``include/scan.h``).  Every step of every operation runs in the library's HIP
kernels; this module only turns torch tensors into device pointers, sizes and
the current HIP stream, and turns status codes into exceptions.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI):

* ``scan_rows(x, op="add", exclusive=False, out=None)`` - scan along the last
  axis of a contiguous ``[rows, n]`` float32/float16/bfloat16 tensor
  (op: add, min, max, mul).
* ``scan_device(x, op="add", out=None, scratch=None)`` - device-wide exclusive
  scan of a 1-D int32/uint32/float32/int64/uint64/float64 tensor.
* ``scan_device_inclusive(x, op="add", out=None, scratch=None)`` - the same,
  inclusive.
* ``reduce_device(x, op="add", out=None, scratch=None)`` - device-wide
  reduction into a 1-element GPU tensor.
* ``reduce_by_key(keys, values, keys_out=None, values_out=None, num_runs=None,
  scratch=None)`` - runs of equal consecutive keys collapsed into (key, sum).
* ``radix_sort(keys, values=None, tmp_keys=None, tmp_values=None, end_bit=None,
  scratch=None)`` - stable ascending sort of a 1-D tensor of 32/64-bit keys in
  place, carrying values along.
* ``select_compact(x, flags, out=None, num_out=None, scratch=None)`` - stable
  stream compaction of a 1-D tensor with elements of 1, 2, 4, 8 or 16 bytes by
  uint8 flags (elements move as raw bits).
* ``scan_device_noalloc(x, op="add", out=None)`` - ``scan_device`` on the
  library's own per-GPU scratch, for callers that cannot allocate (calls that
  overlap on one GPU race).
* ``*_devn`` variants of the device-wide calls (C ABI names; ``n_live`` a
  1-element int32 GPU tensor, ``capacity`` the tensors' length): the count is
  read on the device, so one captured graph serves every count up to the
  capacity.  Python wrappers: ``scan_device(..., n_live=t)`` and likewise.
* ``scan_device_scratch_bytes(n, dtype)``, ``reduce_device_scratch_bytes(n,
  dtype)``, ``reduce_by_key_scratch_bytes(n)``, ``select_compact_scratch_bytes(n)``.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libscan_amd.so")

# codes of include/scan.h
_STATUS = {0: "SCAN_OK", 1: "SCAN_EINVAL", 2: "SCAN_ENOTSUP", 3: "SCAN_EALIAS",
           4: "SCAN_ESCRATCH", 5: "SCAN_EHIP"}
DTYPE_CODES = {"f32": 1, "f16": 2, "bf16": 3, "f64": 4, "i32": 5, "u32": 6, "i64": 7, "u64": 8}
OP_CODES = {"add": 1, "min": 2, "max": 3, "mul": 4}
EXPORTS = ("scan_rows", "scan_device", "scan_device_inclusive", "scan_device_scratch_bytes",
           "reduce_device", "reduce_device_scratch_bytes", "reduce_by_key",
           "reduce_by_key_scratch_bytes", "radix_sort", "radix_sort_scratch_bytes",
           "select_compact", "select_compact_scratch_bytes", "scan_device_devn",
           "scan_device_inclusive_devn", "reduce_device_devn", "reduce_by_key_devn",
           "radix_sort_devn", "select_compact_devn", "scan_device_noalloc", "scan_status_str",
           "scan_last_hip_error")

_lib = None


class ScanError(RuntimeError):
    """A HIP runtime failure reported by the library (SCAN_EHIP)."""


def lib():
    """Load libscan_amd.so (built in-tree by ``python -m stream_compaction_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path):
    """Load a build of the library at ``path`` and declare its C signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m stream_compaction_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.scan_rows.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp]
    L.scan_rows.restype = i32
    L.scan_device_scratch_bytes.argtypes = [i64, i32]
    L.scan_device_scratch_bytes.restype = sz
    L.scan_device.argtypes = [vp, vp, i64, i32, i32, vp, sz, vp]
    L.scan_device.restype = i32
    L.scan_device_noalloc.argtypes = [vp, vp, i64, i32, i32, vp]
    L.scan_device_noalloc.restype = i32
    L.scan_device_inclusive.argtypes = [vp, vp, i64, i32, i32, vp, sz, vp]
    L.scan_device_inclusive.restype = i32
    L.reduce_device_scratch_bytes.argtypes = [i64, i32]
    L.reduce_device_scratch_bytes.restype = sz
    L.reduce_device.argtypes = [vp, vp, i64, i32, i32, vp, sz, vp]
    L.reduce_device.restype = i32
    L.reduce_by_key_scratch_bytes.argtypes = [i64]
    L.reduce_by_key_scratch_bytes.restype = sz
    L.reduce_by_key.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, vp, sz, vp]
    L.reduce_by_key.restype = i32
    L.radix_sort_scratch_bytes.argtypes = [i64, i32]
    L.radix_sort_scratch_bytes.restype = sz
    L.radix_sort.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    L.radix_sort.restype = i32
    L.select_compact_scratch_bytes.argtypes = [i64]
    L.select_compact_scratch_bytes.restype = sz
    L.select_compact.argtypes = [vp, vp, vp, vp, i64, sz, vp, sz, vp]
    L.select_compact.restype = i32
    for name in ("scan_device_devn", "scan_device_inclusive_devn", "reduce_device_devn"):
        getattr(L, name).argtypes = [vp, vp, vp, i64, i32, i32, vp, sz, vp]
        getattr(L, name).restype = i32
    L.reduce_by_key_devn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, vp, sz, vp]
    L.reduce_by_key_devn.restype = i32
    L.radix_sort_devn.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    L.radix_sort_devn.restype = i32
    L.select_compact_devn.argtypes = [vp, vp, vp, vp, vp, i64, sz, vp, sz, vp]
    L.select_compact_devn.restype = i32
    L.scan_status_str.argtypes = [i32]
    L.scan_status_str.restype = ctypes.c_char_p
    L.scan_last_hip_error.argtypes = []
    L.scan_last_hip_error.restype = i32
    return L


def check(status):
    """Map a scan_status to a Python exception (ValueError / NotImplementedError / ScanError)."""
    if status == 0:
        return
    msg = f"{_STATUS.get(status, status)}: {lib().scan_status_str(status).decode()}"
    if status == 2:
        raise NotImplementedError(msg)
    if status == 5:
        raise ScanError(f"{msg} (hipError_t {lib().scan_last_hip_error()})")
    raise ValueError(msg)


def _torch():
    import torch
    return torch


def dtype_name(dt):
    torch = _torch()
    table = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
             torch.float64: "f64", torch.int32: "i32", torch.int64: "i64"}
    for name in ("uint32", "uint64"):
        t = getattr(torch, name, None)
        if t is not None:
            table[t] = "u" + name[4:]
    if dt not in table:
        raise NotImplementedError(f"dtype {dt} is not supported")
    return table[dt]


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, what):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_SIZES = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8, "i32": 4, "u32": 4, "i64": 8, "u64": 8}


def _name(x, dtype):
    """Element type name: ``dtype`` if given (e.g. "u32" over an int32 tensor), else x's."""
    if dtype is None:
        return dtype_name(x.dtype)
    if dtype not in _SIZES:
        raise NotImplementedError(f"dtype {dtype!r} is not supported")
    if x.element_size() != _SIZES[dtype]:
        raise ValueError(f"dtype {dtype!r} does not match the tensor's element size")
    return dtype


def scan_rows(x, op="add", exclusive=False, out=None, stream=None, dtype=None):
    """Row-wise scan along the last axis of ``x`` (viewed as ``[rows, n]``)."""
    torch = _torch()
    n = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // n if n else 0
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    check(lib().scan_rows(_dev_ptr(x, "x"), _dev_ptr(out, "out"), rows, n,
                          DTYPE_CODES[_name(x, dtype)], OP_CODES[op], int(bool(exclusive)),
                          _stream(stream)))
    return out


def scan_device_scratch_bytes(n, dtype):
    name = dtype if isinstance(dtype, str) else dtype_name(dtype)
    return int(lib().scan_device_scratch_bytes(int(n), DTYPE_CODES[name]))


def _live(n_live, device):
    """The device count of a *_devn call: a 1-element int32 GPU tensor."""
    torch = _torch()
    if n_live.numel() != 1 or n_live.dtype != torch.int32 or n_live.device != device:
        raise ValueError("n_live must be a 1-element int32 tensor on the data's device")
    return _dev_ptr(n_live, "n_live")


def scan_device(x, op="add", out=None, scratch=None, stream=None, dtype=None, n_live=None):
    """Device-wide exclusive scan of the 1-D tensor ``x`` (of its first ``n_live[0]``
    elements when ``n_live`` is given: the count is then read on the device)."""
    L = lib()
    fn = L.scan_device if n_live is None else L.scan_device_devn
    return _scan_device(fn, x, op, out, scratch, stream, dtype, n_live)


def scan_device_noalloc(x, op="add", out=None, stream=None, dtype=None):
    """scan_device with the library's static per-GPU scratch (the C entry point
    allocates nothing; calls overlapping on one GPU race)."""
    torch = _torch()
    if x.dim() != 1:
        raise ValueError("x must be 1-D")
    name = _name(x, dtype)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    check(lib().scan_device_noalloc(_dev_ptr(x, "x"), _dev_ptr(out, "out"), x.shape[0],
                                    DTYPE_CODES[name], OP_CODES[op], _stream(stream)))
    return out


def scan_device_inclusive(x, op="add", out=None, scratch=None, stream=None, dtype=None,
                          n_live=None):
    """Device-wide inclusive scan of the 1-D tensor ``x`` (``n_live`` as for scan_device)."""
    L = lib()
    fn = L.scan_device_inclusive if n_live is None else L.scan_device_inclusive_devn
    return _scan_device(fn, x, op, out, scratch, stream, dtype, n_live)


def _scan_device(fn, x, op, out, scratch, stream, dtype, n_live):
    torch = _torch()
    if x.dim() != 1:
        raise ValueError("x must be 1-D")
    n = x.shape[0]
    name = _name(x, dtype)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    need = scan_device_scratch_bytes(n, name)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    count = (n,) if n_live is None else (_live(n_live, x.device), n)
    check(fn(_dev_ptr(x, "x"), _dev_ptr(out, "out"), *count, DTYPE_CODES[name], OP_CODES[op],
             _dev_ptr(scratch, "scratch"), scratch.numel(), _stream(stream)))
    return out


def reduce_device_scratch_bytes(n, dtype):
    name = dtype if isinstance(dtype, str) else dtype_name(dtype)
    return int(lib().reduce_device_scratch_bytes(int(n), DTYPE_CODES[name]))


def reduce_device(x, op="add", out=None, scratch=None, stream=None, dtype=None, n_live=None):
    """Device-wide reduction of the 1-D tensor ``x`` into ``out`` (1 element, on the GPU);
    ``n_live`` as for scan_device."""
    torch = _torch()
    if x.dim() != 1:
        raise ValueError("x must be 1-D")
    n = x.shape[0]
    name = _name(x, dtype)
    if out is None:
        out = torch.empty(1, dtype=x.dtype, device=x.device)
    if out.numel() != 1 or out.dtype != x.dtype:
        raise ValueError("out must be one element of x's dtype")
    need = reduce_device_scratch_bytes(n, name)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    L = lib()
    fn = L.reduce_device if n_live is None else L.reduce_device_devn
    count = (n,) if n_live is None else (_live(n_live, x.device), n)
    check(fn(_dev_ptr(x, "x"), _dev_ptr(out, "out"), *count, DTYPE_CODES[name], OP_CODES[op],
             _dev_ptr(scratch, "scratch"), scratch.numel(), _stream(stream)))
    return out


def reduce_by_key_scratch_bytes(n):
    return int(lib().reduce_by_key_scratch_bytes(int(n)))


def reduce_by_key(keys, values, keys_out=None, values_out=None, num_runs=None, scratch=None,
                  stream=None, key_dtype=None, value_dtype=None, n_live=None):
    """Collapse runs of equal consecutive keys of the 1-D ``keys`` into (first key, sum of
    ``values``).  Returns ``(keys_out, values_out, num_runs)``; ``num_runs`` is a 1-element
    int32 GPU tensor and only the first ``num_runs`` entries of the outputs are written."""
    torch = _torch()
    if keys.dim() != 1 or values.dim() != 1 or keys.shape[0] != values.shape[0]:
        raise ValueError("keys and values must be 1-D of the same length")
    n = keys.shape[0]
    kd, vd = _name(keys, key_dtype), _name(values, value_dtype)
    if keys_out is None:
        keys_out = torch.empty_like(keys)
    if values_out is None:
        values_out = torch.empty_like(values)
    if keys_out.numel() < n or values_out.numel() < n or keys_out.dtype != keys.dtype or \
            values_out.dtype != values.dtype:
        raise ValueError("outputs must hold n elements of the inputs' dtypes")
    if num_runs is None:
        num_runs = torch.empty(1, dtype=torch.int32, device=keys.device)
    need = reduce_by_key_scratch_bytes(n)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=keys.device)
    L = lib()
    fn = L.reduce_by_key if n_live is None else L.reduce_by_key_devn
    count = (n,) if n_live is None else (_live(n_live, keys.device), n)
    check(fn(_dev_ptr(keys, "keys"), _dev_ptr(values, "values"), _dev_ptr(keys_out, "keys_out"),
             _dev_ptr(values_out, "values_out"), _dev_ptr(num_runs, "num_runs"), *count,
             DTYPE_CODES[kd], DTYPE_CODES[vd], _dev_ptr(scratch, "scratch"), scratch.numel(),
             _stream(stream)))
    return keys_out, values_out, num_runs


def radix_sort_scratch_bytes(n, key_dtype):
    name = key_dtype if isinstance(key_dtype, str) else dtype_name(key_dtype)
    return int(lib().radix_sort_scratch_bytes(int(n), DTYPE_CODES[name]))


def radix_sort(keys, values=None, tmp_keys=None, tmp_values=None, end_bit=None, scratch=None,
               stream=None, key_dtype=None, value_dtype=None, n_live=None):
    """Stable ascending radix sort of the 1-D ``keys`` in place (``values`` in place
    alongside).  Returns ``(keys, values)``."""
    torch = _torch()
    if keys.dim() != 1:
        raise ValueError("keys must be 1-D")
    n = keys.shape[0]
    kd = _name(keys, key_dtype)
    if end_bit is None:
        end_bit = 8 * keys.element_size()
    if tmp_keys is None:
        tmp_keys = torch.empty_like(keys)
    vd = 0
    vptr = tvptr = None
    if values is not None:
        if values.dim() != 1 or values.shape[0] != n:
            raise ValueError("values must be 1-D with one value per key")
        vd = DTYPE_CODES[_name(values, value_dtype)]
        if tmp_values is None:
            tmp_values = torch.empty_like(values)
        vptr, tvptr = _dev_ptr(values, "values"), _dev_ptr(tmp_values, "tmp_values")
    need = radix_sort_scratch_bytes(n, kd)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=keys.device)
    L = lib()
    fn = L.radix_sort if n_live is None else L.radix_sort_devn
    count = (n,) if n_live is None else (_live(n_live, keys.device), n)
    check(fn(_dev_ptr(keys, "keys"), _dev_ptr(tmp_keys, "tmp_keys"), vptr, tvptr, *count,
             DTYPE_CODES[kd], vd, int(end_bit), _dev_ptr(scratch, "scratch"), scratch.numel(),
             _stream(stream)))
    return keys, values


def select_compact_scratch_bytes(n):
    return int(lib().select_compact_scratch_bytes(int(n)))


def select_compact(x, flags, out=None, num_out=None, scratch=None, stream=None, n_live=None):
    """Stable compaction of the 1-D tensor ``x`` by nonzero uint8 ``flags``.

    Returns ``(out, num_out)``; ``num_out`` is a 1-element int32 GPU tensor
    (read it with ``.item()``, which synchronizes).
    """
    torch = _torch()
    if x.dim() != 1 or flags.dim() != 1 or flags.shape[0] != x.shape[0]:
        raise ValueError("x and flags must be 1-D of the same length")
    if flags.dtype != torch.uint8:
        raise ValueError("flags must be uint8")
    n = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if out.numel() < n or out.dtype != x.dtype:
        raise ValueError("out must hold n elements of x's dtype")
    if num_out is None:
        num_out = torch.empty(1, dtype=torch.int32, device=x.device)
    need = select_compact_scratch_bytes(n)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    L = lib()
    fn = L.select_compact if n_live is None else L.select_compact_devn
    count = (n,) if n_live is None else (_live(n_live, x.device), n)
    check(fn(_dev_ptr(x, "x"), _dev_ptr(flags, "flags"), _dev_ptr(out, "out"),
             _dev_ptr(num_out, "num_out"), *count, x.element_size(),
             _dev_ptr(scratch, "scratch"), scratch.numel(), _stream(stream)))
    return out, num_out

"""Helpers shared by the GPU test modules: host <-> device transfers in the
oracle's storage types, seeded inputs, and the size lists that cover the
kernels' launch-shape boundaries."""
import sys

import numpy as np
import torch

import oracle
import workloads


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


STORE_T = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "f64": torch.float64, "i32": torch.int32, "u32": torch.int32, "i64": torch.int64,
           "u64": torch.int64}


def to_dev(a, dt):
    """numpy storage array -> GPU tensor (bf16/f16 bits reinterpret; u32/u64 ride in int32/int64)."""
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    if dt == "f16":
        return torch.from_numpy(a.view(np.float16).copy()).cuda()
    if dt in ("u32", "u64"):
        return torch.from_numpy(a.view(np.int32 if dt == "u32" else np.int64).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def from_dev(t, dt):
    t = t.cpu()
    if dt in ("bf16", "f16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    a = t.numpy()
    if dt == "u32":
        return a.view(np.uint32)
    if dt == "u64":
        return a.view(np.uint64)
    return a


def rand_input(dt, shape, seed):
    rng = np.random.default_rng(seed)
    if dt in ("f32", "f64"):
        return rng.uniform(-1, 1, size=shape).astype(oracle.STORAGE[dt])
    if dt == "bf16":
        return workloads.normal_bf16(shape, seed)
    if dt == "f16":
        return workloads.to_f16_bits(rng.standard_normal(size=shape).astype(np.float32))
    info = np.iinfo(oracle.STORAGE[dt])
    # full-range integers: add scans wrap
    return rng.integers(info.min, info.max, size=shape, dtype=oracle.STORAGE[dt], endpoint=True)


# covers every launch-shape boundary of the row kernel for 4- and 2-byte
# elements (rows touching 64, 256, 320, 512, 768, 1024 and 1280 16-byte
# vectors, with and without the line of slack that windows starting on a
# 128-byte line add) and rows long enough to take several chunks
ROW_SHAPES = [(1, 1), (1, 2), (3, 3), (3, 5), (1, 63), (3, 64), (5, 65), (2, 250), (3, 251),
              (3, 255), (3, 256), (3, 257), (2, 498), (3, 499), (2, 511), (3, 513), (2, 1018),
              (3, 1019), (2, 1023), (2, 1024), (3, 1025), (2, 2034), (3, 2035), (2, 2047),
              (3, 2049), (2, 4090), (3, 4091), (2, 4351), (2, 4352), (3, 4353), (2, 5114),
              (3, 5115), (2, 8178), (3, 8179), (2, 8703), (2, 8704), (3, 8705), (2, 10226),
              (3, 10227), (2, 20000), (3, 50001), (7, 333), (33, 100), (3, 4096), (3, 5120),
              (3, 8192), (2, 10240), (2, 16384), (3, 1249), (3, 1253), (2, 1277), (3, 1281),
              (3, 2017), (2, 2045), (3, 2053), (3, 3041), (2, 3069), (3, 3077), (3, 2497),
              (2, 2553), (3, 2569), (3, 4041), (2, 4093), (3, 4105), (3, 6089), (2, 6141),
              (3, 6153)]


DEV_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 8191, 8192, 8193,
             16383, 16384, 16385, 2 * 16384 + 37, 300_001, 1_000_003, 1_500_001]

"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds random-number generation only: none of the scan or
compaction arithmetic lives here, and it imports neither the oracle nor the
HIP library.  Every generator is numpy ``default_rng(seed)`` (PCG64); bf16
inputs are drawn in float32 and rounded to bf16 by torch's CPU conversion.

The five workloads (sizes, distributions and seeds):

1. row-wise inclusive and exclusive add scan, fp32 ``[1024, 4096]``,
   uniform [-1, 1), seed 0 (the benchmark shape of metaltile-std
   ``src/mlx/scan.rs``);
2. row-wise exclusive add scan, bf16 ``[8192, 8192]`` N(0, 1), seed 1, and the
   ragged ``[8192, 8191]`` (seed 1, drawn separately);
3. device-wide exclusive add scan, i32 uniform integers in [0, 15], seed 2,
   n = 2^28 and n = 2^28 - 37 (the first 2^28 - 37 values of the same draw);
4. device-wide exclusive min and max scans, f32 uniform [-1e6, 1e6), seed 3,
   n = 2^27, and i64 uniform over the full range, seed 4, n = 2^26;
5. select: f32 payload uniform [0, 1), seed 5, n = 2^28, and u8 flags
   Bernoulli(p), p in {0.01, 0.5, 0.99}, seed 6 + floor(100 p).

Beyond the five: the product scans run on the row shapes of workloads 1 and 2
with factors +-(1 + U[-1/64, 1/64)) (random sign), seed 11 for fp32 and 12
for bf16, so that 8192-long products neither overflow nor underflow; the
device-wide inclusive scans and the reductions reuse the inputs of workloads
3 and 4 (plus an f32 add reduction of workload 4's f32 input); reduce-by-key
runs on n = 2^27 i32 keys in runs of geometric length with mean 8 (each run's
key uniform in [0, 2^20), seed 13) and f32 values uniform [0, 1) (seed 14);
the radix sort on n = 2^28 u32 keys uniform over all 2^32 values (seed 15),
keys only and with i32 values (each key's original index).
"""
import numpy as np

SEEDS = {"rows_f32": 0, "rows_bf16": 1, "dev_i32": 2, "dev_f32": 3, "dev_i64": 4,
         "sel_payload": 5, "prod_f32": 11, "prod_bf16": 12, "rbk_keys": 13, "rbk_values": 14,
         "sort_keys": 15}

FULL = {
    "rows_f32": (1024, 4096),
    "rows_bf16": (8192, 8192),
    "rows_bf16_ragged": (8192, 8191),
    "dev_i32": 1 << 28,
    "dev_i32_odd": (1 << 28) - 37,
    "dev_f32": 1 << 27,
    "dev_i64": 1 << 26,
    "sel": 1 << 28,
    "rbk": 1 << 27,
    "sort": 1 << 28,
}
RBK_MEAN_RUN = 8
SELECT_P = (0.01, 0.5, 0.99)


def flags_seed(p):
    return 6 + int(np.floor(100 * p + 1e-9))


def uniform_f32(shape, seed, lo=-1.0, hi=1.0):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def normal_f32(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_bf16_bits(x_f32):
    """float32 array -> bf16 bit patterns (uint16), rounded by torch on the CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x_f32):
    """float32 array -> IEEE binary16 bit patterns (uint16), rounded by numpy."""
    with np.errstate(over="ignore"):
        return np.asarray(x_f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bf16(shape, seed):
    return to_bf16_bits(normal_f32(shape, seed))


def uniform_ints(n, lo, hi, seed, dtype=np.int32):
    """Uniform integers in [lo, hi] (both ends included)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=n, dtype=dtype, endpoint=True)


def full_range_ints(n, seed, dtype=np.int64):
    info = np.iinfo(dtype)
    rng = np.random.default_rng(seed)
    return rng.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True)


def bernoulli_flags(n, p, seed):
    rng = np.random.default_rng(seed)
    return (rng.random(size=n, dtype=np.float32) < np.float32(p)).astype(np.uint8)


def near_one_f32(shape, seed):
    """Factors +-(1 + U[-1/64, 1/64)) with a random sign, as float32."""
    rng = np.random.default_rng(seed)
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), size=shape)
    mag = rng.uniform(1 - 1 / 64, 1 + 1 / 64, size=shape).astype(np.float32)
    return sign * mag


def payload_f32(n, seed):
    rng = np.random.default_rng(seed)
    return rng.random(size=n, dtype=np.float32)


# ---- the named workloads -------------------------------------------------------

def rows_f32(rows=1024, n=4096, seed=SEEDS["rows_f32"]):
    return uniform_f32((rows, n), seed)


def rows_bf16(rows=8192, n=8192, seed=SEEDS["rows_bf16"]):
    return normal_bf16((rows, n), seed)


def dev_i32(n=FULL["dev_i32"], seed=SEEDS["dev_i32"]):
    return uniform_ints(n, 0, 15, seed, np.int32)


def dev_f32(n=FULL["dev_f32"], seed=SEEDS["dev_f32"]):
    return uniform_f32(n, seed, -1e6, 1e6)


def dev_i64(n=FULL["dev_i64"], seed=SEEDS["dev_i64"]):
    return full_range_ints(n, seed, np.int64)


def sel_inputs(n=FULL["sel"], p=0.5, seed=SEEDS["sel_payload"]):
    return payload_f32(n, seed), bernoulli_flags(n, p, flags_seed(p))


def prod_rows_f32(rows=1024, n=4096, seed=SEEDS["prod_f32"]):
    return near_one_f32((rows, n), seed)


def prod_rows_bf16(rows=8192, n=8192, seed=SEEDS["prod_bf16"]):
    return to_bf16_bits(near_one_f32((rows, n), seed))


def run_keys(n, mean_run, seed, key_range=1 << 20):
    """n int32 keys in runs of geometric length (mean `mean_run`), each run's key
    uniform in [0, key_range)."""
    rng = np.random.default_rng(seed)
    lengths = rng.geometric(1.0 / mean_run, size=int(n / mean_run * 1.1) + 64)
    while lengths.sum() < n:
        lengths = np.concatenate([lengths, rng.geometric(1.0 / mean_run, size=lengths.size)])
    return np.repeat(rng.integers(0, key_range, size=lengths.size).astype(np.int32), lengths)[:n]


def rbk_inputs(n=FULL["rbk"]):
    keys = run_keys(n, RBK_MEAN_RUN, SEEDS["rbk_keys"])
    return keys, payload_f32(n, SEEDS["rbk_values"])


def sort_keys_u32(n=FULL["sort"], seed=SEEDS["sort_keys"]):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)

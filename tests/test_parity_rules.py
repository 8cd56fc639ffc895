"""CPU checks of the GPU-vs-oracle comparison rules themselves (tests/parity.py):
each accepts a result computed the way the GPU legitimately may (float32
accumulation in another order) and rejects one with a plausible mistake (a
dropped term or factor, a shifted prefix)."""
import numpy as np

import oracle
import workloads
from parity import check_fp_add, check_fp_mul, check_stable_by_image


def _raises(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_fp_add_rule_accepts_float32_order_and_rejects_a_dropped_term():
    x = workloads.uniform_f32((4, 4096), 3)
    ora, ref, absref = oracle.scan(x, "f32", "add", want_ref=True)
    # float32 pairwise-in-blocks accumulation: another legitimate grouping
    blocks = x.reshape(4, 64, 64)
    within = np.cumsum(blocks, axis=2, dtype=np.float32)
    carry = np.concatenate([np.zeros((4, 1), np.float32),
                            np.cumsum(within[:, :-1, -1], axis=1, dtype=np.float32)], axis=1)
    gpu_like = (within + carry[:, :, None]).reshape(4, 4096).astype(np.float32)
    check_fp_add(gpu_like, ora, ref, absref, "f32", "regrouped")
    bad = gpu_like.copy()
    bad[:, 100:] -= x[:, 100:101]                   # one term dropped from every later prefix
    assert _raises(lambda: check_fp_add(bad, ora, ref, absref, "f32", "dropped"))
    shifted = np.concatenate([np.zeros((4, 1), np.float32), gpu_like[:, :-1]], axis=1)
    assert _raises(lambda: check_fp_add(shifted, ora, ref, absref, "f32", "shifted"))


def test_bf16_add_rule_accepts_float32_order():
    x = workloads.rows_bf16(4, 4096, seed=9)
    ora, ref, absref = oracle.scan(x, "bf16", "add", exclusive=True, want_ref=True)
    xf = workloads_bf16_to_f32(x)
    inc = np.cumsum(xf, axis=1, dtype=np.float32)
    exc = np.concatenate([np.zeros((4, 1), np.float32), inc[:, :-1]], axis=1)
    check_fp_add(workloads.to_bf16_bits(exc), ora, ref, absref, "bf16", "float32 sequential")
    bad = exc.copy()
    bad[:, 2000:] += 0.25
    assert _raises(lambda: check_fp_add(workloads.to_bf16_bits(bad), ora, ref, absref, "bf16",
                                        "offset"))


def workloads_bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_fp_mul_rule_accepts_float32_products_and_rejects_a_dropped_factor():
    x = workloads.prod_rows_f32(4, 8192, seed=21)
    _, ref, _ = oracle.scan(x, "f32", "mul", want_ref=True)
    m = np.broadcast_to(np.arange(1, 8193), x.shape)
    seq = np.multiply.accumulate(x, axis=1, dtype=np.float32)      # 8191 float32 roundings
    check_fp_mul(seq, ref, m, "f32", "float32 sequential")
    bad = seq.copy()
    bad[:, 4000:] /= x[:, 4000:4001]                # one factor dropped from every later prefix
    assert _raises(lambda: check_fp_mul(bad, ref, m, "f32", "dropped"))
    # the same in bf16: the float32 products rounded once
    xb = workloads.prod_rows_bf16(4, 8192, seed=22)
    _, refb, _ = oracle.scan(xb, "bf16", "mul", exclusive=True, want_ref=True)
    xf = workloads_bf16_to_f32(xb)
    inc = np.multiply.accumulate(xf, axis=1, dtype=np.float32)
    exc = np.concatenate([np.ones((4, 1), np.float32), inc[:, :-1]], axis=1)
    mb = np.broadcast_to(np.arange(0, 8192), xb.shape)
    check_fp_mul(workloads.to_bf16_bits(exc), refb, mb, "bf16", "bf16 sequential")
    badb = exc.copy()
    badb[:, 3000:] /= xf[:, 3000:3001]
    assert _raises(lambda: check_fp_mul(workloads.to_bf16_bits(badb), refb, mb, "bf16", "dropped"))


def test_stable_order_rule_accepts_the_oracle_sort_and_rejects_mistakes():
    rng = np.random.default_rng(31)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 2.5], np.float32)
    cases = [(rng.integers(0, 5, size=3000).astype(np.uint32), "u32"),
             (rng.integers(-(1 << 63), (1 << 63) - 1, size=3000, dtype=np.int64), "i64"),
             (specials[rng.integers(0, specials.size, size=3000)], "f32")]
    for keys, dt in cases:
        ok, ov = oracle.sort(keys, dt, np.arange(keys.size, dtype=np.int64))
        check_stable_by_image(keys, ok, ov, dt, f"oracle sort {dt}")
        # two equal-image neighbours in the wrong order (stability broken)
        img = oracle.sort_image(ok, dt)
        ties = np.flatnonzero(img[1:] == img[:-1])
        if ties.size:
            i = int(ties[0])
            bk, bv = ok.copy(), ov.copy()
            bk[[i, i + 1]], bv[[i, i + 1]] = bk[[i + 1, i]], bv[[i + 1, i]]
            assert _raises(lambda: check_stable_by_image(keys, bk, bv, dt, "tie swapped"))
        # a key that does not travel with its index
        bk = ok.copy()
        bk[[0, -1]] = bk[[-1, 0]]
        assert _raises(lambda: check_stable_by_image(keys, bk, ov, dt, "key moved alone"))
        # an index repeated (not a permutation)
        bv = ov.copy()
        bv[1] = bv[0]
        assert _raises(lambda: check_stable_by_image(keys, ok, bv, dt, "index repeated"))
        # keys in descending image order, carried consistently
        assert _raises(lambda: check_stable_by_image(keys, ok[::-1].copy(), ov[::-1].copy(), dt,
                                                     "reversed"))

"""Pins of the CPU oracle for the temperature draw of the accept step.

Generator: Philox4x64-10 against numpy's own implementation of it (an independent
library routine).  Draw: frequencies over many rows against softmax(logits / T) (the
Gumbel-max identity, here in base-2 form), the T -> 0 limit, -inf entries, and planted
mistakes.
"""
import inspect
import types

import numpy as np
import pytest

from oracle import ddtree_f32 as D
from oracle import sample_f32 as S


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)), ((123, 456), (7, 8, 9, 10)),
                                     ((2**64 - 1, 2**63 + 5), (2**64 - 2, 1, 2**40, 3))])
def test_philox_matches_numpy(key, ctr):
    g = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
    raw = g.random_raw(12)
    for blk in range(3):  # numpy produces block k from counter + 1 + k
        c0 = (ctr[0] + 1 + blk) % 2**64
        carry = (ctr[0] + 1 + blk) // 2**64
        c = (c0, ctr[1] + carry, ctr[2], ctr[3])
        mine = S.philox4x64_10(tuple(np.array([v], np.uint64) for v in c), key)
        assert [int(w[0]) for w in mine] == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_uniforms_open_interval_and_layout():
    u = S.uniforms(3, 4096, seed=11, offset=5)
    assert u.dtype == np.float32 and (u > 0).all() and (u < 1).all()
    # entries 8k .. 8k+7 come from one generator block: the same counter (k, row)
    x = S.philox4x64_10((np.array([2], np.uint64), np.array([3], np.uint64),
                         np.array([0], np.uint64), np.array([0], np.uint64)), (11, 5))
    for j in range(8):
        x32 = (int(x[j // 2][0]) >> (32 * (j % 2))) & 0xFFFFFFFF
        assert u[16 + j] == np.float32(((x32 >> 9) * 2 + 1) * 2.0 ** -24)
    assert abs(float(u.mean()) - 0.5) < 0.02


@pytest.mark.parametrize("temperature", [0.5, 1.0, 2.0])
def test_frequencies_follow_softmax(temperature):
    logits = np.array([1.0, 0.2, -0.5, 2.0, -3.0, 0.0], np.float32)
    rows = 20000
    tok = S.sample_tokens(np.tile(logits, (rows, 1)), temperature, seed=7, offset=int(temperature * 10))
    counts = np.bincount(tok, minlength=6).astype(np.float64)
    p = np.exp(logits.astype(np.float64) / temperature)
    p /= p.sum()
    expected = rows * p
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 30.0, (chi2, counts, expected)  # 5 dof: p(chi2 > 30) ~ 1.5e-5


def test_zero_temperature_is_argmax_and_small_temperature_converges():
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 3, size=(50, 1000)).astype(np.float32)
    np.testing.assert_array_equal(S.sample_tokens(logits, 0.0, 1, 2), np.argmax(logits, axis=1))
    gap = np.sort(logits, axis=1)[:, -1] - np.sort(logits, axis=1)[:, -2]
    ok = gap > 1e-2  # T = 1e-4 turns a gap of 1e-2 into 100, beyond any Gumbel variate here
    got = S.sample_tokens(logits, 1e-4, 1, 2)
    np.testing.assert_array_equal(got[ok], np.argmax(logits, axis=1)[ok])


def test_masked_entries_never_drawn_and_all_masked_row():
    logits = np.full((300, 8), -np.inf, np.float32)
    logits[:, [2, 5]] = 0.0
    logits[-1] = -np.inf
    tok = S.sample_tokens(logits, 1.0, 9, 0)
    assert set(tok[:-1].tolist()) == {2, 5} and tok[-1] == -1
    assert S.sample_tokens(logits, 0.0, 9, 0)[-1] == -1


def test_seed_and_offset_change_the_draw():
    logits = np.zeros((200, 64), np.float32)
    a = S.sample_tokens(logits, 1.0, 1, 0)
    assert (a != S.sample_tokens(logits, 1.0, 2, 0)).mean() > 0.9
    assert (a != S.sample_tokens(logits, 1.0, 1, 1)).mean() > 0.9
    np.testing.assert_array_equal(a, S.sample_tokens(logits, 1.0, 1, 0))


def test_temperature_walk_reduces_to_greedy_at_zero():
    """The temperature accept is the greedy walk fed with drawn tokens."""
    rng = np.random.default_rng(5)
    lp = -np.sort(-rng.random((6, 3)).astype(np.float32), axis=1)
    ids = np.arange(18, dtype=np.int32).reshape(6, 3)
    t = D.build_ddtree(np.log(lp), ids, 99, 12)
    n = len(t["parent"])
    logits = rng.normal(size=(n, 18)).astype(np.float32)
    for i in range(n):  # make the target favour one child where there is one
        kids = [c for c in range(n) if t["parent"][c] == i]
        if kids:
            logits[i, t["token"][kids[0]]] += 5.0
    drawn = S.sample_tokens(logits, 0.0, 0, 0)
    assert D.tree_accept(t["token"], t["first_child"], t["next_sibling"], drawn) == \
        D.tree_accept(t["token"], t["first_child"], t["next_sibling"], np.argmax(logits, 1))


def _mutant(old, new):
    src = inspect.getsource(S)
    assert src.count(old) == 1, old
    mod = types.ModuleType("sample_mutant")
    exec(compile(src.replace(old, new), "sample_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("(lg * c)", "(lg * np.float32(temperature))"),               # T applied the wrong way
    ("g = log2_f32(-log2_f32(u))", "g = -log2_f32(-log2_f32(u))"),   # Gumbel sign flipped
    ("g = log2_f32(-log2_f32(u))", "g = log2_f32(u)"),               # not a Gumbel variate
    ("LOG2_SERIES = [np.float32(2.0 / ((2 * k + 1) * np.log(2.0))) for k in range(5)]",
     "LOG2_SERIES = [np.float32(2.0 / ((2 * k + 1) * np.log(10.0))) for k in range(5)]"),
    # a logarithm of the wrong base: keys scaled, so softmax(logit / T) no longer holds
    ("np.float32(LOG2E) / np.float32(temperature)",
     "np.float32(1.0) / np.float32(temperature)"),               # base mismatch
])
def test_planted_mistakes_fail_the_frequency_pin(old, new):
    mod = _mutant(old, new)
    logits = np.array([1.0, 0.2, -0.5, 2.0, -3.0, 0.0], np.float32)
    rows, temperature = 20000, 0.5
    tok = mod.sample_tokens(np.tile(logits, (rows, 1)), temperature, seed=7, offset=5)
    counts = np.bincount(tok, minlength=6).astype(np.float64)
    p = np.exp(logits.astype(np.float64) / temperature)
    p /= p.sum()
    chi2 = float(((counts - rows * p) ** 2 / (rows * p)).sum())
    assert chi2 > 30.0


def test_planted_generator_mistake_fails_the_numpy_pin():
    mod = _mutant("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0",
                  "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k0, lo0")
    g = np.random.Philox(key=np.array([123, 456], np.uint64), counter=np.array([7, 8, 9, 10], np.uint64))
    raw = g.random_raw(4)
    mine = mod.philox4x64_10(tuple(np.array([v], np.uint64) for v in (8, 8, 9, 10)), (123, 456))
    assert [int(w[0]) for w in mine] != [int(x) for x in raw]


# ------------------------------------------------------------------ the float32 logarithm
def test_log2_f32_accuracy_and_exact_points():
    """The draw's float32 base-2 logarithm (a fixed sequence of rounded float32 operations,
    which the GPU evaluates the same way) against float64 log2: within 3 ulp of the result
    over 30 binades of random values and all powers of two, within 3e-7 relative on (0.5, 1)
    where -log2(u) near 0 decides the argmax, exact at powers of two."""
    rng = np.random.default_rng(900)
    x = np.concatenate([(2.0 ** rng.uniform(-126, 127, 400000)).astype(np.float32),
                        rng.uniform(0.5, 1.0, 200000).astype(np.float32),
                        (1.0 - np.arange(1, 30000) * 2.0 ** -24).astype(np.float32),
                        (1.0 + np.arange(1, 30000) * 2.0 ** -23).astype(np.float32)])
    got = S.log2_f32(x).astype(np.float64)
    ref = np.log2(x.astype(np.float64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    nz = ref != 0
    assert (np.abs(got - ref)[nz] <= 3 * ulp[nz]).all()
    near = (x > 0.5) & (x < 1)
    assert (np.abs(got - ref)[near] <= 3e-7 * np.abs(ref[near])).all()
    k = np.arange(-126, 128)
    assert np.array_equal(S.log2_f32(np.float32(2.0) ** k.astype(np.float32)), k.astype(np.float32))
    assert S.log2_f32(np.float32(1.0)) == 0.0


def test_log2_f32_is_a_fixed_float32_sequence():
    """The steps are float32 operations in a fixed order: recomputing them one by one with
    Python floats rounded to float32 after every operation gives the same bits."""
    import struct

    def f32(v):
        return struct.unpack("f", struct.pack("f", v))[0]
    a = [float(c) for c in S.LOG2_SERIES]
    rng = np.random.default_rng(901)
    for x in (2.0 ** rng.uniform(-30, 30, 300)).astype(np.float32):
        bits = int(np.array(x).view(np.uint32))
        e = ((bits >> 23) & 0xFF) - 127
        mb = (bits & 0x7FFFFF) | 0x3F800000
        if mb > 0x3FB504F3:
            mb -= 0x800000
            e += 1
        m = struct.unpack("f", struct.pack("I", mb))[0]
        f = f32(m - 1.0)
        s = f32(f / f32(2.0 + f))
        z = f32(s * s)
        p = a[4]
        for c in (a[3], a[2], a[1], a[0]):
            p = f32(f32(p * z) + c)
        want = f32(float(e) + f32(s * p))
        assert float(S.log2_f32(x)) == want, float(x)


def test_gumbel_log2_error_bound_over_every_uniform():
    """Every uniform the draw can produce, u = (2k + 1) 2^-24 for k < 2^23: the fixed
    float32 evaluation of log2(-log2 u) stays within 5.2e-7 + 3 ulp of the exact value
    (float64), and that exact value falls as u rises.  The GPU's pruning test skips a
    block of 8 entries only when its keys are provably below the running best; its
    margin is built on this bound, so that pruning never changes a draw."""
    k = np.arange(2 ** 23, dtype=np.int64)
    u = ((2 * k + 1).astype(np.float64) * 2.0 ** -24).astype(np.float32)
    assert np.array_equal(u.astype(np.float64), (2 * k + 1) * 2.0 ** -24)  # exact in float32
    g = np.log2(-np.log2(u.astype(np.float64)))
    assert (np.diff(g) < 0).all()
    got = S.log2_f32(-S.log2_f32(u)).astype(np.float64)
    ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64)
    err = np.abs(got - g)
    assert (err <= 5.2e-7 + 3 * ulp).all(), float((err / (5.2e-7 + 3 * ulp)).max())

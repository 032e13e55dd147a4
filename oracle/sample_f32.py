"""CPU oracle for the temperature path of the accept step: drawing the target model's next
token at every tree node from softmax(logits / T).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path never
imports, calls or links anything here, and this module imports nothing from it.

The pages name a temperature rejection-sampling path of the accept step ("The Milestone
Commit: Cementing Phase 1 ...", sections "Why This Message Was Written" and "How
Decisions Were Made": production notes on the sampling path) without giving it.  The
reading taken: the drafted tree holds the drafter's top-k candidates, which are chosen,
not sampled, so a ratio test against the drafter's probabilities would not keep the
target's distribution.  The lossless rule is to draw the target's token at the current
node and follow the child that carries it, else end with the drawn token; that is the
greedy walk with drawn tokens in place of the argmax, and T = 0 is the greedy accept.
This module draws those tokens; the walk is ``ddtree_f32.tree_accept``.

Draw (T > 0), per row r and vocabulary entry i, all in float32 except the generator:
  x     = Philox4x64-10(counter = (i // 8, r, 0, 0), key = (seed, offset))  (Salmon et al.,
          "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), word (i // 2) % 4,
          low 32 bits for even i, high 32 bits for odd i
  u     = (2 * (x32 >> 9) + 1) * 2^-24, in (0, 1)
  c     = log2(e) / T                                    (float32 constants, rounded)
  z     = logit * c - L(-L(u))                           (each operation rounded)
  token = argmax_i z, lowest i on ties; -1 if every logit is -inf.
L is the float32 base-2 logarithm of ``log2_f32`` below, a fixed sequence of rounded
float32 operations, so that a GPU evaluating the same sequence draws the same tokens.
z is log2(e) times the Gumbel-max key logit / T - ln(-ln u), less the constant
log2(ln 2): the same argmax, so token ~ softmax(logit / T) (the Gumbel-max identity), with
base-2 logarithms throughout.  T = 0: token = argmax_i logit.
"""
from __future__ import annotations

import numpy as np

# Philox4x64 round multipliers and key increments, from the generator's definition
M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = np.uint64(0x9E3779B97F4A7C15)
W1 = np.uint64(0xBB67AE8584CAA73B)
LOG2E = np.float32(1.4426950408889634)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a: np.uint64, b: np.ndarray):
    """(high, low) 64-bit halves of the 128-bit products a * b (b an array), from
    32-bit limbs in uint64 arithmetic."""
    a_lo, a_hi = a & _LO, a >> _S32
    b_lo, b_hi = b & _LO, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO) + (hl & _LO)
    lo = (ll & _LO) | ((mid & _LO) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds.  ctr: 4 uint64 arrays (broadcastable), key: 2 uint64.
    Returns the 4 output words (uint64 arrays)."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(c, np.uint64) for c in ctr)
        k0, k1 = np.uint64(key[0]), np.uint64(key[1])
        for _ in range(10):
            hi0, lo0 = _mulhilo64(M0, c0)
            hi1, lo1 = _mulhilo64(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0 = k0 + W0
            k1 = k1 + W1
    return c0, c1, c2, c3


# log2(1 + f) = (2 / ln 2) atanh(s), s = f / (2 + f): the classical series
# ln z = 2 (s + s^3 / 3 + s^5 / 5 + ...) with s = (z - 1) / (z + 1), z = 1 + f, times log2(e).
# Coefficient k of the series in s^2 (float32): 2 / ((2k + 1) ln 2).
LOG2_SERIES = [np.float32(2.0 / ((2 * k + 1) * np.log(2.0))) for k in range(5)]
_SQRT2_BITS = np.uint32(0x3FB504F3)  # float32 sqrt(2), rounded


def log2_f32(x) -> np.ndarray:
    """Base-2 logarithm of positive normal float32 values as a fixed sequence of float32
    operations, each rounded to nearest (no fused multiply-add):
      x = 2^e m, m in [1, 2) from the bits; if m > sqrt(2): m = m / 2, e = e + 1 (exact);
      f = m - 1 (exact), s = f / (2 + f), z = s * s;
      p = ((((A4 z + A3) z + A2) z + A1) z + A0), A_k = 2 / ((2k + 1) ln 2);
      L = e + s * p.
    |s| <= 0.172, so the series' truncation after s^9 is below 2e-9 relative; the
    rounding keeps L within a few ulp of log2(x), and exact at powers of two."""
    xf = np.asarray(x, np.float32)
    bits = xf.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - np.int32(127)
    mbits = (bits & np.uint32(0x7FFFFF)) | np.uint32(0x3F800000)
    big = mbits > _SQRT2_BITS
    mbits = np.where(big, mbits - np.uint32(0x00800000), mbits).astype(np.uint32)
    e = np.where(big, e + 1, e)
    m = mbits.view(np.float32)
    f = (m - np.float32(1.0)).astype(np.float32)
    s = (f / (np.float32(2.0) + f).astype(np.float32)).astype(np.float32)
    z = (s * s).astype(np.float32)
    p = LOG2_SERIES[4]
    for a in (LOG2_SERIES[3], LOG2_SERIES[2], LOG2_SERIES[1], LOG2_SERIES[0]):
        p = ((p * z).astype(np.float32) + a).astype(np.float32)
    return (e.astype(np.float32) + (s * p).astype(np.float32)).astype(np.float32)


def uniforms(rows, vocab: int, seed: int, offset: int) -> np.ndarray:
    """u in (0, 1) (float32) for vocabulary entries 0..vocab-1 of the given row index(es):
    shape [vocab] for one row, [len(rows), vocab] for several."""
    r = np.asarray(rows, np.uint64)
    one = r.ndim == 0
    r = r.reshape(-1, 1)
    i = np.arange(vocab, dtype=np.uint64).reshape(1, -1)
    shape = (r.shape[0], vocab)
    words = philox4x64_10((np.broadcast_to(i >> np.uint64(3), shape), np.broadcast_to(r, shape),
                           np.zeros(shape, np.uint64), np.zeros(shape, np.uint64)),
                          (seed, offset))
    w = np.broadcast_to((i >> np.uint64(1)) & np.uint64(3), shape)
    x = np.select([w == np.uint64(k) for k in range(4)], list(words))
    x32 = np.where(np.broadcast_to((i & np.uint64(1)) == np.uint64(0), shape), x & _LO, x >> _S32)
    num = (x32 >> np.uint64(9)) * np.uint64(2) + np.uint64(1)
    u = (num.astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)
    return u[0] if one else u


def perturbed(logits: np.ndarray, temperature: float, rows, seed: int, offset: int):
    """z of the given rows (float32), as the module docstring defines it; logits holds
    those rows' values ([vocab] for one row index, [len(rows), vocab] for several)."""
    lg = np.asarray(logits, np.float32)
    c = np.float32(LOG2E) / np.float32(temperature)
    u = uniforms(rows, lg.shape[-1], seed, offset)
    g = log2_f32(-log2_f32(u))
    with np.errstate(invalid="ignore"):
        return (lg * c).astype(np.float32) - g


def sample_tokens(logits: np.ndarray, temperature: float, seed: int, offset: int,
                  rows_per_chunk: int = 64) -> np.ndarray:
    """Next token of every row of logits [rows, vocab] (float32 values) at temperature T."""
    lg = np.asarray(logits, np.float32)
    n = lg.shape[0]
    out = np.full(n, -1, np.int32)
    chunk = max(1, min(n, (1 << 22) // max(lg.shape[1], 1), rows_per_chunk * 1000))
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        z = lg[rows] if temperature == 0 else perturbed(lg[rows], temperature, rows, seed, offset)
        best = np.argmax(z, axis=1)  # first maximum: lowest index on ties
        dead = np.all(np.isneginf(z), axis=1)
        out[rows] = np.where(dead, -1, best).astype(np.int32)
    return out

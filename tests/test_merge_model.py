"""CPU checks of the reformulation the kernels compute, against the fp64 oracle.

The kernels never evaluate the textbook log-sum-exp of a row in one piece:
lanes, wavefronts, chunks and (for split rows) workgroups each keep a pair
(m, s) -- the largest logit they saw and the sum of exp(x - m) over their
elements -- and the pairs are merged with the associative rule of the
POPCORNBENCH "Kimi-K2.6 l1_p95" trace (online normalizer): M = max(m_a, m_b),
S = s_a exp(m_a - M) + s_b exp(m_b - M), a pair whose m is -inf contributing
0.  The first test checks, in fp64, that any split of a row into pieces
merged in any order reproduces the oracle's log-sum-exp (so the
reformulation is exact up to rounding).  The second runs a float32 model of
the streamed kernel's pass (chunked, base-2 exponentials, one rescale per
chunk, the target left out of the sum and added back) and checks that the
arithmetic alone stays inside the tolerance the GPU parity tests use for row
losses; it predicts the GPU's error budget and is not a check of the GPU.
"""
import math

import numpy as np
import pytest

import oracle
from softmax_cross_entropy_fwd_amd import inputs

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def merge(a, b):
    (ma, sa), (mb, sb) = a, b
    M = max(ma, mb)
    if M == -math.inf:
        return M, 0.0
    ra = 0.0 if ma == -math.inf else sa * math.exp(ma - M)
    rb = 0.0 if mb == -math.inf else sb * math.exp(mb - M)
    return M, ra + rb


def piece(x):
    m = float(np.max(x)) if x.size else -math.inf
    if m == -math.inf:
        return m, 0.0
    return m, float(np.sum(np.exp(x - m)))


def rows_with_structure(rng, M, V):
    x = rng.normal(0.0, 3.0, size=(M, V))
    x[rng.random((M, V)) < 0.05] = -np.inf
    x[0, : V // 2] = -np.inf          # a long -inf run: whole pieces of -inf
    x[1] = 2.5                        # all equal
    t = rng.integers(0, V, size=M)
    x[np.arange(M), t] = np.where(np.isinf(x[np.arange(M), t]), 0.25, x[np.arange(M), t])
    x[2, t[2]] = np.max(x[2]) + 30.0  # dominant target
    return x, t


@pytest.mark.parametrize("V", [1, 2, 7, 1000, 5003])
def test_lse_merge_any_split_and_order(V):
    rng = np.random.default_rng(V)
    x, t = rows_with_structure(rng, 6, V)
    # the oracle takes the stored float32 values
    xs = x.astype(np.float32)
    _, lse = oracle.loss_rows(xs, t, dtype="f32", with_lse=True)
    for i in range(xs.shape[0]):
        row = xs[i].astype(np.float64)
        for _ in range(20):
            cuts = np.sort(rng.choice(np.arange(1, V), size=min(V - 1, rng.integers(0, 9)),
                                      replace=False)) if V > 1 else []
            parts = [piece(p) for p in np.split(row, cuts)]
            rng.shuffle(parts)
            acc = (-math.inf, 0.0)
            for p in parts:
                acc = merge(acc, p) if rng.random() < 0.5 else merge(p, acc)
            got = acc[0] + math.log(acc[1])
            assert abs(got - lse[i]) <= 4e-15 * max(1.0, abs(lse[i])), (V, i, got, lse[i])


def fp32_stream_loss(row, t, chunk=1024):
    """float32 model of the streamed pass: per chunk, the running max takes
    every element, the running sum (base 2, rescaled once per chunk when the
    max grows) every element but the target's; the target's term is added
    back at the end."""
    f = np.float32
    x = row.astype(np.float32)
    xt = x[t]
    m_run, s_run = f(-np.inf), f(0.0)
    for c0 in range(0, x.size, chunk):
        c = x[c0:c0 + chunk].copy()
        cm = max(m_run, f(np.max(c)))
        if c0 <= t < c0 + chunk:
            c[t - c0] = -np.inf
        if cm != -np.inf:
            cmL = f(cm * f(LOG2E))
            add = f(np.sum(np.exp2(c * f(LOG2E) - cmL, dtype=np.float32), dtype=np.float32))
            scale = f(0.0) if m_run == -np.inf else f(np.exp2(f((m_run - cm) * f(LOG2E))))
            s_run = f(s_run * scale + add)
            m_run = cm
    m = m_run
    et = f(np.exp2(f(xt * f(LOG2E) - f(m * f(LOG2E)))))
    s = f(s_run + et)
    if et > f(0.5) * s:
        return float(f(np.log1p(f(s_run / et))))
    return float(f(f(m - xt) + f(f(LN2) * f(np.log2(s)))))


@pytest.mark.parametrize("name,rows", [("tiny", 64), ("classifier", 12), ("lmhead", 3),
                                       ("stress", 40), ("skinny", 400)])
def test_fp32_stream_model_within_row_loss_tolerance(name, rows):
    c = inputs.CONFIGS[name]
    x, t = inputs.make(c["dtype"], rows, c["V"], c["sigma"], c["seed"], c["structure"])
    xb, tn = inputs.host_bits(x), t.numpy()
    want = oracle.loss_rows(xb, tn, dtype=c["dtype"])
    w = (np.asarray(oracle.widen(xb.ravel(), c["dtype"]), dtype=np.float64).reshape(xb.shape)
         if c["dtype"] != "f32" else xb.astype(np.float64))
    for i in range(rows):
        got = fp32_stream_loss(w[i], int(tn[i]))
        m = float(np.max(w[i]))
        xt = float(w[i][tn[i]])
        ulp = float(np.spacing(np.float32(max(abs(m), abs(xt), 1.0))))
        bound = 1e-5 * abs(want[i]) + 4 * ulp
        assert abs(got - want[i]) <= bound, (name, i, got, want[i], bound)

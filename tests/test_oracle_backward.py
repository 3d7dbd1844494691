"""Pins for the oracle's backward pass (prefill_backward).

* automatic differentiation (torch, float64, CPU) of a forward written here
  independently, with the per-dim keep mask, for dense, grouped and exact
  tables, GQA ratios 1 and 2;
* central finite differences of <dO, O> on a tiny case where every tile
  class occurs."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _torch_forward(q, k, v, dim_cut):
    """Causal attention with per-dim keep masks, written directly in torch:
    S_ij = sum_d [i-j <= cut_d] q_id k_jd / sqrt(d); q [n, Hq, d]."""
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    dist = i - j
    keep = (dist[:, :, None] <= torch.as_tensor(np.asarray(dim_cut, dtype=np.int64))[None, None, :])
    outs = []
    for h in range(Hq):
        kv = h // r
        prod = q[:, h, None, :] * k[None, :, kv, :]                 # [n, n, d]
        S = (prod * keep).sum(-1) / math.sqrt(d)
        S = S.masked_fill(dist < 0, float("-inf"))
        outs.append(torch.softmax(S, dim=-1) @ v[:, kv, :])
    return torch.stack(outs, dim=1)


@pytest.mark.parametrize("n,Hq,Hkv,d,table", [
    (40, 2, 1, 16, "dense"),
    (40, 2, 2, 16, "grouped"),
    (33, 4, 2, 32, "grouped"),
    (29, 2, 1, 16, "exact"),
])
def test_backward_matches_autograd(n, Hq, Hkv, d, table):
    rng = np.random.default_rng(7 + n)
    q = rng.standard_normal((n, Hq, d))
    k = rng.standard_normal((n, Hkv, d))
    v = rng.standard_normal((n, Hkv, d))
    do = rng.standard_normal((n, Hq, d))
    theta = 50.0
    if table == "dense":
        cut = O.dim_cutoffs_dense(d)
    elif table == "exact":
        cut = O.dim_cutoffs_exact(theta, d)
    else:
        cut = O.dim_cutoffs_grouped(O.group_cutoffs(theta, d, 8), 8)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = _torch_forward(tq, tk, tv, cut)
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv = O.prefill_backward(q, k, v, do, cut)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)
    # the oracle's forward agrees with the torch forward too
    assert np.allclose(O.prefill(q, k, v, cut), out.detach().numpy(), rtol=1e-12, atol=1e-13)


def test_backward_finite_differences():
    n, Hq, Hkv, d = 12, 2, 1, 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((n, Hq, d))
    k = rng.standard_normal((n, Hkv, d))
    v = rng.standard_normal((n, Hkv, d))
    do = rng.standard_normal((n, Hq, d))
    cut = O.dim_cutoffs_grouped(O.group_cutoffs(30.0, d, 2), 2)     # cutoffs 4, 13, ...
    assert cut.min() < n - 1                                         # some terms truncated

    def loss(q_, k_, v_):
        return float((O.prefill(q_, k_, v_, cut) * do).sum())

    dq, dk, dv = O.prefill_backward(q, k, v, do, cut)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0, 0), (5, 0, 3), (11, Hq - 1 if arr is q else 0, 7), (7, 0, 1)]:
            a1 = arr.copy()
            a2 = arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = [a1 if arr is x else x for x in (q, k, v)]
            args2 = [a2 if arr is x else x for x in (q, k, v)]
            fd = (loss(*args1) - loss(*args2)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


@pytest.mark.parametrize("n,Hq,Hkv,d,table,key_from", [
    (40, 4, 1, 16, "grouped", 30),
    (33, 2, 2, 32, "exact", 20),
    (21, 2, 1, 16, "dense", 0),
])
def test_backward_rows_matches_autograd(n, Hq, Hkv, d, table, key_from):
    """prefill_backward_rows (the row-sampled backward used at full sizes)
    against torch autograd of the forward written above: dQ at scattered
    rows, dK and dV of the keys >= key_from from every row >= key_from."""
    rng = np.random.default_rng(11 + n)
    q = rng.standard_normal((n, Hq, d))
    k = rng.standard_normal((n, Hkv, d))
    v = rng.standard_normal((n, Hkv, d))
    do = rng.standard_normal((n, Hq, d))
    theta = 40.0
    if table == "dense":
        cut = O.dim_cutoffs_dense(d)
    elif table == "exact":
        cut = O.dim_cutoffs_exact(theta, d)
    else:
        cut = O.dim_cutoffs_grouped(O.group_cutoffs(theta, d, 8), 8)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    (_torch_forward(tq, tk, tv, cut) * torch.tensor(do)).sum().backward()
    rows = np.array(sorted({0, 3, n // 2} | set(range(key_from, n))))
    dq, dk, dv = O.prefill_backward_rows(q, k, v, do, cut, rows, key_from)
    assert np.allclose(dq, tq.grad.numpy()[rows], rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy()[key_from:], rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy()[key_from:], rtol=1e-10, atol=1e-12)

"""Pins of the oracle's pi-Attention forms ("pi-Attention: Online Efficient
Sparse Transformers for Long-Context Modeling", Sections 3.4-3.5).

The union working set U(i) = N_r(i) u N_pi(i) (Eqs. 8-9) with one softmax
(Eqs. 10-11), fixed fusion (the log-prior logits of Eqs. 16-17) and the
separate softmax of Eq. 15 are checked against dense attention written with
library routines (scipy softmax, torch autograd in float64) over masks and
prior matrices built by brute force from the definitions, against closed
forms, and against central finite differences.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _wl(N, left, right, skip, both=0, mode="union", prior=0.5, D=4, H=2, hilbert=None):
    pat = dict(kind="band", left=left, right=right, skip=skip, skip_both=both, skip_mode=mode,
               skip_prior=prior)
    if hilbert:
        return dict(name="pi", B=1, H=H, D=D, dtype="fp32", grid=[hilbert, hilbert],
                    order="hilbert", pattern=pat)
    return dict(name="pi", B=1, H=H, D=D, dtype="fp32", grid=[N], order="row_major", pattern=pat)


def _sets(N, left, right, skip, both):
    """Brute force over positions: local[i, j] for j in N_r(i) (band, Eq. 5
    generalised), part[i, j] for j in N_pi(i) (Eq. 9: j = i - pi, and i + pi
    when both directions are fetched)."""
    local = np.zeros((N, N), bool)
    part = np.zeros((N, N), bool)
    for i in range(N):
        for j in range(N):
            local[i, j] = -left <= j - i <= right
            part[i, j] = j == i - skip or (both and j == i + skip)
    return local, part


def _dense(q, k, v, scale, mask, prior=None):
    """softmax(scale q k^T + prior) v over the masked keys, with scipy."""
    z = scale * q @ k.T + (0.0 if prior is None else prior)
    z = np.where(mask, z, -np.inf)
    with np.errstate(invalid="ignore"):  # rows with no key at all (no partner)
        p = softmax(z, axis=1)
        return p @ v, logsumexp(z, axis=1)


CASES = [(40, 4, 0, 16, 0), (40, 4, 0, 3, 0), (33, 2, 2, 9, 1), (20, 0, 0, 5, 1), (25, 3, 0, 30, 0)]


@pytest.mark.parametrize("N,left,right,skip,both", CASES)
def test_union_is_one_softmax_over_the_union(N, left, right, skip, both):
    wl = _wl(N, left, right, skip, both)
    q, k, v = (_rand((1, 2, N, 4), s) for s in (1, 2, 3))
    out, lse = oracle.attention(wl, q, k, v, 0.6)
    local, part = _sets(N, left, right, skip, both)
    for h in range(2):
        ref, ref_lse = _dense(q[0, h], k[0, h], v[0, h], 0.6, local | part)
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], ref_lse, atol=1e-12)
    # the neighbourhood the tile map covers is the union
    for i in range(N):
        assert oracle.neighbors(wl, i).tolist() == np.nonzero(local[i] | part[i])[0].tolist()


@pytest.mark.parametrize("alpha", [0.5, 0.3, 0.9])
@pytest.mark.parametrize("N,left,right,skip,both", CASES)
def test_fixed_fusion_is_log_prior_softmax(N, left, right, skip, both, alpha):
    wl = _wl(N, left, right, skip, both, mode="fixed_fusion", prior=alpha)
    q, k, v = (_rand((1, 2, N, 4), s) for s in (4, 5, 6))
    out, lse = oracle.attention(wl, q, k, v, 0.6)
    local, part = _sets(N, left, right, skip, both)
    # omega = alpha on N_r, 1 - alpha on partners outside N_r (Eq. 16)
    prior = np.where(local, math.log(alpha), math.log(1 - alpha))
    for h in range(2):
        ref, ref_lse = _dense(q[0, h], k[0, h], v[0, h], 0.6, local | part, prior)
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], ref_lse, atol=1e-12)
    if alpha == 0.5:
        # a uniform prior cancels in the softmax: the union output, lse - log 2
        u_out, u_lse = oracle.attention(_wl(N, left, right, skip, both), q, k, v, 0.6)
        np.testing.assert_allclose(out, u_out, atol=1e-12)
        np.testing.assert_allclose(lse, u_lse + math.log(0.5), atol=1e-12)


@pytest.mark.parametrize("N,left,right,skip,both", CASES)
def test_separate_softmax_sums_the_branches(N, left, right, skip, both):
    wl = _wl(N, left, right, skip, both, mode="separate")
    q, k, v = (_rand((1, 2, N, 4), s) for s in (7, 8, 9))
    out, lse = oracle.attention(wl, q, k, v, 0.6)
    local, part = _sets(N, left, right, skip, both)
    for h in range(2):
        loc_out, loc_lse = _dense(q[0, h], k[0, h], v[0, h], 0.6, local)
        has = part.any(axis=1)
        skip_out = np.zeros_like(loc_out)
        skip_out[has] = _dense(q[0, h], k[0, h], v[0, h], 0.6, part)[0][has]
        np.testing.assert_allclose(out[0, h], loc_out + skip_out, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], loc_lse, atol=1e-12)
        if not both:
            # one partner: its softmax is 1, so the skip branch adds v[i - pi]
            i = np.arange(skip, N)
            np.testing.assert_allclose(out[0, h, i] - loc_out[i], v[0, h, i - skip], atol=1e-12)


def test_partner_inside_window_changes_nothing():
    """pi <= k: the partner already belongs to N_r, so U = N_r (Eq. 8 is a set union)."""
    q, k, v = (_rand((1, 2, 30, 4), s) for s in (1, 2, 3))
    band = oracle.attention(_wl(30, 5, 0, 0), q, k, v, 0.5)
    for mode in ("union", "fixed_fusion"):
        got = oracle.attention(_wl(30, 5, 0, 3, mode=mode, prior=0.5), q, k, v, 0.5)
        np.testing.assert_allclose(got[0], band[0], atol=1e-12)


def test_partner_on_the_hilbert_curve():
    """On a Hilbert order the partner is pi positions back along the curve."""
    wl = _wl(None, 2, 2, 5, both=1, hilbert=8)
    perm = oracle.order(wl)
    pos = np.argsort(perm)
    for i in range(64):
        x = pos[i]
        want = sorted(int(perm[p]) for p in range(64)
                      if abs(p - x) <= 2 or p == x - 5 or p == x + 5)
        assert oracle.neighbors(wl, i).tolist() == want


@pytest.mark.parametrize("mode,alpha", [("union", 0.5), ("fixed_fusion", 0.3),
                                        ("separate", 0.5)])
def test_pairs_count(mode, alpha):
    wl = _wl(50, 4, 0, 16, both=1, mode=mode, prior=alpha)
    local, part = _sets(50, 4, 0, 16, 1)
    want = int((local | part).sum()) if mode != "separate" else int(local.sum() + part.sum())
    assert oracle.attended_pairs(wl) == want


# ---------------------------------------------------------------------------
# gradients
# ---------------------------------------------------------------------------

GRAD = [("union", 0.5, 0), ("fixed_fusion", 0.25, 0), ("fixed_fusion", 0.8, 1),
        ("separate", 0.5, 0), ("separate", 0.5, 1)]


@pytest.mark.parametrize("mode,alpha,both", GRAD)
def test_gradients_finite_differences(mode, alpha, both):
    wl = _wl(14, 2, 0, 5, both, mode=mode, prior=alpha, D=3, H=1)
    q, k, v, g = (_rand((1, 1, 14, 3), s) for s in (21, 22, 23, 24))
    dq, dk, dv = oracle.attention_backward(wl, q, k, v, g, 0.7)

    def loss(q_, k_, v_):
        return float(np.sum(oracle.attention(wl, q_, k_, v_, 0.7)[0] * g))

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else a for n, a in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else a for n, a in (("q", q), ("k", k), ("v", v))]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, atol=1e-6, err_msg=name)


@pytest.mark.parametrize("mode,alpha,both", GRAD)
def test_gradients_match_dense_autograd(mode, alpha, both):
    N = 24
    wl = _wl(N, 3, 1, 7, both, mode=mode, prior=alpha, D=5, H=1)
    q, k, v, g = (_rand((1, 1, N, 5), s) for s in (31, 32, 33, 34))
    dq, dk, dv = oracle.attention_backward(wl, q, k, v, g, 0.4)
    local, part = _sets(N, 3, 1, 7, both)
    tq, tk, tv = (torch.tensor(x[0, 0], dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    z = 0.4 * tq @ tk.T

    def attend(mask, prior=0.0):
        zz = torch.where(torch.tensor(mask), z + prior, torch.tensor(-math.inf, dtype=torch.float64))
        p = torch.softmax(zz, dim=1)
        p = torch.where(torch.tensor(mask.any(axis=1))[:, None], p, torch.zeros_like(p))
        return p @ tv

    if mode == "separate":
        out = attend(local) + attend(part)
    else:
        prior = torch.tensor(np.where(local, math.log(alpha), math.log(1 - alpha)))
        out = attend(local | part, prior)
    (out * torch.tensor(g[0, 0])).sum().backward()
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got[0, 0], t.grad.numpy(), atol=1e-10)

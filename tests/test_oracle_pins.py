"""Pins of the float64 oracle against facts other than itself (CPU only).

Each pin ties the oracle to something it does not compute the same way: values
worked by hand, a different least-squares route (QR/SVD via lstsq), the textbook
token-wise delta rule, the contraction bound, fixed points, limits, symmetries.
``test_mutants_are_caught`` plants plausible mistakes into the oracle (on the
CPU) and checks that at least one pin fails for each.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import vda_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-10


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    conv = lambda a: np.vectorize(lambda s: float(Fraction(s)))(np.array(a, dtype=object)).astype(np.float64)
    out = {k: conv(g[k]) for k in ("text_k", "text_v", "k", "v", "q", "x_text", "x_fwd", "x_bwd", "out")}
    out["lam"] = float(Fraction(g["lam"]))
    return out


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _rownorm(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _tiny_head(seed=0, F=4, n=5, d=3, dv=2, T=3):
    rng = np.random.default_rng(seed)
    return dict(q=_rand(rng, F, n, d), k=_rownorm(_rand(rng, F, n, d)), v=_rand(rng, F, n, dv),
                text_k=_rownorm(_rand(rng, T, d)), text_v=_rand(rng, T, dv))


# ---------------------------------------------------------------------------
# pin predicates (return True when the pin holds) -- reused by the mutant test
# ---------------------------------------------------------------------------

def pin_golden():
    ok = True
    for name in ("scalar_two_frames_lam1.json", "scalar_two_frames_lam_half.json"):
        g = _load_golden(name)
        xt, xf, xb = oracle.head_states(g["k"], g["v"], g["text_k"], g["text_v"], g["lam"])
        out = oracle.vda_forward_head(g["q"], g["k"], g["v"], g["text_k"], g["text_v"], g["lam"])
        ok &= np.allclose(xt, g["x_text"], rtol=RTOL, atol=1e-14)
        ok &= np.allclose(xf, g["x_fwd"], rtol=RTOL, atol=1e-14)
        ok &= np.allclose(xb, g["x_bwd"], rtol=RTOL, atol=1e-14)
        ok &= out.shape == g["out"].shape and np.allclose(out, g["out"], rtol=RTOL, atol=1e-14)
    return bool(ok)


def _stacked_lstsq_step(X_prev, K_f, V_f, lam):
    """The least-squares problem min ||K X - V||^2 + lam ||X - X_prev||^2 solved by QR/SVD
    on the stacked system [K; sqrt(lam) I] X = [V; sqrt(lam) X_prev] -- no normal equations."""
    d = K_f.shape[1]
    A = np.vstack([K_f, np.sqrt(lam) * np.eye(d)])
    R = np.vstack([V_f, np.sqrt(lam) * X_prev])
    return np.linalg.lstsq(A, R, rcond=None)[0]


def pin_lstsq(seed=1, lam=0.7, n=5, d=3, dv=2, F=4, T=3):
    h = _tiny_head(seed, F=F, n=n, d=d, dv=dv, T=T)
    xt, xf, xb = oracle.head_states(h["k"], h["v"], h["text_k"], h["text_v"], lam)
    ref_t = _stacked_lstsq_step(np.zeros((d, dv)), h["text_k"], h["text_v"], lam)
    ok = np.allclose(xt, ref_t, rtol=1e-9, atol=1e-12)
    x = ref_t
    for f in range(F):
        x = _stacked_lstsq_step(x, h["k"][f], h["v"][f], lam)
        ok &= np.allclose(xf[f], x, rtol=1e-9, atol=1e-12)
    x = ref_t
    for f in reversed(range(F)):
        x = _stacked_lstsq_step(x, h["k"][f], h["v"][f], lam)
        ok &= np.allclose(xb[f], x, rtol=1e-9, atol=1e-12)
    out = oracle.vda_forward_head(h["q"], h["k"], h["v"], h["text_k"], h["text_v"], lam)
    ok &= np.allclose(out, np.stack([h["q"][f] @ (0.5 * (xf[f] + xb[f])) for f in range(F)]),
                      rtol=1e-12, atol=1e-13)
    return bool(ok)


def _delta_rule(tokens_k, tokens_v, lam, d, dv):
    """Textbook token-wise delta rule (DeltaNet, Schlag et al. 2021) with step size
    beta = 1/(lam + ||k||^2), from a zero state: X <- X + beta k^T (v - k X)."""
    X = np.zeros((d, dv))
    states = []
    for kt, vt in zip(tokens_k, tokens_v):
        beta = 1.0 / (lam + kt @ kt)
        X = X + beta * np.outer(kt, vt - kt @ X)
        states.append(X.copy())
    return states


def pin_delta_rule(seed=2, lam=0.6, F=5, d=4, dv=3):
    h = _tiny_head(seed, F=F, n=1, d=d, dv=dv, T=1)
    xt, xf, xb = oracle.head_states(h["k"], h["v"], h["text_k"], h["text_v"], lam)
    fwd_k = [h["text_k"][0]] + [h["k"][f, 0] for f in range(F)]
    fwd_v = [h["text_v"][0]] + [h["v"][f, 0] for f in range(F)]
    s = _delta_rule(fwd_k, fwd_v, lam, d, dv)
    ok = np.allclose(xt, s[0], rtol=1e-10, atol=1e-13)
    ok &= np.allclose(xf, np.stack(s[1:]), rtol=1e-10, atol=1e-13)
    bwd_k = [h["text_k"][0]] + [h["k"][f, 0] for f in reversed(range(F))]
    bwd_v = [h["text_v"][0]] + [h["v"][f, 0] for f in reversed(range(F))]
    s = _delta_rule(bwd_k, bwd_v, lam, d, dv)
    ok &= np.allclose(xb, np.stack(s[1:][::-1]), rtol=1e-10, atol=1e-13)
    return bool(ok)


def pin_fixed_point(seed=3, lam=0.3, F=4, n=6, d=3, dv=2):
    rng = np.random.default_rng(seed)
    M = _rand(rng, dv, d)
    K = _rownorm(_rand(rng, F, n, d))
    V = K @ M.T
    xs = oracle.scan_from(M.T, K, V, lam)
    return bool(np.allclose(xs, np.broadcast_to(M.T, xs.shape), rtol=1e-11, atol=1e-12))


LN3, LN7 = np.log(3.0), np.log(7.0)


def pin_gate_worked_examples():
    """Gated epilogue, worked by hand with gate arguments whose sigmoid is rational
    (sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4, sigmoid(ln 7) = 7/8).
    Weights are [output feature][input feature]."""
    ok = True
    # 1. zero gate weights, bias (ln 3, -ln 3): gates 3/4 and 1/4 on output features 0 and 1;
    #    W_o = [[0, 1], [2, 0]] maps (o0, o1) to (o1, 2 o0): tokens (1, 2) -> (2, 2), (3, -1) -> (-1, 6)
    y = oracle.gated_output(np.array([[1.0, 2.0], [3.0, -1.0]]), np.zeros((2, 2)),
                            np.array([LN3, -LN3]), np.array([[0.0, 1.0], [2.0, 0.0]]))
    ok &= np.allclose(y, [[1.5, 0.5], [-0.75, 1.5]], rtol=1e-14, atol=0)
    # 2. W_g = [[0, ln 3], [0, 0]]: gate argument of output 0 is o1 ln 3; bias (0, ln 7); W_o = I.
    #    token (1, 1): gates (3/4, 7/8) -> (0.75, 0.875); token (2, 1): gates (3/4, 7/8) -> (1.5, 0.875);
    #    token (1, 0): gates (1/2, 7/8) -> (0.5, 0)
    y = oracle.gated_output(np.array([[1.0, 1.0], [2.0, 1.0], [1.0, 0.0]]), np.array([[0.0, LN3], [0.0, 0.0]]),
                            np.array([0.0, LN7]), np.eye(2))
    ok &= np.allclose(y, [[0.75, 0.875], [1.5, 0.875], [0.5, 0.0]], rtol=1e-14, atol=1e-15)
    return bool(ok)


def pin_gate_limits(seed=11, dv=5):
    """Gate saturation and the logistic function itself: a bias of +60 passes O W_o^T
    through, -60 closes the gate; with W_g = 0, b = 0 the output is half the projection;
    the gate agrees with scipy's expit."""
    from scipy.special import expit
    rng = np.random.default_rng(seed)
    Orow = rng.standard_normal((7, dv))
    Wg, Wo, b = rng.standard_normal((dv, dv)), rng.standard_normal((dv, dv)), rng.standard_normal(dv)
    P = Orow @ Wo.T
    ok = np.allclose(oracle.gated_output(Orow, np.zeros((dv, dv)), np.full(dv, 60.0), Wo), P, rtol=1e-14, atol=0)
    ok &= np.all(np.abs(oracle.gated_output(Orow, np.zeros((dv, dv)), np.full(dv, -60.0), Wo)) <= 1e-25 * np.abs(P).max())
    ok &= np.allclose(oracle.gated_output(Orow, np.zeros((dv, dv)), np.zeros(dv), Wo), 0.5 * P, rtol=1e-15, atol=0)
    ok &= np.allclose(oracle.gated_output(Orow, Wg, b, np.eye(dv)), expit(Orow @ Wg.T + b) * Orow, rtol=1e-13, atol=0)
    return bool(ok)


def _loss_grads_fd(h, lam, d_out, rng, eps=1e-6):
    """Central differences of L = sum(d_out * O) along one random direction per input."""
    names = ("q", "k", "v", "text_k", "text_v")
    out = []
    for name in names:
        dirn = rng.standard_normal(np.shape(h[name]))
        hp = dict(h); hp[name] = h[name] + eps * dirn
        hm = dict(h); hm[name] = h[name] - eps * dirn
        lp = np.sum(d_out * oracle.vda_forward_head(**hp, lam=lam))
        lm = np.sum(d_out * oracle.vda_forward_head(**hm, lam=lam))
        out.append((dirn, (lp - lm) / (2 * eps)))
    return out


def pin_backward_finite_differences(seed=31, lam=0.7, F=3, n=4, d=3, dv=2, T=2):
    """Directional derivatives of sum(d_out * O) by central differences (a route that never
    uses the adjoint equations) against the oracle's gradients."""
    rng = np.random.default_rng(seed)
    h = _tiny_head(seed, F=F, n=n, d=d, dv=dv, T=T)
    d_out = rng.standard_normal((F, n, dv))
    g = oracle.vda_backward_head(**h, lam=lam, d_out=d_out)
    ok = True
    for gi, (dirn, fd) in zip(g, _loss_grads_fd(h, lam, d_out, rng)):
        ok &= abs(np.sum(gi * dirn) - fd) <= 1e-6 * max(1.0, abs(fd))
    return bool(ok)


def _torch_forward_head(q, k, v, tk, tv, lam):
    """The forward op written again with torch float64 ops (solves by torch.linalg.solve)."""
    import torch
    d = k.shape[-1]
    eye = torch.eye(d, dtype=torch.float64)

    def upd(x, kk, vv):
        return torch.linalg.solve(lam * eye + kk.T @ kk, lam * x + kk.T @ vv)

    xt = upd(torch.zeros(d, v.shape[-1], dtype=torch.float64), tk, tv)
    fwd, x = [], xt
    for f in range(k.shape[0]):
        x = upd(x, k[f], v[f])
        fwd.append(x)
    bwd, x = [None] * k.shape[0], xt
    for f in reversed(range(k.shape[0])):
        x = upd(x, k[f], v[f])
        bwd[f] = x
    return torch.stack([q[f] @ (0.5 * (fwd[f] + bwd[f])) for f in range(k.shape[0])])


def pin_backward_torch_autograd(seed=32, lam=0.4, F=4, n=5, d=4, dv=3, T=3):
    """Every gradient element against torch's reverse-mode autograd of the same op written
    independently in torch (float64, CPU)."""
    import torch
    rng = np.random.default_rng(seed)
    h = _tiny_head(seed, F=F, n=n, d=d, dv=dv, T=T)
    d_out = rng.standard_normal((F, n, dv))
    g = oracle.vda_backward_head(**h, lam=lam, d_out=d_out)
    ts = [torch.tensor(h[name], dtype=torch.float64, requires_grad=True)
          for name in ("q", "k", "v", "text_k", "text_v")]
    (torch.sum(torch.tensor(d_out) * _torch_forward_head(*ts, lam))).backward()
    return bool(all(np.allclose(gi, t.grad.numpy(), rtol=1e-9, atol=1e-12) for gi, t in zip(g, ts)))


def pin_backward_batched(seed=36, lam=0.6, B=2, H=3, F=2, n=3, d=3, dv=2, T=2):
    """The [B,H] gradient wrapper against central differences of the batched forward op
    (``vda_forward`` over [B,H,...] arrays, pinned on its own), one random direction per input
    over the whole batch, and against the one-head gradients of every (b,h) slice.  A slice
    written to the wrong (b,h), or two slices swapped, fails the directional derivative."""
    rng = np.random.default_rng(seed)
    x = {"q": _rand(rng, B, H, F, n, d), "k": _rownorm(_rand(rng, B, H, F, n, d)),
         "v": _rand(rng, B, H, F, n, dv), "text_k": _rownorm(_rand(rng, B, H, T, d)),
         "text_v": _rand(rng, B, H, T, dv)}
    d_out = rng.standard_normal((B, H, F, n, dv))
    g = oracle.vda_backward(**x, lam=lam, d_out=d_out)
    ok = len(g) == 5
    eps = 1e-6
    for name, gi in zip(("q", "k", "v", "text_k", "text_v"), g):
        dirn = rng.standard_normal(x[name].shape)
        lp = np.sum(d_out * oracle.vda_forward(**{**x, name: x[name] + eps * dirn}, lam=lam))
        lm = np.sum(d_out * oracle.vda_forward(**{**x, name: x[name] - eps * dirn}, lam=lam))
        fd = (lp - lm) / (2 * eps)
        ok &= gi.shape == x[name].shape and abs(np.sum(gi * dirn) - fd) <= 1e-6 * max(1.0, abs(fd))
    for b in range(B):
        for h in range(H):
            ref = oracle.vda_backward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["text_k"][b, h],
                                           x["text_v"][b, h], lam, d_out[b, h])
            ok &= all(np.array_equal(gi[b, h], r) for gi, r in zip(g, ref))
    return bool(ok)


PINS = [pin_golden, pin_lstsq, lambda: pin_lstsq(seed=4, n=6, d=3, dv=3), pin_delta_rule,
        pin_fixed_point, pin_gate_worked_examples, pin_gate_limits,
        pin_backward_finite_differences, pin_backward_torch_autograd, pin_backward_batched]


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

def test_golden_scalar_cases():
    assert pin_golden()


@pytest.mark.parametrize("shape", [dict(n=5, d=3, dv=2), dict(n=2, d=4, dv=3), dict(n=7, d=2, dv=5)])
def test_every_step_is_the_stacked_least_squares_solution(shape):
    assert pin_lstsq(**shape)


def test_n1_reduces_to_token_delta_rule():
    assert pin_delta_rule()


def test_fixed_point_state_is_kept():
    assert pin_fixed_point()


def test_fixed_point_readout_and_text_start_contracts():
    rng = np.random.default_rng(4)
    F, n, d, dv, T, lam = 5, 7, 4, 3, 5, 0.2
    M = _rand(rng, dv, d)
    K = _rownorm(_rand(rng, F, n, d))
    Q = _rand(rng, F, n, d)
    tk = _rownorm(_rand(rng, T, d))
    xt, xf, xb = oracle.head_states(K, K @ M.T, tk, tk @ M.T, lam)
    # start at the text state, which differs from M^T; the gap never grows
    gaps = [np.linalg.norm(xt - M.T)] + [np.linalg.norm(xf[f] - M.T) for f in range(F)]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(gaps, gaps[1:]))
    gaps = [np.linalg.norm(xt - M.T)] + [np.linalg.norm(xb[f] - M.T) for f in reversed(range(F))]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(gaps, gaps[1:]))
    # starting exactly at M^T, the readout is Q M^T
    xs = oracle.scan_from(M.T, K, K @ M.T, lam)
    out = oracle.readout(Q, xs, xs)
    assert np.allclose(out, Q @ M.T, rtol=1e-11, atol=1e-12)


def test_non_expansive_with_contraction_bound():
    rng = np.random.default_rng(5)
    F, n, d, dv, lam = 6, 5, 4, 3, 0.4
    K = _rownorm(_rand(rng, F, n, d))
    V = _rand(rng, F, n, dv)
    X0, X1 = _rand(rng, d, dv), _rand(rng, d, dv)
    a, b = oracle.scan_from(X0, K, V, lam), oracle.scan_from(X1, K, V, lam)
    prev = np.linalg.norm(X0 - X1)
    for f in range(F):
        sig_min = np.linalg.eigvalsh(K[f].T @ K[f]).min()
        cur = np.linalg.norm(a[f] - b[f])
        assert cur <= prev * lam / (lam + sig_min) * (1 + 1e-10) + 1e-14
        assert cur <= prev
        prev = cur


def test_small_lambda_gives_per_frame_ols():
    rng = np.random.default_rng(6)
    F, n, d, dv = 3, 9, 4, 3
    K = _rand(rng, F, n, d)
    V = _rand(rng, F, n, dv)
    xs = oracle.scan_from(_rand(rng, d, dv), K, V, 1e-10)
    for f in range(F):
        ols = np.linalg.lstsq(K[f], V[f], rcond=None)[0]
        assert np.allclose(xs[f], ols, rtol=1e-6, atol=1e-7)


def test_single_frame_closed_form():
    h = _tiny_head(7, F=1, n=6, d=3, dv=4, T=2)
    lam = 0.9
    xt = _stacked_lstsq_step(np.zeros((3, 4)), h["text_k"], h["text_v"], lam)
    x1 = _stacked_lstsq_step(xt, h["k"][0], h["v"][0], lam)
    out = oracle.vda_forward_head(h["q"], h["k"], h["v"], h["text_k"], h["text_v"], lam)
    assert np.allclose(out[0], h["q"][0] @ x1, rtol=1e-10, atol=1e-12)


def test_no_text_gives_zero_text_state():
    h = _tiny_head(8, T=0)
    xt, _, _ = oracle.head_states(h["k"], h["v"], h["text_k"], h["text_v"], 0.5)
    assert xt.shape == (3, 2) and np.all(xt == 0)


def test_frame_reversal_reverses_outputs():
    h = _tiny_head(9, F=5)
    lam = 0.8
    out = oracle.vda_forward_head(h["q"], h["k"], h["v"], h["text_k"], h["text_v"], lam)
    rev = oracle.vda_forward_head(h["q"][::-1], h["k"][::-1], h["v"][::-1], h["text_k"], h["text_v"], lam)
    assert np.allclose(rev, out[::-1], rtol=1e-12, atol=1e-13)


def test_token_permutation_within_a_frame():
    h = _tiny_head(10, F=4, n=6)
    lam = 0.8
    out = oracle.vda_forward_head(h["q"], h["k"], h["v"], h["text_k"], h["text_v"], lam)
    perm = np.random.default_rng(0).permutation(6)
    q, k, v = h["q"].copy(), h["k"].copy(), h["v"].copy()
    q[2], k[2], v[2] = q[2][perm], k[2][perm], v[2][perm]
    out2 = oracle.vda_forward_head(q, k, v, h["text_k"], h["text_v"], lam)
    exp = out.copy()
    exp[2] = out[2][perm]
    assert np.allclose(out2, exp, rtol=1e-11, atol=1e-12)


def test_linearity_in_values_and_queries():
    h = _tiny_head(11)
    lam = 0.5
    f = lambda **kw: oracle.vda_forward_head(**{**h, **kw}, lam=lam)
    base = f()
    assert np.allclose(f(v=2.5 * h["v"], text_v=2.5 * h["text_v"]), 2.5 * base, rtol=1e-11, atol=1e-12)
    q2 = np.random.default_rng(1).standard_normal(h["q"].shape)
    assert np.allclose(f(q=h["q"] + q2) - f(q=q2), base, rtol=1e-10, atol=1e-11)


def test_heads_and_batch_are_independent():
    rng = np.random.default_rng(12)
    B, H, F, n, d, dv, T = 2, 3, 3, 4, 3, 2, 2
    q, k, v = _rand(rng, B, H, F, n, d), _rownorm(_rand(rng, B, H, F, n, d)), _rand(rng, B, H, F, n, dv)
    tk, tv = _rownorm(_rand(rng, B, H, T, d)), _rand(rng, B, H, T, dv)
    out = oracle.vda_forward(q, k, v, tk, tv, 0.6)
    for b in range(B):
        for hh in range(H):
            ref = oracle.vda_forward_head(q[b, hh], k[b, hh], v[b, hh], tk[b, hh], tv[b, hh], 0.6)
            assert np.array_equal(out[b, hh], ref)
    k2 = k.copy()
    k2[1, 2] = _rownorm(_rand(rng, F, n, d))
    out2 = oracle.vda_forward(q, k2, v, tk, tv, 0.6)
    assert np.array_equal(out2[0], out[0]) and np.array_equal(out2[1, :2], out[1, :2])


def test_gate_worked_examples():
    assert pin_gate_worked_examples()


def test_gate_limits_and_logistic():
    assert pin_gate_limits()


def test_gated_forward_applies_each_heads_weights():
    rng = np.random.default_rng(21)
    B, H, F, n, d, dv, T = 2, 3, 3, 4, 3, 2, 2
    q, k, v = rng.standard_normal((B, H, F, n, d)), _rownorm(rng.standard_normal((B, H, F, n, d))), \
        rng.standard_normal((B, H, F, n, dv))
    tk, tv = _rownorm(rng.standard_normal((B, H, T, d))), rng.standard_normal((B, H, T, dv))
    Wg, Wo, bg = rng.standard_normal((H, dv, dv)), rng.standard_normal((H, dv, dv)), rng.standard_normal((H, dv))
    y = oracle.vda_forward_gated(q, k, v, tk, tv, 0.5, Wg, bg, Wo)
    for b in range(B):
        for h in range(H):
            o = oracle.vda_forward_head(q[b, h], k[b, h], v[b, h], tk[b, h], tv[b, h], 0.5)
            assert np.array_equal(y[b, h], oracle.gated_output(o, Wg[h], bg[h], Wo[h]))
            assert np.array_equal(y[b, h], oracle.vda_forward_gated_head(q[b, h], k[b, h], v[b, h], tk[b, h],
                                                                         tv[b, h], 0.5, Wg[h], bg[h], Wo[h]))


def test_backward_matches_finite_differences():
    assert pin_backward_finite_differences()
    assert pin_backward_finite_differences(seed=33, lam=0.2, F=1, n=6, d=2, dv=3, T=1)


def test_backward_matches_torch_autograd():
    assert pin_backward_torch_autograd()
    assert pin_backward_torch_autograd(seed=34, lam=1.0, F=2, n=1, d=3, dv=3, T=1)


def test_batched_backward_wrapper():
    assert pin_backward_batched()
    assert pin_backward_batched(seed=37, lam=0.3, B=3, H=2, F=1, n=2, d=2, dv=3, T=1)


def test_backward_with_no_text_and_linearity_in_d_out():
    rng = np.random.default_rng(35)
    h = _tiny_head(35, F=3, n=4, d=3, dv=2, T=0)
    h["text_k"], h["text_v"] = np.zeros((0, 3)), np.zeros((0, 2))
    d1, d2 = rng.standard_normal((3, 4, 2)), rng.standard_normal((3, 4, 2))
    g1 = oracle.vda_backward_head(**h, lam=0.5, d_out=d1)
    g2 = oracle.vda_backward_head(**h, lam=0.5, d_out=d2)
    g12 = oracle.vda_backward_head(**h, lam=0.5, d_out=2 * d1 - d2)
    for a, b, c in zip(g1, g2, g12):
        assert np.allclose(c, 2 * a - b, rtol=1e-10, atol=1e-12)
    assert g1[3].shape == (0, 3) and g1[4].shape == (0, 2)


def test_rejects_nonpositive_lambda():
    h = _tiny_head(13)
    with pytest.raises(ValueError):
        oracle.vda_forward_head(**h, lam=0.0)


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _update_no_lam_on_prev(X_prev, K_f, V_f, lam):
    G, Bm = O.frame_statistics(K_f, V_f)
    return np.linalg.solve(lam * np.eye(G.shape[0]) + G, X_prev + Bm)


def _update_no_lam_on_identity(X_prev, K_f, V_f, lam):
    G, Bm = O.frame_statistics(K_f, V_f)
    return np.linalg.solve(np.eye(G.shape[0]) + G, lam * X_prev + Bm)


def _update_sign(X_prev, K_f, V_f, lam):
    G, Bm = O.frame_statistics(K_f, V_f)
    return np.linalg.solve(lam * np.eye(G.shape[0]) + G, lam * X_prev - Bm)


def _update_n_scaled(X_prev, K_f, V_f, lam):
    G, Bm = O.frame_statistics(K_f, V_f)
    n = K_f.shape[0]
    return np.linalg.solve(lam * np.eye(G.shape[0]) + G / n, lam * X_prev + Bm / n)


def _stats_transposed_cross(K_f, V_f):
    return K_f.T @ K_f, V_f.T @ K_f


def _readout_sum(q, X_fwd, X_bwd):
    return np.stack([q[f] @ (X_fwd[f] + X_bwd[f]) for f in range(q.shape[0])])


def _readout_forward_only(q, X_fwd, X_bwd):
    return np.stack([q[f] @ X_fwd[f] for f in range(q.shape[0])])


def _states_bwd_from_zero(k, v, text_k, text_v, lam):
    d, dv = k.shape[-1], v.shape[-1]
    X_text = O.text_state(text_k, text_v, lam, d, dv)
    return X_text, O.scan_from(X_text, k, v, lam), O.scan_from(np.zeros((d, dv)), k[::-1], v[::-1], lam)[::-1]


def _states_bwd_not_reversed(k, v, text_k, text_v, lam):
    d, dv = k.shape[-1], v.shape[-1]
    X_text = O.text_state(text_k, text_v, lam, d, dv)
    return X_text, O.scan_from(X_text, k, v, lam), O.scan_from(X_text, k[::-1], v[::-1], lam)


def _states_exclusive(k, v, text_k, text_v, lam):
    d, dv = k.shape[-1], v.shape[-1]
    X_text = O.text_state(text_k, text_v, lam, d, dv)
    f = O.scan_from(X_text, k, v, lam)
    b = O.scan_from(X_text, k[::-1], v[::-1], lam)[::-1]
    fx = np.concatenate([X_text[None], f[:-1]])
    bx = np.concatenate([b[1:], X_text[None]])
    return X_text, fx, bx


def _gate_tanh(O_rows, w_gate, b_gate, w_out):
    return np.tanh(O_rows @ w_gate.T + b_gate) * (O_rows @ w_out.T)


def _gate_bias_sign(O_rows, w_gate, b_gate, w_out):
    return 1.0 / (1.0 + np.exp(-(O_rows @ w_gate.T - b_gate))) * (O_rows @ w_out.T)


def _gate_w_out_transposed(O_rows, w_gate, b_gate, w_out):
    return 1.0 / (1.0 + np.exp(-(O_rows @ w_gate.T + b_gate))) * (O_rows @ w_out)


def _gate_w_gate_transposed(O_rows, w_gate, b_gate, w_out):
    return 1.0 / (1.0 + np.exp(-(O_rows @ w_gate + b_gate))) * (O_rows @ w_out.T)


def _gate_additive(O_rows, w_gate, b_gate, w_out):
    return 1.0 / (1.0 + np.exp(-(O_rows @ w_gate.T + b_gate))) + (O_rows @ w_out.T)


MUTANTS = {
    "gate_tanh": ("gated_output", _gate_tanh),
    "gate_bias_sign": ("gated_output", _gate_bias_sign),
    "gate_w_out_transposed": ("gated_output", _gate_w_out_transposed),
    "gate_w_gate_transposed": ("gated_output", _gate_w_gate_transposed),
    "gate_additive": ("gated_output", _gate_additive),
    "no_lam_on_prev": ("normal_equation_update", _update_no_lam_on_prev),
    "no_lam_on_identity": ("normal_equation_update", _update_no_lam_on_identity),
    "sign_of_cross_term": ("normal_equation_update", _update_sign),
    "frame_size_scaling": ("normal_equation_update", _update_n_scaled),
    "cross_term_wrong_operand": ("frame_statistics", _stats_transposed_cross),
    "readout_without_half": ("readout", _readout_sum),
    "readout_forward_only": ("readout", _readout_forward_only),
    "backward_from_zero": ("head_states", _states_bwd_from_zero),
    "backward_not_reordered": ("head_states", _states_bwd_not_reversed),
    "exclusive_states": ("head_states", _states_exclusive),
}


# mistakes planted in the backward pass: one-line edits of the oracle's own source
BACKWARD_MUTANTS = {
    "adjoint_no_lam": ("half_dW[f - 1] + lam * U[f + 1]", "half_dW[f - 1] + U[f + 1]"),
    "adjoint_wrong_direction": ("half_dW[f - 1] + lam * V[f - 1]", "half_dW[f - 1] + lam * V[f - 1] * 0"),
    "dA_states_swapped": ("U[f] @ X_fwd[f - 1].T + V[f] @ X_bwd[f - 1].T",
                          "U[f] @ X_bwd[f - 1].T + V[f] @ X_fwd[f - 1].T"),
    "dA_not_symmetrised": ("k[f - 1] @ (dA + dA.T)", "k[f - 1] @ (2 * dA)"),
    "dW_not_halved": ("half_dW = [0.5 * (q[f].T", "half_dW = [(q[f].T"),
    "text_adjoint_dropped": ("gamma_text = lam * (U[1] + V[F])", "gamma_text = lam * U[1]"),
    "dq_forward_state_only": ("d_out[f] @ W[f].T", "d_out[f] @ X_fwd[f].T"),
}


def _backward_mutant(name):
    import inspect
    src = inspect.getsource(O.vda_backward_head)
    old, new = BACKWARD_MUTANTS[name]
    assert old in src, name
    ns = dict(vars(O))
    exec(src.replace(old, new), ns)
    return ns["vda_backward_head"]


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutants_are_caught(name, monkeypatch):
    fn = _backward_mutant(name)
    monkeypatch.setattr(O, "vda_backward_head", fn)
    monkeypatch.setattr(oracle, "vda_backward_head", fn, raising=False)
    results = []
    for pin in (pin_backward_finite_differences, pin_backward_torch_autograd):
        try:
            results.append(pin())
        except Exception:
            results.append(False)
    assert not all(results), f"mutant {name} passes every pin"


# mistakes planted in the [B,H] gradient wrapper: one-line edits of its own source
BATCHED_BACKWARD_MUTANTS = {
    "slices_to_first_head": ("g[b, h] = r", "g[b, 0] = r"),
    "heads_reversed": ("g[b, h] = r", "g[b, H - 1 - h] = r"),
    "d_out_of_other_head": ("                                    d_out[b, h])",
                            "                                    d_out[b, (h + 1) % H])"),
    "gradients_rotated": ("for g, r in zip(grads, res):", "for g, r in zip(grads, res[1:] + res[:1]):"),
}


def _batched_backward_mutant(name):
    import inspect
    src = inspect.getsource(O.vda_backward)
    old, new = BATCHED_BACKWARD_MUTANTS[name]
    assert old in src, name
    ns = dict(vars(O))
    exec(src.replace(old, new), ns)
    return ns["vda_backward"]


@pytest.mark.parametrize("name", sorted(BATCHED_BACKWARD_MUTANTS))
def test_batched_backward_mutants_are_caught(name, monkeypatch):
    fn = _batched_backward_mutant(name)
    monkeypatch.setattr(O, "vda_backward", fn)
    monkeypatch.setattr(oracle, "vda_backward", fn, raising=False)
    try:
        ok = pin_backward_batched()
    except Exception:
        ok = False
    assert not ok, f"mutant {name} passes the batched pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    results = []
    for pin in PINS:
        try:
            results.append(pin())
        except Exception:
            results.append(False)
    assert not all(results), f"mutant {name} passes every pin"

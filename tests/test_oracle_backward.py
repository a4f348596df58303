"""Pins for the oracle's backward pass, checked against things other than its
own formulas:

* central finite differences of the (separately pinned) forward oracle, for
  every input and weight entry of tiny blocks, both activations, several P
  and ring orders;
* the activation derivatives against finite differences of the activations,
  their exact values at 0 and their limits;
* the sharding identities: gradients do not depend on P or on the ring
  order, equal the unsharded block's, and a simulated TSP group (each rank
  its own tokens) adds up to the full-sequence weight gradients;
* special cases: a one-hot output gradient selects one token's hidden
  activations as a column of the down gradient (compared with the forward's
  hidden activations), gradients are linear in dY;
* the column-restricted weight gradients equal the full ones.

A mutation test plants plausible mistakes in the backward and checks that
at least one pin fails for each.
"""
import math

import numpy as np
import pytest

import oracle.tsp_oracle as O


def _inputs(T, d, f, act, seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((T, d))
    wg = r.standard_normal((d, f)) / math.sqrt(d) if act == "swiglu" else None
    wu = r.standard_normal((d, f)) / math.sqrt(d)
    wd = r.standard_normal((f, d)) / math.sqrt(f)
    dY = r.standard_normal((T, d))
    return X, wg, wu, wd, dY


def _close(a, b, tol):
    scale = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / scale <= tol


# ---------------------------------------------------------------- pin functions

def pin_bwd_finite_differences(o):
    """Every gradient entry against a central difference of
    L = sum(dY * forward(...)) in float64 (step 1e-5: truncation ~1e-10,
    cancellation ~1e-11 relative)."""
    h = 1e-5
    for act, T, d, f, P, order in (("swiglu", 3, 4, 6, 2, [1, 0]), ("swiglu", 2, 3, 6, 3, [2, 0, 1]),
                                   ("gelu_tanh", 3, 4, 6, 2, [0, 1]), ("gelu_tanh", 2, 5, 4, 4, [3, 2, 1, 0])):
        X, wg, wu, wd, dY = _inputs(T, d, f, act, 7 + T + d)
        X = 1.5 * X                                     # reach the curved part of both activations
        g = o.mlp_backward(X, wg, wu, wd, dY, P, order, act)

        def loss(X=X, wg=wg, wu=wu, wd=wd):
            return float(np.sum(dY * O.mlp_forward(X, wg, wu, wd, P, order, act)))

        for name, arr, key in (("X", X, "dX"), ("wg", wg, "dW_gate"), ("wu", wu, "dW_up"), ("wd", wd, "dW_down")):
            if arr is None:
                assert g[key] is None
                continue
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                e = np.zeros_like(arr)
                e[idx] = h
                fd[idx] = (loss(**{name: arr + e}) - loss(**{name: arr - e})) / (2 * h)
            assert g[key].shape == arr.shape, (act, name)
            assert _close(g[key], fd, 1e-7), (act, name, float(np.max(np.abs(g[key] - fd))))


def pin_bwd_activation_derivatives(o):
    x = np.linspace(-12.0, 12.0, 2401)
    h = 1e-5
    fd_s = (O.silu(x + h) - O.silu(x - h)) / (2 * h)
    fd_g = (O.gelu_tanh(x + h) - O.gelu_tanh(x - h)) / (2 * h)
    assert np.max(np.abs(o.silu_grad(x) - fd_s)) < 1e-9
    assert np.max(np.abs(o.gelu_tanh_grad(x) - fd_g)) < 1e-9
    # exact values at 0, limits, no NaN far out
    assert o.silu_grad(np.array([0.0]))[0] == 0.5
    assert o.gelu_tanh_grad(np.array([0.0]))[0] == 0.5
    big = np.array([-1000.0, -100.0, 100.0, 1000.0])
    sg, gg = o.silu_grad(big), o.gelu_tanh_grad(big)
    assert np.all(np.isfinite(sg)) and np.all(np.isfinite(gg))
    assert abs(sg[0]) < 1e-300 and abs(sg[1]) < 1e-40 and sg[2] == 1.0 and sg[3] == 1.0
    assert gg[0] == 0.0 and gg[3] == 1.0
    # SiLU' has its minimum near g = -2.3994 (SiLU'' = 0 there) with value about -0.0998
    gm = np.linspace(-3.0, -2.0, 100001)
    v = o.silu_grad(gm)
    assert abs(gm[np.argmin(v)] + 2.3994) < 1e-3 and abs(v.min() + 0.0998) < 1e-3


def pin_bwd_sharding_identity(o):
    T, d, f = 5, 8, 24
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd, dY = _inputs(T, d, f, act, 21)
        ref = o.mlp_backward(X, wg, wu, wd, dY, 1, None, act)
        for P in (2, 3, 4, 6, 8):
            for order in (o.ring_order(P, 0), o.ring_order(P, P - 1), o.ring_order(P, 1)[::-1]):
                g = o.mlp_backward(X, wg, wu, wd, dY, P, order, act)
                for k in ("dX", "dW_gate", "dW_up", "dW_down"):
                    if ref[k] is None:
                        assert g[k] is None
                    else:
                        assert _close(g[k], ref[k], 1e-12), (act, P, order, k)
        # a TSP group: rank r holds token rows [r*n, (r+1)*n) and visits the shards
        # from its own starting point; dX rows concatenate, weight gradients add up
        P = 4
        Xf, _, _, _, dYf = _inputs(4 * 3, d, f, act, 22)
        full = o.mlp_backward(Xf, wg, wu, wd, dYf, P, None, act)
        acc = {k: None for k in ("dW_gate", "dW_up", "dW_down")}
        rows = []
        for r in range(P):
            g = o.mlp_backward(Xf[3 * r:3 * r + 3], wg, wu, wd, dYf[3 * r:3 * r + 3], P, o.ring_order(P, r), act)
            rows.append(g["dX"])
            for k in acc:
                if g[k] is not None:
                    acc[k] = g[k] if acc[k] is None else acc[k] + g[k]
        assert _close(np.concatenate(rows), full["dX"], 1e-12)
        for k in acc:
            if full[k] is not None:
                assert _close(acc[k], full[k], 1e-12), (act, k)


def pin_bwd_special_cases(o):
    T, d, f, P = 4, 6, 8, 2
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd, dY = _inputs(T, d, f, act, 31)
        g = o.mlp_backward(X, wg, wu, wd, dY, P, None, act)
        g2 = o.mlp_backward(X, wg, wu, wd, 2.0 * dY, P, None, act)
        for k in ("dX", "dW_gate", "dW_up", "dW_down"):
            if g[k] is not None:
                assert np.array_equal(g2[k], 2.0 * g[k]), (act, k)       # exact: scaling by 2
        zero = o.mlp_backward(X, wg, wu, wd, np.zeros_like(dY), P, None, act)
        assert all(zero[k] is None or np.all(zero[k] == 0.0) for k in zero)
        # one-hot dY at (t, n): column n of dW_down is token t's hidden row (forward oracle)
        t, n = 2, 5
        e = np.zeros_like(dY)
        e[t, n] = 1.0
        ge = o.mlp_backward(X, wg, wu, wd, e, P, [1, 0], act)
        H = np.concatenate([O.shard_hidden(X, wg, wu, s, f // P, act) for s in range(P)], axis=1)
        assert _close(ge["dW_down"][:, n], H[t], 1e-14)
        others = np.delete(ge["dW_down"], n, axis=1)
        assert np.all(others == 0.0)
        # only token t's dX row is non-zero
        assert np.all(np.delete(ge["dX"], t, axis=0) == 0.0) and np.any(ge["dX"][t] != 0.0)


def pin_bwd_columns(o):
    T, d, f, P = 6, 8, 16, 4
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd, dY = _inputs(T, d, f, act, 41)
        g = o.mlp_backward(X, wg, wu, wd, dY, P, None, act)
        cols = [0, 5, 6, 15, 9]
        c = o.mlp_backward_columns(X, wg, wu, wd, dY, cols, act)
        assert _close(c["dW_up"], g["dW_up"][:, cols], 1e-13)
        assert _close(c["dW_down"], g["dW_down"][cols, :], 1e-13)
        if act == "swiglu":
            assert _close(c["dW_gate"], g["dW_gate"][:, cols], 1e-13)


def pin_bwd_round_bf16(o):
    """The diagnostic rounding moves the gradients by about bf16's relative
    precision and no more."""
    T, d, f, P = 16, 32, 64, 4
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd, dY = _inputs(T, d, f, act, 51)
        g = o.mlp_backward(X, wg, wu, wd, dY, P, None, act)
        gr = o.mlp_backward(X, wg, wu, wd, dY, P, None, act, round_bf16=True)
        for k in ("dX", "dW_gate", "dW_up", "dW_down"):
            if g[k] is None:
                continue
            el2 = np.linalg.norm(gr[k] - g[k]) / np.linalg.norm(g[k])
            assert 1e-5 < el2 < 4e-3, (act, k, el2)


ALL_PINS = [pin_bwd_finite_differences, pin_bwd_activation_derivatives, pin_bwd_sharding_identity,
            pin_bwd_special_cases, pin_bwd_columns, pin_bwd_round_bf16]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


def test_invalid_arguments():
    X, wg, wu, wd, dY = _inputs(2, 4, 8, "swiglu", 1)
    with pytest.raises(ValueError):
        O.mlp_backward(X, wg, wu, wd, dY[:, :3], 2)
    with pytest.raises(ValueError):
        O.mlp_backward(X, wg, wu, wd, dY, 3)
    with pytest.raises(ValueError):
        O.mlp_backward(X, None, wu, wd, dY, 2, None, "swiglu")
    with pytest.raises(ValueError):
        O.mlp_backward(X, wg, wu, wd, dY, 2, [0, 0])


def test_backward_flops():
    assert O.backward_flops(1, 1, 1, "swiglu") == 12
    assert O.backward_flops(2, 3, 5, "gelu_tanh") == 8 * 30


# ---------------------------------------------------------------- mutation test

_orig_shard_backward = O.shard_backward


def _mut_silu_grad_sign(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 - g * (1.0 - sig))


def _mut_gelu_grad_drop_term(u):
    u = np.asarray(u, dtype=np.float64)
    th = np.tanh(O.SQRT_2_OVER_PI * (u + O.GELU_TANH_CUBIC * u ** 3))
    return 0.5 * (1.0 + th)


def _mut_dx_drop_up(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16=False):
    dX, dWg, dWu, dWd = _orig_shard_backward(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16)
    if act != "swiglu":
        return 0.5 * dX, dWg, dWu, dWd
    cols = slice(s * F, (s + 1) * F)
    X64 = np.asarray(X, dtype=np.float64)
    u = X64 @ w_up[:, cols]
    g = X64 @ w_gate[:, cols]
    dH = np.asarray(dY, dtype=np.float64) @ w_down[cols, :].T
    dG = dH * u * O.silu_grad(g)
    return dG @ w_gate[:, cols].T, dWg, dWu, dWd


def _mut_dwd_wrong_shard(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16=False):
    P = w_up.shape[1] // F
    dX, dWg, dWu, _ = _orig_shard_backward(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16)
    _, _, _, dWd2 = _orig_shard_backward(X, w_gate, w_up, w_down, dY, (s + 1) % P, F, act, round_bf16)
    return dX, dWg, dWu, dWd2


def _mut_swap_dg_du(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16=False):
    dX, dWg, dWu, dWd = _orig_shard_backward(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16)
    if act != "swiglu":
        return dX, dWg, 1.01 * dWu, dWd
    return dX, dWu, dWg, dWd


def _mut_dx_uses_down_transposed(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16=False):
    # dH from the down block read as if it were stored output x input
    cols = slice(s * F, (s + 1) * F)
    wd = np.asarray(w_down, dtype=np.float64)
    wdT = wd.T if wd.shape[0] == wd.shape[1] else wd[::-1]
    wd2 = wd.copy()
    wd2[cols, :] = wdT[cols, :]
    return _orig_shard_backward(X, w_gate, w_up, wd2, dY, s, F, act, round_bf16)


MUTANTS = {
    "silu_grad_sign": ("silu_grad", _mut_silu_grad_sign),
    "gelu_grad_drop_term": ("gelu_tanh_grad", _mut_gelu_grad_drop_term),
    "dx_drop_up_term": ("shard_backward", _mut_dx_drop_up),
    "dwd_wrong_shard": ("shard_backward", _mut_dwd_wrong_shard),
    "swap_dg_du": ("shard_backward", _mut_swap_dg_du),
    "dh_from_wrong_down_rows": ("shard_backward", _mut_dx_uses_down_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"

"""Pins for the fp64 oracle: it is checked against things other than itself.

* exact integer worked examples (tests/golden/worked_examples.json);
* pure-Python brute force of the unsharded block on tiny shapes;
* closed forms of the activations and a high-precision evaluation;
* the column-then-row identity: the result does not depend on P, on the ring
  rotation or on any shard permutation, and a simulated TSP group equals the
  unsharded block;
* a negative case: splitting the first matrix by rows (before the
  nonlinearity) gives a visibly different answer;
* special cases: identity and selection weights, linearity and scaling.

A mutation test plants plausible mistakes in the oracle and checks that at
least one pin fails for each.
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle.tsp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _arr(a):
    return None if a is None else np.array(a, dtype=np.float64)


def _rng_inputs(T, d, f, act, seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((T, d))
    wg = r.standard_normal((d, f)) / math.sqrt(d) if act == "swiglu" else None
    wu = r.standard_normal((d, f)) / math.sqrt(d)
    wd = r.standard_normal((f, d)) / math.sqrt(f)
    return X, wg, wu, wd


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- pin functions
# Each takes the oracle module so the mutation test can run them on a planted
# mistake. Each raises AssertionError (or a shape error) when the pin fails.

def pin_golden(o):
    ex = json.load(open(GOLDEN))
    for key, e in ex.items():
        X, wg, wu, wd = _arr(e["X"]), _arr(e["w_gate"]), _arr(e["w_up"]), _arr(e["w_down"])
        P = e["P"]
        F = wu.shape[1] // P
        for r0 in range(P):
            for order in (o.ring_order(P, r0), o.ring_order(P, r0)[::-1]):
                Y = o.mlp_forward(X, wg, wu, wd, P, order, e["act"])
                assert np.array_equal(Y, _arr(e["Y"])), (key, order)
        H = np.concatenate([o.shard_hidden(X, wg, wu, s, F, e["act"]) for s in range(P)], axis=1)
        assert np.array_equal(H, _arr(e["hidden"])), key
        if "partials_by_shard" in e:
            for s in range(P):
                Ps = o.shard_partial(X, wg, wu, wd, s, F, e["act"])
                assert np.array_equal(Ps, _arr(e["partials_by_shard"][s])), (key, s)


def _brute(X, wg, wu, wd, act):
    """Unsharded block with Python floats and explicit loops (no numpy)."""
    T, d = len(X), len(X[0])
    f = len(wu[0])
    Y = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for c in range(f):
            u = 0.0
            for i in range(d):
                u += X[t][i] * wu[i][c]
            if act == "swiglu":
                g = 0.0
                for i in range(d):
                    g += X[t][i] * wg[i][c]
                h = g / (1.0 + math.exp(-g)) * u
            else:
                h = 0.5 * u * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))
            for n in range(d):
                Y[t][n] += h * wd[c][n]
    return np.array(Y)


def pin_brute_force(o):
    cases = [(1, 1, 2), (3, 5, 8), (2, 4, 6), (3, 3, 12), (2, 4, 4)]   # last: square d == f
    for ci, (T, d, f) in enumerate(cases):
        for act in ("swiglu", "gelu_tanh"):
            X, wg, wu, wd = _rng_inputs(T, d, f, act, 100 + ci)
            ref = _brute(X.tolist(), None if wg is None else wg.tolist(), wu.tolist(),
                         wd.tolist(), act)
            for P in [p for p in range(1, f + 1) if f % p == 0]:
                orders = (itertools.permutations(range(P)) if P <= 4
                          else [o.ring_order(P, r) for r in range(P)])
                for order in orders:
                    Y = o.mlp_forward(X, wg, wu, wd, P, list(order), act)
                    assert _rel(Y, ref) <= 1e-13, (T, d, f, act, P, order)


def pin_silu(o):
    assert o.silu(np.array([0.0]))[0] == 0.0
    for k in (2, 3, 7):
        x = math.log(k)                       # sigmoid(ln k) = k / (k + 1)
        assert abs(o.silu(np.array([x]))[0] - k / (k + 1) * x) <= 4e-16 * x
    xs = np.linspace(-30, 30, 601)
    assert np.max(np.abs(o.silu(xs) - o.silu(-xs) - xs)) <= 1e-14   # SiLU(x) - SiLU(-x) = x
    assert np.all(o.silu(np.array([-1e3, -1e5])) == 0.0)           # limit, no NaN
    assert abs(o.silu(np.array([50.0]))[0] / 50.0 - 1.0) <= 1e-15
    assert o.silu(np.array([1.0]))[0] > 0.7 and o.silu(np.array([-1.0]))[0] < 0


def _gelu_tanh_decimal(x):
    getcontext().prec = 50
    pi = Decimal("3.14159265358979323846264338327950288419716939937510")
    x = Decimal(x)
    z = (Decimal(2) / pi).sqrt() * (x + Decimal("0.044715") * x ** 3)
    e = (2 * z).exp()
    return Decimal("0.5") * x * (1 + (e - 1) / (e + 1))


def pin_gelu(o):
    assert o.gelu_tanh(np.array([0.0]))[0] == 0.0
    xs = np.linspace(-8, 8, 16001)
    gt = o.gelu_tanh(xs)
    assert np.max(np.abs(gt - o.gelu_tanh(-xs) - xs)) <= 1e-14      # odd part is x / 2
    exact = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in xs])
    dev = np.abs(gt - exact)
    assert dev.max() <= 5e-4          # the tanh form approximates the erf form closely ...
    assert dev.max() >= 1e-4          # ... but is not the erf form
    x = 1e-4                          # second-order Taylor: 0.5 x + x^2 / sqrt(2 pi)
    assert abs(o.gelu_tanh(np.array([x]))[0] - (0.5 * x + x * x / math.sqrt(2 * math.pi))) <= 1e-15
    for xv in ("1", "-0.5", "2.25", "-3", "0.125"):
        ref = float(_gelu_tanh_decimal(xv))
        got = o.gelu_tanh(np.array([float(xv)]))[0]
        assert abs(got - ref) <= 4e-16 * max(abs(ref), abs(float(xv))), (xv, got, ref)


def pin_identity_weights(o):
    d = 16
    X = np.random.default_rng(5).standard_normal((5, d)) * 3
    I = np.eye(d)
    for P in (1, 2, 4, 16):
        Y = o.mlp_forward(X, I, I, I, P, o.ring_order(P, 1), "swiglu")
        assert _rel(Y, X / (1.0 + np.exp(-X)) * X) <= 1e-15
        Y = o.mlp_forward(X, None, I, I, P, o.ring_order(P, 1), "gelu_tanh")
        ref = np.array([[float(_gelu_tanh_decimal(float(v))) for v in row] for row in X])
        assert _rel(Y, ref) <= 1e-15


def pin_selection_weights(o):
    """0/1 weights pick single inputs: fixes orientation and the gate/up roles."""
    T, d, f, P = 4, 3, 6, 3
    X = np.random.default_rng(9).standard_normal((T, d)) * 2
    a = [0, 1, 2, 2, 1, 0]       # gate of hidden c reads x[a[c]]
    b = [1, 2, 0, 1, 0, 2]       # up of hidden c reads x[b[c]]
    e = [2, 0, 1, 0, 2, 1]       # hidden c feeds output e[c]
    wg = np.zeros((d, f)); wu = np.zeros((d, f)); wd = np.zeros((f, d))
    for c in range(f):
        wg[a[c], c] = 1.0
        wu[b[c], c] = 1.0
        wd[c, e[c]] = 1.0
    ref = np.zeros((T, d))
    for t in range(T):
        for c in range(f):
            g = X[t, a[c]]
            ref[t, e[c]] += g / (1.0 + math.exp(-g)) * X[t, b[c]]
    for order in itertools.permutations(range(P)):
        Y = o.mlp_forward(X, wg, wu, wd, P, list(order), "swiglu")
        assert _rel(Y, ref) <= 1e-15, order


def pin_column_then_row_identity(o):
    T, d, f = 7, 24, 48
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd = _rng_inputs(T, d, f, act, 21)
        ref = o.mlp_forward(X, wg, wu, wd, 1, [0], act)
        for P in [p for p in range(1, f + 1) if f % p == 0]:
            F = f // P
            parts = sum(o.shard_partial(X, wg, wu, wd, s, F, act) for s in range(P))
            assert _rel(parts, ref) <= 1e-13, (act, P)
            for r0 in range(P):
                assert _rel(o.mlp_forward(X, wg, wu, wd, P, o.ring_order(P, r0), act), ref) <= 1e-13
            rng = np.random.default_rng(P)
            for _ in range(3):
                perm = list(rng.permutation(P))
                assert _rel(o.mlp_forward(X, wg, wu, wd, P, perm, act), ref) <= 1e-13
        for P in (1, 2, 4, 8):                # the folded group equals the unsharded block
            S = 8 * P
            Xs = np.random.default_rng(P + 40).standard_normal((S, d))
            full = o.mlp_forward(Xs, wg, wu, wd, 1, [0], act)
            assert _rel(o.tsp_simulate(Xs, wg, wu, wd, P, act, r0=1), full) <= 1e-13


def pin_linearity(o):
    T, d, f, P = 6, 16, 32, 4
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd = _rng_inputs(T, d, f, act, 33)
        Y = o.mlp_forward(X, wg, wu, wd, P, o.ring_order(P, 2), act)
        assert np.all(o.mlp_forward(np.zeros_like(X), wg, wu, wd, P, None, act) == 0.0)
        assert np.all(o.mlp_forward(X, wg, np.zeros_like(wu), wd, P, None, act) == 0.0)
        Y2 = o.mlp_forward(X, wg, wu, 2.0 * wd, P, o.ring_order(P, 2), act)
        assert np.array_equal(Y2, 2.0 * Y)                 # exact: scaling by 2
        if act == "swiglu":
            Y3 = o.mlp_forward(X, wg, 2.0 * wu, wd, P, o.ring_order(P, 2), act)
            assert np.array_equal(Y3, 2.0 * Y)
        perm = np.random.default_rng(1).permutation(d)     # permuting outputs permutes Y
        Y4 = o.mlp_forward(X, wg, wu, wd[:, perm], P, o.ring_order(P, 2), act)
        assert np.array_equal(Y4, Y[:, perm])
        rows = [5, 0, 3]
        Y5 = o.mlp_forward(X, wg, wu, wd, P, o.ring_order(P, 2), act, rows=rows)
        assert np.array_equal(Y5, Y[rows])


def pin_round_bf16(o):
    """bfloat16 round-to-nearest-even: representable values stay, halfway
    cases go to the even neighbour, and fp32 inputs match torch's own
    fp32 -> bfloat16 conversion (a single rounding there too)."""
    exact = np.array([0.0, 1.0, -1.5, 3.25, 2.0 ** -100, -(2.0 ** 90), 255.0, 1.0 + 2.0 ** -7])
    assert np.array_equal(o.round_bf16(exact), exact)
    # near 1 the bfloat16 spacing is 2^-7
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2 + 2.0 ** -7, 2 + 3 * 2.0 ** -7])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 2.0, 2 + 2.0 ** -5])
    assert np.array_equal(o.round_bf16(ties), want)
    assert np.array_equal(o.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30])), np.array([1 + 2.0 ** -7]))
    import torch
    g = torch.Generator().manual_seed(5)
    x = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 8)
    ref = x.to(torch.bfloat16).double().numpy()
    assert np.array_equal(o.round_bf16(x.double().numpy()), ref)
    # rounding H moves each hidden value by at most 2^-9 of itself
    T, d, f, P = 5, 16, 32, 4
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd = _rng_inputs(T, d, f, act, 13)
        Y = o.mlp_forward(X, wg, wu, wd, P, None, act)
        Yr = o.mlp_forward(X, wg, wu, wd, P, None, act, round_h_bf16=True)
        H = np.concatenate([o.shard_hidden(X, wg, wu, s, f // P, act) for s in range(P)], axis=1)
        bound = 2.0 ** -9 * (np.abs(H) @ np.abs(wd)) * (1 + 1e-12)
        assert np.all(np.abs(Yr - Y) <= bound + 1e-15)
        assert not np.array_equal(Yr, Y)


ALL_PINS = [pin_golden, pin_brute_force, pin_silu, pin_gelu, pin_identity_weights,
            pin_selection_weights, pin_column_then_row_identity, pin_linearity, pin_round_bf16]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


def test_row_split_before_nonlinearity_is_wrong():
    """Cutting the first matrix by rows and applying the nonlinearity to the
    partial sums is not the block ("Why the column-then-row split")."""
    T, d, f = 8, 32, 64
    for act in ("swiglu", "gelu_tanh"):
        X, wg, wu, wd = _rng_inputs(T, d, f, act, 77)
        ref = O.mlp_forward(X, wg, wu, wd, 1, [0], act)
        P, Dk = 2, d // 2
        wrong = np.zeros_like(ref)
        for s in range(P):
            ks = slice(s * Dk, (s + 1) * Dk)
            u = X[:, ks] @ wu[ks, :]
            h = O.silu(X[:, ks] @ wg[ks, :]) * u if act == "swiglu" else O.gelu_tanh(u)
            wrong += h @ wd
        assert _rel(wrong, ref) > 0.05


def test_golden_row_split_counterexample():
    e = json.load(open(GOLDEN))["walkthrough_gelu_P2"]
    X, A = _arr(e["X"]), _arr(e["w_up"])
    # token 1, hidden column 0: rows {0,1} of A give 4, row {2} gives -4; GeLU(0) = 0
    a = O.gelu_tanh(X[1, :2] @ A[:2, 0]) + O.gelu_tanh(X[1, 2:] @ A[2:, 0])
    assert abs(a - 0.0) > 3.9


def test_invalid_arguments():
    X, wg, wu, wd = _rng_inputs(2, 4, 6, "swiglu", 1)
    with pytest.raises(ValueError):
        O.mlp_forward(X, wg, wu, wd, 4)                  # 4 does not divide 6
    with pytest.raises(ValueError):
        O.mlp_forward(X, wg, wu, wd, 3, [0, 0, 1])        # not a permutation
    with pytest.raises(ValueError):
        O.mlp_forward(X, None, wu, wd, 3)                 # swiglu without a gate
    with pytest.raises(ValueError):
        O.mlp_forward(X, wg, wu, wd.T, 3)                 # wrong orientation


def test_bf16_inputs_promote_exactly():
    import torch
    t = torch.randn(64, 64).to(torch.bfloat16)
    a = O.f64(t.float().numpy())
    assert np.array_equal(a, t.double().numpy())


# ---------------------------------------------------------------- mutation test

def _mut_silu_sign(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def _mut_gelu_erf(u):
    u = np.asarray(u, dtype=np.float64)
    from scipy.special import erf
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def _mut_gelu_const(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(O.SQRT_2_OVER_PI * (u + 0.0447 * u ** 3)))


def _mut_swap_gate_up(X, w_gate, w_up, s, F, act):
    if act != "swiglu":
        return O.gelu_tanh(O.f64(X) @ O.f64(w_up[:, s * F:(s + 1) * F]))
    return _orig_shard_hidden(X, w_up, w_gate, s, F, act)


def _mut_wrong_down_rows(X, w_gate, w_up, w_down, s, F, act, round_h_bf16=False):
    P = w_down.shape[0] // F
    h = O.shard_hidden(X, w_gate, w_up, s, F, act)
    s2 = (s + 1) % P
    return h @ O.f64(w_down[s2 * F:(s2 + 1) * F, :])


def _mut_drop_last_shard(X, w_gate, w_up, w_down, P, order=None, act="swiglu", rows=None, round_h_bf16=False):
    X = O.f64(X) if rows is None else O.f64(X)[np.asarray(rows)]
    F = w_up.shape[1] // P
    order = O.ring_order(P) if order is None else list(order)
    Y = np.zeros((X.shape[0], X.shape[1]))
    for s in order[:-1]:
        Y += O.shard_partial(X, w_gate, w_up, w_down, s, F, act)
    return Y


def _mut_down_transposed(X, w_gate, w_up, w_down, s, F, act, round_h_bf16=False):
    h = O.shard_hidden(X, w_gate, w_up, s, F, act)
    wt = O.f64(w_down).T if w_down.shape[0] == w_down.shape[1] else O.f64(w_down)
    return h @ wt[s * F:(s + 1) * F, :]


def _mut_gate_cols_shifted(X, w_gate, w_up, s, F, act):
    f = w_up.shape[1]
    if act != "swiglu" or f == F:
        return _orig_shard_hidden(X, w_gate, w_up, s, F, act)
    cols = slice(((s + 1) * F) % f, ((s + 1) * F) % f + F)
    g = O.f64(X) @ O.f64(w_gate[:, cols])
    u = O.f64(X) @ O.f64(w_up[:, s * F:(s + 1) * F])
    return O.silu(g) * u


_orig_shard_hidden = O.shard_hidden

MUTANTS = {
    "silu_sign": ("silu", _mut_silu_sign),
    "gelu_erf": ("gelu_tanh", _mut_gelu_erf),
    "gelu_const": ("gelu_tanh", _mut_gelu_const),
    "swap_gate_up": ("shard_hidden", _mut_swap_gate_up),
    "wrong_down_rows": ("shard_partial", _mut_wrong_down_rows),
    "drop_last_shard": ("mlp_forward", _mut_drop_last_shard),
    "down_transposed": ("shard_partial", _mut_down_transposed),
    "gate_cols_shifted": ("shard_hidden", _mut_gate_cols_shifted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError) as exc:  # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"

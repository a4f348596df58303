"""Pins of the fp64 attention oracle (oracle/attn_oracle.py) against things
other than itself: a pure-Python brute force of the unsplit block, PyTorch's
scaled_dot_product_attention in float64 (a library routine), the identity
that every rank's TSP output equals its rows of the unsplit block for any
visiting order and any P, closed forms (uniform attention when Wq = 0, the
first token seeing only itself), and planted mistakes that must be caught."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle.attn_oracle as ao


def rand_block(seed, S, d, H, Hkv, dh):
    g = np.random.default_rng(seed)
    X = g.standard_normal((S, d))
    Wq = g.standard_normal((d, H * dh)) / math.sqrt(d)
    Wk = g.standard_normal((d, Hkv * dh)) / math.sqrt(d)
    Wv = g.standard_normal((d, Hkv * dh)) / math.sqrt(d)
    Wo = g.standard_normal((H * dh, d)) / math.sqrt(H * dh)
    return X, Wq, Wk, Wv, Wo


def brute_rows(X, Wq, Wk, Wv, Wo, H, Hkv, rows, causal=True):
    """Unsplit attention block, token rows `rows`, in plain Python loops."""
    S, d = len(X), len(X[0])
    dh = len(Wq[0]) // H
    G = H // Hkv

    def proj(W, t, col):
        return sum(X[t][a] * W[a][col] for a in range(d))

    out = []
    for p in rows:
        y = [0.0] * d
        for h in range(H):
            j = h // G
            q = [proj(Wq, p, h * dh + c) for c in range(dh)]
            keys = [t for t in range(S) if t <= p or not causal]
            sc = []
            for t in keys:
                k = [proj(Wk, t, j * dh + c) for c in range(dh)]
                sc.append(sum(q[c] * k[c] for c in range(dh)) / math.sqrt(dh))
            m = max(sc)
            w = [math.exp(v - m) for v in sc]
            z = sum(w)
            o = [0.0] * dh
            for wt, t in zip(w, keys):
                for c in range(dh):
                    o[c] += wt / z * proj(Wv, t, j * dh + c)
            for c in range(dh):
                for n in range(d):
                    y[n] += o[c] * Wo[h * dh + c][n]
        out.append(y)
    return np.array(out)


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    S, d, H, Hkv, dh, P = 6, 3, 4, 2, 2, 2
    X, Wq, Wk, Wv, Wo = rand_block(1, S, d, H, Hkv, dh)
    T = S // P
    for r in range(P):
        ref = brute_rows(X.tolist(), Wq.tolist(), Wk.tolist(), Wv.tolist(), Wo.tolist(), H, Hkv,
                         range(r * T, (r + 1) * T), causal)
        got = ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, r, causal=causal)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("H,Hkv,causal", [(4, 4, True), (8, 2, True), (4, 1, False), (6, 3, True)])
def test_unsharded_matches_torch_sdpa(H, Hkv, causal):
    S, d, dh = 37, 24, 8
    X, Wq, Wk, Wv, Wo = rand_block(2, S, d, H, Hkv, dh)
    q = torch.from_numpy(X @ Wq).reshape(S, H, dh).transpose(0, 1)
    k = torch.from_numpy(X @ Wk).reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(H // Hkv, dim=0)
    v = torch.from_numpy(X @ Wv).reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(H // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ref = o.transpose(0, 1).reshape(S, H * dh).numpy() @ Wo
    got = ao.attention_unsharded(X, Wq, Wk, Wv, Wo, H, Hkv, causal)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("P", [1, 2, 4])
def test_every_rank_equals_unsharded_rows_any_order(P):
    S, d, H, Hkv, dh = 32, 16, 8, 4, 4
    X, Wq, Wk, Wv, Wo = rand_block(3, S, d, H, Hkv, dh)
    full = ao.attention_unsharded(X, Wq, Wk, Wv, Wo, H, Hkv)
    T = S // P
    orders = list(itertools.permutations(range(P))) if P <= 3 else [None, [3, 1, 0, 2], [0, 1, 2, 3]]
    for r in range(P):
        for order in orders:
            got = ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, r, order=order)
            np.testing.assert_allclose(got, full[r * T:(r + 1) * T], rtol=0, atol=1e-12 * np.max(np.abs(full)))


def test_zero_queries_give_prefix_means():
    """Wq = 0: every visible key scores 0, so each query averages the values
    of positions 0..p (a cumulative mean, no softmax involved)."""
    S, d, H, Hkv, dh, P = 24, 12, 4, 2, 3, 2
    X, _, Wk, Wv, Wo = rand_block(4, S, d, H, Hkv, dh)
    Wq = np.zeros((d, H * dh))
    V = (X @ Wv).reshape(S, Hkv, dh)
    mean = np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None, None]
    O = np.repeat(mean, H // Hkv, axis=1).reshape(S, H * dh)
    ref = O @ Wo
    T = S // P
    for r in range(P):
        got = ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, r)
        np.testing.assert_allclose(got, ref[r * T:(r + 1) * T], rtol=0, atol=1e-13)


def test_first_token_sees_only_itself():
    S, d, H, Hkv, dh, P = 8, 6, 2, 2, 3, 2
    X, Wq, Wk, Wv, Wo = rand_block(5, S, d, H, Hkv, dh)
    got = ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, 0)[0]
    ref = (X[0] @ Wv) @ Wo                               # one visible key: its value, projected
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_flop_count():
    T, d, H, Hkv, dh, P, r = 5, 8, 4, 2, 2, 3, 1
    pairs = sum(1 for i in range(T) for j in range(P * T) if j <= r * T + i)
    assert ao.attention_flops(T, d, H, Hkv, dh, P, r) == 2 * T * d * dh * (2 * H + 2 * Hkv) + 4 * dh * H * pairs
    assert ao.attention_flops(T, d, H, Hkv, dh, P, r, causal=False) == (
        2 * T * d * dh * (2 * H + 2 * Hkv) + 4 * dh * H * T * P * T)


# ---- planted mistakes in the oracle must be caught by the pins above

def _case():
    S, d, H, Hkv, dh, P = 24, 12, 8, 4, 3, 2         # two key/value heads per head group
    return rand_block(7, S, d, H, Hkv, dh), (H, Hkv, P)


def _matches_unsharded():
    (X, Wq, Wk, Wv, Wo), (H, Hkv, P) = _case()
    full = ao.attention_unsharded(X, Wq, Wk, Wv, Wo, H, Hkv)
    T = len(X) // P
    return all(np.allclose(ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, r), full[r * T:(r + 1) * T],
                           rtol=0, atol=1e-10) for r in range(P))


def _matches_brute():
    (X, Wq, Wk, Wv, Wo), (H, Hkv, P) = _case()
    T = len(X) // P
    r = P - 1
    ref = brute_rows(X.tolist(), Wq.tolist(), Wk.tolist(), Wv.tolist(), Wo.tolist(), H, Hkv,
                     range(r * T, (r + 1) * T))
    return np.allclose(ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, r), ref, rtol=0, atol=1e-10)


def test_unmutated_oracle_passes_both_checks():
    assert _matches_unsharded() and _matches_brute()


def _mutant(monkeypatch, wrap):
    orig = ao.attention_heads
    monkeypatch.setattr(ao, "attention_heads", lambda Q, K, V, qp, kp, causal, group: wrap(orig, Q, K, V, qp, kp,
                                                                                          causal, group))


def test_mutant_scale_dropped(monkeypatch):
    _mutant(monkeypatch, lambda f, Q, K, V, qp, kp, c, g: f(Q * math.sqrt(Q.shape[2]), K, V, qp, kp, c, g))
    assert not _matches_brute()


def test_mutant_head_mapping_modulo(monkeypatch):
    def wrap(f, Q, K, V, qp, kp, c, g):
        idx = [h % K.shape[1] for h in range(Q.shape[1])]   # h % Hkv instead of h // group
        return f(Q, K[:, idx], V[:, idx], qp, kp, c, 1)
    _mutant(monkeypatch, wrap)
    assert not _matches_brute()


def test_mutant_local_positions(monkeypatch):
    _mutant(monkeypatch, lambda f, Q, K, V, qp, kp, c, g: f(Q, K, V, qp - qp[0], kp, c, g))
    assert not _matches_unsharded()


def test_mutant_no_exchange(monkeypatch):
    def wrap(f, Q, K, V, qp, kp, c, g):
        own = (kp >= qp[0]) & (kp <= qp[-1])              # the rank's own keys only
        return f(Q, K[own], V[own], qp, kp[own], c, g)
    _mutant(monkeypatch, wrap)
    assert not _matches_unsharded()


def test_row_subset_equals_full_rows():
    S, d, H, Hkv, dh, P = 32, 16, 4, 2, 4, 2
    X, Wq, Wk, Wv, Wo = rand_block(8, S, d, H, Hkv, dh)
    full = ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, 1)
    rows = [0, 5, 15]
    np.testing.assert_array_equal(ao.tsp_attention(X, Wq, Wk, Wv, Wo, H, Hkv, P, 1, rows=rows), full[rows])

"""fp64 CPU oracle for one rank's attention block under TSP (tensor and
sequence parallelism on one device axis).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call
this module: only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` use it. It shares no code with the HIP path
and imports nothing from the package.

What it computes, and where that is stated:

* "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
  Training & Inference", Abstract: each rank holds one parameter shard and
  one sequence shard; for attention the ranks go through the parameter shards
  one after another (each broadcast by its owner) and rebuild the full
  context by exchanging keys and values along the sequence.
* "Tensor Parallelism: Splitting the Math", section "Why the column-then-row
  split - and what happens in attention": attention heads are independent,
  so the Q, K and V projections split by columns (a device owns whole heads
  and runs their attention locally) and the output projection splits by
  rows, the matching partial outputs summing to the unsplit result.
* "Tensor Parallelism" (AI terminology page), table "Key Points", row
  "Attention split": a device owns a contiguous range of heads.

So rank r, holding tokens X_r = rows [r T, (r+1) T) of an S = P T token
sequence, does for k = 0..P-1 with s = order[k]: project its tokens with the
head group s columns of Wq, Wk, Wv; gather every rank's K and V rows of head
group s (the sequence-wise exchange: rank rho supplies X_rho Wk_s, X_rho Wv_s);
attend with its queries over that full context; multiply by the head group s
rows of Wo and add the product into its output Y_r.

Readings where the pages are silent:

* scaled dot-product softmax attention with scale 1/sqrt(dh); no bias terms,
  no rotary or other position encoding, no dropout;
* causal (a decoder's training step): a query at sequence position p sees
  keys at positions <= p; the non-causal form is kept as an option;
* grouped query heads: H query heads share Hkv key/value heads, query head h
  using key/value head h // (H / Hkv); head group s owns query heads
  [s H/P, (s+1) H/P) and key/value heads [s Hkv/P, (s+1) Hkv/P) (P divides
  Hkv);
* sequence shards are contiguous and equal, rank r owning positions
  [r T, (r+1) T);
* orientation Y = X W, W stored input x output; head h occupies columns
  [h dh, (h+1) dh) of Wq (rows of Wo), key/value head j columns
  [j dh, (j+1) dh) of Wk and Wv.

Matrix products are numpy's float64 matmul used as a library step, the
softmax is written out; there is no blocking, no online softmax and no fusion.
Inputs are promoted exactly to float64.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def attention_heads(Q, K, V, q_pos, k_pos, causal: bool, group: int) -> np.ndarray:
    """Softmax attention per head.

    Q: Tq x Hq x dh, K and V: Tk x Hk x dh, Hq = group * Hk; query head h reads
    key/value head h // group. q_pos (Tq) and k_pos (Tk) are sequence
    positions; with ``causal`` a key is visible to a query when
    k_pos <= q_pos. Returns Tq x Hq x dh.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    Tq, Hq, dh = Q.shape
    out = np.empty_like(Q)
    visible = (np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]) if causal else None
    for h in range(Hq):
        j = h // group
        scores = (Q[:, h, :] @ K[:, j, :].T) / np.sqrt(dh)
        if visible is not None:
            scores = np.where(visible, scores, -np.inf)
        m = np.max(scores, axis=1, keepdims=True)
        e = np.exp(scores - m)
        p = e / np.sum(e, axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, j, :]
    return out


def head_columns(s: int, heads_per_shard: int, dh: int) -> slice:
    """Columns of Wq (rows of Wo) or of Wk/Wv owned by head group s."""
    return slice(s * heads_per_shard * dh, (s + 1) * heads_per_shard * dh)


def attention_unsharded(X, Wq, Wk, Wv, Wo, H: int, Hkv: int, causal: bool = True) -> np.ndarray:
    """The plain multi-head attention block over a whole sequence X (S x d):
    Y = concat_h(attention_h) Wo. The definition TSP must reproduce."""
    X = _f64(X)
    S = X.shape[0]
    dh = Wq.shape[1] // H
    Q = (X @ _f64(Wq)).reshape(S, H, dh)
    K = (X @ _f64(Wk)).reshape(S, Hkv, dh)
    V = (X @ _f64(Wv)).reshape(S, Hkv, dh)
    pos = np.arange(S)
    O = attention_heads(Q, K, V, pos, pos, causal, H // Hkv)
    return O.reshape(S, H * dh) @ _f64(Wo)


def tsp_attention(X_all, Wq, Wk, Wv, Wo, H: int, Hkv: int, P: int, rank: int,
                  order: Optional[Sequence[int]] = None, causal: bool = True,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rank ``rank``'s output rows of the attention block under TSP.

    X_all: the whole S x d sequence (rank rho's tokens are rows
    [rho T, (rho+1) T), T = S / P); the other ranks' rows stand for what the
    key/value exchange delivers. order: the head groups in the order the
    rank visits them (default: rank, rank+1, ... mod P). rows: only these of
    the rank's token rows (queries are independent of each other).
    """
    X_all = _f64(X_all)
    S, d = X_all.shape
    if S % P or H % Hkv or Hkv % P or Wq.shape[1] % H:
        raise ValueError("S, H, Hkv must divide by P (and H by Hkv)")
    T = S // P
    dh = Wq.shape[1] // H
    Hs, Hks = H // P, Hkv // P
    if order is None:
        order = [(rank + k) % P for k in range(P)]
    if sorted(order) != list(range(P)):
        raise ValueError("order must be a permutation of 0..P-1")
    X_r = X_all[rank * T:(rank + 1) * T]
    q_pos = np.arange(rank * T, (rank + 1) * T)
    if rows is not None:
        X_r, q_pos = X_r[np.asarray(rows)], q_pos[np.asarray(rows)]
    Tq = len(q_pos)
    k_pos = np.arange(S)
    Y = np.zeros((Tq, d))
    for s in order:
        cq, ckv = head_columns(s, Hs, dh), head_columns(s, Hks, dh)
        Q = (X_r @ _f64(Wq)[:, cq]).reshape(Tq, Hs, dh)
        # sequence-wise exchange: every rank's keys and values of head group s
        K = np.concatenate([X_all[rho * T:(rho + 1) * T] @ _f64(Wk)[:, ckv] for rho in range(P)])
        V = np.concatenate([X_all[rho * T:(rho + 1) * T] @ _f64(Wv)[:, ckv] for rho in range(P)])
        O = attention_heads(Q, K.reshape(S, Hks, dh), V.reshape(S, Hks, dh), q_pos, k_pos, causal, Hs // Hks)
        Y += O.reshape(Tq, Hs * dh) @ _f64(Wo)[cq, :]
    return Y


def attention_flops(T: int, d: int, H: int, Hkv: int, dh: int, P: int, rank: int, causal: bool = True) -> int:
    """Algorithmic flops of one rank's forward: the four projections of its T
    tokens (Q and output: 2 T d H dh each; K and V: 2 T d Hkv dh each) plus
    the two attention products, 4 dh flops per (query, visible key, head)."""
    S = P * T
    if causal:
        pairs = sum(rank * T + i + 1 for i in range(T))   # keys visible to query i of the rank
    else:
        pairs = T * S
    return 4 * T * d * H * dh + 4 * T * d * Hkv * dh + 4 * dh * H * pairs

"""fp64 CPU oracle for one rank's gated-MLP block under TSP weight sharding.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call
this module: only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` use it. It shares no code with the HIP path
and imports nothing from the package.

What it computes, and where that is stated:

* "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
  Training & Inference", Abstract: TSP gives each rank one weight shard and
  one sequence shard; in the gated MLP the weight shards travel round a ring
  and each rank adds every shard's partial output into its own local result.
  On one rank that is: for ring step k = 0..P-1, take shard ``order[k]``,
  compute its partial output for the rank's tokens X, and add it into Y.
* "Tensor Parallelism: Splitting the Math", section "One transformer MLP,
  split across two GPUs (Megatron-style)", steps 2-6: the first weight
  matrix is cut into column blocks, the nonlinearity is applied to each
  block's output on its own, the second matrix is cut into the row blocks
  that match, and the per-block products are partial sums whose total is the
  output of the unsplit MLP.
* Same page, section "Why the column-then-row split": the split has to be
  by columns of the first matrix because the nonlinearity is elementwise and
  does not distribute over a sum.

Readings where the pages are silent:

* gated activation = SwiGLU, h = SiLU(x.Wg) * (x.Wu) with SiLU(g) = g/(1+e^-g);
* the non-gated block uses the tanh form of GeLU,
  0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)));
* no bias terms; shard s owns hidden columns [s*F, (s+1)*F), F = f/P, for the
  gate, up (or first) matrices and the same rows of the down (or second)
  matrix;
* ring order is the rotation order[k] = (r0 + k) mod P; any permutation of
  the shards is accepted and gives the same result up to rounding;
* orientation is Y = X W with W stored input x output.

Every matrix product below is numpy's float64 matmul used as a library step;
there is no blocking and no fusion beyond the shard loop the method itself
describes. Inputs are promoted exactly to float64 (bf16 and fp32 values are
representable exactly).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

SQRT_2_OVER_PI = float(np.sqrt(2.0 / np.pi))
GELU_TANH_CUBIC = 0.044715


def f64(a) -> np.ndarray:
    """Exact promotion of an fp32 (or already fp64) array to float64."""
    return np.asarray(a, dtype=np.float64)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU (Swish with beta = 1): g / (1 + exp(-g)).

    For very negative g, exp(-g) overflows to +inf and the quotient is -0.0,
    which is the function's limit; the overflow warning is silenced.
    """
    g = f64(g)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GeLU in its tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = f64(u)
    return 0.5 * u * (1.0 + np.tanh(SQRT_2_OVER_PI * (u + GELU_TANH_CUBIC * u * u * u)))


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (the fp32 exponent range). With
    a = m * 2**e and 0.5 <= |m| < 1, m * 2**8 is rounded to an integer (numpy
    rounds halves to even) and scaled back; every step but the rounding is an
    exact power-of-two scaling. Covers the normal range only (no bfloat16
    subnormals or overflow occur in this block). Diagnostic use: it lets a test
    give the oracle the same rounding of the hidden activations that the bf16
    kernels apply before the down product.
    """
    m, e = np.frexp(f64(a))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


round_bf16_fn = round_bf16


def ring_order(P: int, r0: int = 0) -> list:
    """Rotated ring order: at step k the rank holds shard (r0 + k) mod P."""
    return [(r0 + k) % P for k in range(P)]


def _check_order(order: Sequence[int], P: int) -> list:
    order = [int(s) for s in order]
    if sorted(order) != list(range(P)):
        raise ValueError(f"order {order} is not a permutation of 0..{P - 1}")
    return order


def shard_hidden(X, w_gate, w_up, s: int, F: int, act: str) -> np.ndarray:
    """Hidden activations of shard s: the block's columns [s*F, (s+1)*F).

    Column-parallel step (Megatron walk-through, steps 2-3): each shard owns
    complete columns of X.W, so the nonlinearity is exact on its own block.
    """
    cols = slice(s * F, (s + 1) * F)
    u = f64(X) @ f64(w_up[:, cols])
    if act == "swiglu":
        g = f64(X) @ f64(w_gate[:, cols])
        return silu(g) * u
    if act == "gelu_tanh":
        return gelu_tanh(u)
    raise ValueError(f"unknown activation {act!r}")


def shard_partial(X, w_gate, w_up, w_down, s: int, F: int, act: str,
                  round_h_bf16: bool = False) -> np.ndarray:
    """Shard s's partial output H_s . W_down[rows of shard s, :] (walk-through steps 4-5).

    ``round_h_bf16`` (diagnostic, never the pass/fail reference) rounds H_s to
    bfloat16 first, as the bf16 kernels store it.
    """
    h = shard_hidden(X, w_gate, w_up, s, F, act)
    if round_h_bf16:
        h = round_bf16(h)
    return h @ f64(w_down[s * F:(s + 1) * F, :])


def mlp_forward(X, w_gate, w_up, w_down, P: int, order: Optional[Sequence[int]] = None,
                act: str = "swiglu", rows=None, round_h_bf16: bool = False) -> np.ndarray:
    """One rank's TSP gated-MLP forward in float64.

    X: T x d; w_gate, w_up: d x f (w_gate None for gelu_tanh, where w_up is the
    first matrix A); w_down: d x f's partner, f x d. P must divide f. The rank
    visits shard order[k] at ring step k and adds its partial output into the
    local fp64 accumulator Y (TSP abstract; walk-through step 6 with the
    all-reduce replaced by this local sum). ``rows`` restricts the token rows
    (rows are independent: the block is applied token by token).
    ``round_h_bf16`` is the diagnostic form of ``shard_partial``.
    """
    X = f64(X)
    if rows is not None:
        X = X[np.asarray(rows)]
    T, d = X.shape
    f = w_up.shape[1]
    if w_up.shape[0] != d or w_down.shape != (f, d):
        raise ValueError("shape mismatch")
    if act == "swiglu" and (w_gate is None or w_gate.shape != (d, f)):
        raise ValueError("swiglu needs a d x f gate matrix")
    if P < 1 or f % P:
        raise ValueError(f"P={P} must divide f={f}")
    F = f // P
    order = _check_order(ring_order(P) if order is None else order, P)
    Y = np.zeros((T, d), dtype=np.float64)
    for s in order:
        Y += shard_partial(X, w_gate, w_up, w_down, s, F, act, round_h_bf16)
    return Y


def tsp_simulate(X_full, w_gate, w_up, w_down, P: int, act: str = "swiglu",
                 r0: int = 0) -> np.ndarray:
    """All P ranks of a TSP group, simulated one after another.

    The sequence (S tokens) is cut into P contiguous sequence shards; rank r
    holds tokens [r*S/P, (r+1)*S/P) and, since the shards circulate, visits
    weight shard (r + r0 + k) mod P at step k. Returns the ranks' outputs
    concatenated in sequence order. P must divide S.
    """
    X_full = f64(X_full)
    S = X_full.shape[0]
    if S % P:
        raise ValueError("P must divide the sequence length")
    n = S // P
    outs = []
    for r in range(P):
        outs.append(mlp_forward(X_full[r * n:(r + 1) * n], w_gate, w_up, w_down, P,
                                ring_order(P, (r + r0) % P), act))
    return np.concatenate(outs, axis=0)


# ---------------------------------------------------------------- backward
#
# The pages name the backward pass only as the other half of a training step
# ("Tensor Parallelism: Splitting the Math", the paragraph after the
# walk-through: the split synchronises in the forward and in the backward
# pass; "Folding Tensor and Sequence Parallelism ...", Abstract: the method is
# for training). Reading taken: the backward of one
# rank's block is the exact gradient of the forward above for a loss whose
# gradient with respect to Y is dY. The rank visits the shards in the same ring
# order; for shard s it forms that shard's part of dX (added into a local
# accumulator, as Y is in the forward) and the full gradient of shard s's
# weight blocks (columns [s*F, (s+1)*F) of the gate and up matrices, the same
# rows of the down matrix), which go back to the shard's owner. Everything is
# the chain rule applied to shard_hidden / shard_partial; numpy's matmul is the
# only library step.


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d SiLU / dg = sigma(g) (1 + g (1 - sigma(g))), sigma(g) = 1 / (1 + e^-g).

    For very negative g, e^-g overflows, sigma is 0 and so is the derivative.
    """
    g = f64(g)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 + g * (1.0 - sig))


def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d/du of 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3):
    0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) sqrt(2/pi) (1 + 3 * 0.044715 u^2)."""
    u = f64(u)
    th = np.tanh(SQRT_2_OVER_PI * (u + GELU_TANH_CUBIC * u * u * u))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_TANH_CUBIC * u * u)


def shard_backward(X, w_gate, w_up, w_down, dY, s: int, F: int, act: str,
                   round_bf16: bool = False):
    """Gradients from shard s: (part of dX, dWg block, dWu block, dWd block).

    With G = X.Wg_s, U = X.Wu_s (or U = X.A_s), H = act(G, U), Y_s = H.Wd_s:
    dH = dY.Wd_s^T; SwiGLU: dG = dH * U * SiLU'(G), dU = dH * SiLU(G); GeLU:
    dU = dH * GeLU'(U); dX_s = dG.Wg_s^T + dU.Wu_s^T; dWg_s = X^T.dG,
    dWu_s = X^T.dU, dWd_s = H^T.dY. ``round_bf16`` (diagnostic only) rounds
    dG, dU and H to bfloat16 before the products that consume them, as the
    bf16 kernels store them.
    """
    X, dY = f64(X), f64(dY)
    cols = slice(s * F, (s + 1) * F)
    wu = f64(w_up[:, cols])
    wd = f64(w_down[cols, :])
    u = X @ wu
    dH = dY @ wd.T
    rb = round_bf16_fn if round_bf16 else (lambda a: a)
    if act == "swiglu":
        wg = f64(w_gate[:, cols])
        g = X @ wg
        sg = silu(g)
        h = rb(sg * u)
        dG = rb(dH * u * silu_grad(g))
        dU = rb(dH * sg)
        dX = dG @ wg.T + dU @ wu.T
        dWg = X.T @ dG
    elif act == "gelu_tanh":
        h = rb(gelu_tanh(u))
        dU = rb(dH * gelu_tanh_grad(u))
        dX = dU @ wu.T
        dWg = None
    else:
        raise ValueError(f"unknown activation {act!r}")
    return dX, dWg, X.T @ dU, h.T @ dY


def mlp_backward(X, w_gate, w_up, w_down, dY, P: int, order: Optional[Sequence[int]] = None,
                 act: str = "swiglu", round_bf16: bool = False) -> dict:
    """One rank's TSP gated-MLP backward in float64.

    Returns {"dX": T x d, "dW_gate": d x f (None for gelu_tanh), "dW_up": d x f,
    "dW_down": f x d}. Ring step k visits shard order[k]; its dX part is added
    into the local accumulator and its weight-gradient blocks are stored at the
    shard's own columns / rows.
    """
    X, dY = f64(X), f64(dY)
    T, d = X.shape
    f = w_up.shape[1]
    if dY.shape != (T, d) or w_up.shape[0] != d or w_down.shape != (f, d):
        raise ValueError("shape mismatch")
    if act == "swiglu" and (w_gate is None or w_gate.shape != (d, f)):
        raise ValueError("swiglu needs a d x f gate matrix")
    if P < 1 or f % P:
        raise ValueError(f"P={P} must divide f={f}")
    F = f // P
    order = _check_order(ring_order(P) if order is None else order, P)
    dX = np.zeros((T, d))
    dWg = np.zeros((d, f)) if act == "swiglu" else None
    dWu = np.zeros((d, f))
    dWd = np.zeros((f, d))
    for s in order:
        cols = slice(s * F, (s + 1) * F)
        px, pg, pu, pd = shard_backward(X, w_gate, w_up, w_down, dY, s, F, act, round_bf16)
        dX += px
        if pg is not None:
            dWg[:, cols] = pg
        dWu[:, cols] = pu
        dWd[cols, :] = pd
    return {"dX": dX, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd}


def mlp_backward_columns(X, w_gate, w_up, w_down, dY, cols, act: str = "swiglu") -> dict:
    """Weight gradients restricted to hidden columns ``cols`` (any subset of
    0..f-1): dW_gate[:, cols], dW_up[:, cols], dW_down[cols, :]. Each hidden
    column's gradients depend only on that column (every token row is
    needed), so large shapes can be checked on sampled columns. Same formulas
    as shard_backward, evaluated column by column block."""
    X, dY = f64(X), f64(dY)
    cols = np.asarray(cols)
    wu = f64(w_up[:, cols])
    wd = f64(w_down[cols, :])
    u = X @ wu
    dH = dY @ wd.T
    if act == "swiglu":
        g = X @ f64(w_gate[:, cols])
        sg = silu(g)
        h = sg * u
        dG = dH * u * silu_grad(g)
        dU = dH * sg
        dWg = X.T @ dG
    else:
        h = gelu_tanh(u)
        dU = dH * gelu_tanh_grad(u)
        dWg = None
    return {"dW_gate": dWg, "dW_up": X.T @ dU, "dW_down": h.T @ dY}


def backward_flops(T: int, d: int, f: int, act: str) -> int:
    """GEMM flops of one backward's gradients (2 per multiply-add): dH, then
    dX, dW of the first matrices (two each for SwiGLU), dW of the down matrix.
    A recomputation of the forward's hidden activations is not counted."""
    return 2 * (6 if act == "swiglu" else 4) * T * d * f


def flops(T: int, d: int, f: int, act: str) -> int:
    """GEMM flops of one forward: 2 per multiply-add, three matrices (two for GeLU)."""
    return 2 * (3 if act == "swiglu" else 2) * T * d * f

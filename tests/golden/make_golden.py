"""Writes worked_examples.json: small integer worked examples with exact answers.

The pages print no numbers for the sharded MLP, so these fixtures instantiate
the structure they describe with integer data chosen in the activations'
saturated regime, where float64 evaluation of both nonlinearities is exact:

* tanh-form GeLU: for u >= 8 the tanh argument exceeds 24, tanh rounds to
  exactly 1.0 and GeLU(u) == u; for u <= -8 it rounds to exactly -1.0 and
  GeLU(u) == 0; GeLU(0) == 0.
* SiLU: for g >= 40, exp(-g) < 2^-57 so 1 + exp(-g) rounds to 1.0 and
  SiLU(g) == g; for g <= -750, exp(-g) overflows and SiLU(g) == -0.0;
  SiLU(0) == 0.

Under those conditions the whole block is integer arithmetic, so the expected
outputs below are computed here with Python integers only (no oracle, no GPU
code) and are exact. Run from the repository root:
``python tests/golden/make_golden.py``.
"""
import json
import os


def matmul(a, b):
    return [[sum(a[i][k] * b[k][j] for k in range(len(b))) for j in range(len(b[0]))]
            for i in range(len(a))]


def relu_exact_gelu(u):
    assert u == 0 or abs(u) >= 8, u
    return u if u > 0 else 0


def relu_exact_silu(g):
    assert g == 0 or g >= 40 or g <= -750, g
    return g if g > 0 else 0


def walkthrough_gelu():
    # "Tensor Parallelism: Splitting the Math", section "One transformer MLP,
    # split across two GPUs (Megatron-style)": Y = GeLU(X.A).B with A cut into
    # two column halves A1 | A2 and B into the matching row halves.
    X = [[2, -1, 3], [1, 4, -2]]
    A = [[4, 0, 5, -3], [0, -8, 2, 1], [2, 0, 1, -4]]
    B = [[1, 0, -1], [2, 1, 0], [0, -1, 3], [1, 1, 1]]
    U = matmul(X, A)
    H = [[relu_exact_gelu(u) for u in row] for row in U]
    Y = matmul(H, B)
    F = 2
    partials = []
    for s in range(2):
        Hs = [row[s * F:(s + 1) * F] for row in H]
        Bs = B[s * F:(s + 1) * F]
        partials.append(matmul(Hs, Bs))
    assert all(partials[0][i][j] + partials[1][i][j] == Y[i][j]
               for i in range(len(Y)) for j in range(len(Y[0])))
    return {
        "cite": "Tensor Parallelism: Splitting the Math -- section 'One transformer MLP, "
                "split across two GPUs (Megatron-style)', steps 1-7; activations in the "
                "saturated regime so float64 evaluation is exact",
        "act": "gelu_tanh", "P": 2,
        "X": X, "w_gate": None, "w_up": A, "w_down": B,
        "pre_activation": U, "hidden": H,
        "partials_by_shard": partials, "Y": Y,
    }


def ring_swiglu():
    # "Folding Tensor and Sequence Parallelism ...", Abstract: weight shards
    # circulate in a ring and partial outputs accumulate locally. P = 4
    # shards of a gated (SwiGLU) block; every ring rotation must give Y.
    X = [[1, 2, 1, 3], [2, 1, 4, 1], [3, 3, 1, 2]]          # positive entries
    # gate columns: all entries >= 10 (g >= 40), all zero (g = 0) or <= -200 (g <= -750)
    big, zero, neg = 10, 0, -200
    Wg_cols = [[big, 11, 12, big], [zero] * 4, [neg, -210, neg, -220], [13, big, big, 14],
               [zero] * 4, [big, big, 15, big], [neg] * 4, [12, 12, 10, 11]]
    Wg = [[Wg_cols[c][i] for c in range(8)] for i in range(4)]
    Wu = [[1, -2, 3, 0, 1, -1, 2, 1],
          [0, 1, -1, 2, 3, 0, -2, 1],
          [2, 0, 1, -3, 0, 1, 1, -1],
          [-1, 3, 0, 1, -2, 2, 0, 1]]
    Wd = [[1, 0, -1, 2], [0, 2, 1, -1], [3, -1, 0, 1], [1, 1, 1, 0],
          [-2, 0, 1, 1], [0, 1, -1, 3], [1, -3, 2, 0], [2, 1, 0, -1]]
    G = matmul(X, Wg)
    U = matmul(X, Wu)
    H = [[relu_exact_silu(G[t][c]) * U[t][c] for c in range(8)] for t in range(3)]
    Y = matmul(H, Wd)
    return {
        "cite": "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer "
                "Training & Inference -- Abstract (gated MLP: shards circulate in a ring, "
                "partials accumulate locally); SiLU saturated so float64 is exact",
        "act": "swiglu", "P": 4,
        "X": X, "w_gate": Wg, "w_up": Wu, "w_down": Wd,
        "gate_pre_activation": G, "up_pre_activation": U, "hidden": H, "Y": Y,
    }


def main():
    out = {"walkthrough_gelu_P2": walkthrough_gelu(), "ring_swiglu_P4": ring_swiglu()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

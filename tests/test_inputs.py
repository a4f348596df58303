"""The seeded generator is frozen: per-tensor checksums of every workload.

If a torch upgrade changes the random stream, these fail before any parity
number silently moves.
"""
import math

import pytest
import torch

from sharded_transformer_mlp_amd.inputs import WORKLOADS, make_inputs, n_outlier_rows, sample_rows

# name -> {tensor: (sum, sum of squares, first three values)}, fp64 sums of the stored values
FROZEN = {
    "tiny-f32-swiglu-T64-d256-f1024-P2": {
        "x": (-124.11269989912398, 16522.110311606775, [-1.1258398294448853, -1.152360200881958, -0.2505785822868347]),
        "w_gate": (-49.85175637617249, 1023.5868317274757, [-0.03448975458741188, 0.09623795747756958, 0.06272242218255997]),
        "w_up": (-19.291440156809898, 1026.1754109313897, [0.048159919679164886, -0.002935579279437661, 0.031140580773353577]),
        "w_down": (5.822132667094436, 255.18966902144638, [0.03768981993198395, 0.024939773604273796, -0.014169270172715187])},
    "megatron-gelu-bf16-T2048-d4096-f16384-P2": {
        "x": (-231.38727228424978, 8395484.010020405, [-1.5234375, -0.75, -0.65234375]),
        "w_up": (47.20756435088606, 16380.29978562468, [-0.0216064453125, 0.005859375, 0.0157470703125]),
        "w_down": (73.99684553785278, 4096.827464443262, [-0.0068359375, 0.006256103515625, 0.0078125])},
    "llama3-8b-swiglu-bf16-T4096-d4096-f14336-P8": {
        "x": (-998.7104127709754, 16767546.267841818, [-1.0390625, 0.91796875, -1.3046875]),
        "w_gate": (77.43029108245469, 14341.327155009109, [-0.014404296875, 0.0108642578125, -0.0244140625]),
        "w_up": (78.5454236739572, 14339.966280078515, [0.01031494140625, -0.0174560546875, -0.004791259765625]),
        "w_down": (-146.64056041034974, 4095.1845122906116, [0.0013885498046875, 4.0531158447265625e-05, 0.00075531005859375])},
    "70b-long-swiglu-bf16-T16384-d8192-f28672-P8": {
        "x": (2921.5367556027195, 218795337.25343895, [-0.07666015625, 0.359375, -0.78125]),
        "w_gate": (267.9391701928861, 28672.226480145706, [-0.006744384765625, 0.011474609375, 0.005096435546875]),
        "w_up": (-42.00014923122626, 28670.39460365825, [0.0087890625, -0.000408172607421875, 0.0028533935546875]),
        "w_down": (-119.16671642206518, 8192.54334948114, [0.00885009765625, 0.00848388671875, -0.0054931640625])},
    "70b-decode-swiglu-bf16-T16-d8192-f28672-P8": {
        "x": (-505.9071483016014, 131049.52444034774, [-0.94140625, 1.265625, -0.18359375]),
        "w_gate": (65.56023881555757, 28672.153447112178, [-0.0036163330078125, 0.00958251953125, 0.002227783203125]),
        "w_up": (-58.49764545764674, 28675.16439116496, [-0.0042724609375, -0.002288818359375, 0.0205078125]),
        "w_down": (-139.48782308297461, 8191.906936447371, [-0.003936767578125, 0.000957489013671875, -0.00042724609375])},
}


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_frozen_checksums(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    want = FROZEN[name]
    for key in ("x", "w_gate", "w_up", "w_down"):
        t = getattr(inp, key)
        if key not in want:
            assert t is None
            continue
        assert t.dtype == (torch.float32 if w.dtype == "f32" else torch.bfloat16)
        a = t.double()
        s, ss, first = want[key]
        assert math.isclose(float(a.sum()), s, rel_tol=1e-9, abs_tol=1e-9), key
        assert math.isclose(float((a * a).sum()), ss, rel_tol=1e-12), key
        assert [float(v) for v in t.flatten()[:3]] == first, key
    shapes = {"x": (w.T, w.d), "w_up": (w.d, w.f), "w_down": (w.f, w.d)}
    for key, shp in shapes.items():
        assert tuple(getattr(inp, key).shape) == shp
    if w.outlier_frac:
        assert len(inp.outlier_rows) == n_outlier_rows(w.T, w.outlier_frac) == 164
        assert inp.outlier_rows[:5].tolist() == [16116, 8188, 4558, 16128, 8139]


def test_outlier_rows_are_scaled_by_eight():
    w = WORKLOADS["70b-long-swiglu-bf16-T16384-d8192-f28672-P8"].with_(T=512, d=64, f=128)
    inp = make_inputs(w)
    plain = make_inputs(w.with_(outlier_frac=0.0))
    # the permutation draw shifts the weight stream, but X is drawn first
    rows = inp.outlier_rows
    assert len(rows) == 5
    assert torch.equal(inp.x[rows].float(), plain.x[rows].float() * 8)
    mask = torch.ones(512, dtype=torch.bool)
    mask[rows] = False
    assert torch.equal(inp.x[mask], plain.x[mask])


def test_ring_order_and_sizes():
    w = WORKLOADS["llama3-8b-swiglu-bf16-T4096-d4096-f14336-P8"]
    assert w.order() == [3, 4, 5, 6, 7, 0, 1, 2]
    assert w.F == 1792
    assert w.flops() == 6 * 4096 * 4096 * 14336
    assert WORKLOADS["70b-decode-swiglu-bf16-T16-d8192-f28672-P8"].bytes() == \
        3 * 8192 * 28672 * 2 + 16 * 8192 * 2 + 16 * 8192 * 4


def test_sample_rows():
    must = torch.tensor([7, 3, 3])
    r = sample_rows(100, 10, seed=1, must_include=must)
    assert len(r) == 10 and 3 in r.tolist() and 7 in r.tolist()
    assert r.tolist() == sorted(set(r.tolist()))
    assert sample_rows(5, 10, seed=1).tolist() == [0, 1, 2, 3, 4]

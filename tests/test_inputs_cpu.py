"""CPU checks of the seeded input recipes (mxsynth): the shapes, value
distributions and routing structure the parity tests and bench.py use.

The MoE loads are Zipf(1.1) over 128 experts for 20480 tokens x top-8
(163840 rows), capped at 20480 rows per expert (each token sends at most one
row to an expert) with the excess water-filled over the rest in proportion,
largest-remainder rounding.  The first and last sizes below were derived by
hand from that recipe."""
import numpy as np
import torch

import mxsynth


def test_zipf_expert_rows():
    rows = mxsynth.zipf_expert_rows(20480, 128, 8, 1.1)
    assert rows.shape == (128,) and rows.sum() == 163840
    assert (np.diff(rows) <= 0).all() and rows.max() == 20480
    assert rows[:5].tolist() == [20480, 19492, 12478, 9093, 7114]
    assert rows[-3:].tolist() == [204, 203, 201]
    assert (rows < 256).sum() == 26


def test_moe_routing_structure():
    ids, w = mxsynth.moe_routing(num_tokens=2048, num_experts=32, top_k=4)
    rows = mxsynth.zipf_expert_rows(2048, 32, 4, 1.1)
    assert ids.shape == (2048, 4) and w.shape == (2048, 4)
    # distinct experts per token, per-expert counts as the Zipf sizes
    assert all(len(set(r)) == 4 for r in ids.tolist())
    assert np.array_equal(np.bincount(ids.reshape(-1), minlength=32), rows)
    assert (w > 0).all() and np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    ids2, w2 = mxsynth.moe_routing(num_tokens=2048, num_experts=32, top_k=4)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)      # seeded


def test_offsets_from_rows():
    off = mxsynth.offsets_from_rows(np.array([3, 0, 5]))
    assert off.tolist() == [0, 3, 3, 8] and off.dtype == np.int64


def test_normal_bf16_recipe():
    x = mxsynth.normal_bf16((512, 1024), 0.02, seed=7, outlier_frac=0.001, outlier_mul=20.0)
    plain = mxsynth.normal_bf16((512, 1024), 0.02, seed=7)
    assert x.dtype == torch.bfloat16 and x.shape == (512, 1024)
    xf, pf = x.float(), plain.float()
    # the same normal draws; exactly round(0.001 n) of them multiplied by 20
    out = xf.abs() > 5 * pf.abs()
    assert int(out.sum()) == round(0.001 * x.numel())
    assert torch.equal(xf[~out], pf[~out])
    assert abs(pf.std().item() - 0.02) < 0.0005
    y = mxsynth.normal_bf16((512, 1024), 0.02, seed=7, outlier_frac=0.001, outlier_mul=20.0)
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_tiny_workload():
    A, B = mxsynth.tiny()
    assert A.shape == (128, 256) and B.shape == (256, 256)
    a = A.float()
    # four all-zero 32-blocks along A's rows
    blocks = a.reshape(128, 8, 32).abs().amax(dim=2)
    assert int((blocks == 0).sum()) == 4

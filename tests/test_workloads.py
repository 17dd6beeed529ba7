"""Seeded synthetic inputs: determinism and the stated distributions (CPU)."""
import numpy as np

import workloads


def test_same_seed_same_bytes():
    a = workloads.make_moe(3, 64, 32, 6, 2, seed=5, config_id=9, zipf=True)
    b = workloads.make_moe(3, 64, 32, 6, 2, seed=5, config_id=9, zipf=True)
    for nm in ("x", "logits", "gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s", "down_ts"):
        assert np.array_equal(getattr(a, nm), getattr(b, nm)), nm
    c = workloads.make_moe(3, 64, 32, 6, 2, seed=6, config_id=9, zipf=True)
    assert not np.array_equal(a.gate_q, c.gate_q)


def test_draws_independent_of_other_tensors():
    # the x draw of a configuration does not depend on the weight shapes drawn beside it
    a = workloads.make_moe(3, 64, 32, 6, 2, seed=1, config_id=9)
    b = workloads.make_moe(3, 64, 64, 7, 3, seed=1, config_id=9)
    assert np.array_equal(a.x, b.x)


def test_ranges():
    a = workloads.make_moe(16, 256, 128, 8, 2, seed=0, config_id=0)
    assert a.gate_s.min() >= 0x18 and a.gate_s.max() <= 0x48
    assert a.down_ts.min() >= 0.5 and a.down_ts.max() <= 2.0
    assert a.x.dtype == np.uint16 and a.logits.dtype == np.float32
    nib = np.concatenate([a.gate_q & 15, a.gate_q >> 4]).ravel()
    assert np.bincount(nib, minlength=16).min() > 0
    m = workloads.make_mxfp8(2, 64, 128, seed=0)
    assert not np.any((m.w & 0x7F) == 0x7F)
    assert m.s.min() >= 121 and m.s.max() <= 129


def test_named_configs_shapes():
    t = workloads.moe_config("tiny")
    assert (t.T, t.d, t.f, t.E, t.k) == (4, 256, 128, 8, 2)
    d = workloads.moe_config("decode", experts=False)
    assert (d.T, d.d, d.f, d.E, d.k) == (4, 2048, 768, 128, 8)
    assert d.gate_q.size == 0


def test_tp_share_slices_features():
    """The TP share keeps features rank*f/tp .. of gate/up and the matching K range of down."""
    inp = workloads.make_moe(2, 64, 256, 3, 2, seed=2, config_id=91)
    sh = workloads.tp_share(inp, 8, 3)
    assert sh.f == 32 and sh.gate_q.shape == (3, 32, 32) and sh.down_q.shape == (3, 64, 16)
    assert np.array_equal(sh.gate_q, inp.gate_q[:, 96:128]) and np.array_equal(sh.up_s, inp.up_s[:, 96:128])
    assert np.array_equal(sh.down_q, inp.down_q[:, :, 48:64]) and np.array_equal(sh.down_s, inp.down_s[:, :, 6:8])
    assert sh.down_q.flags["C_CONTIGUOUS"] and sh.gate_ts is inp.gate_ts

"""Seeded generators: determinism, rounding, gains and the local-mean query."""
import numpy as np
import torch

from adaptive_sparse_attention_amd import synth


def test_deterministic_and_shapes():
    w = synth.small(130, 64, 1.5, True, B=2, H=3, gain=2.0)
    a = synth.make(w)
    b = synth.make(w)
    for key in ("q", "k", "v", "do"):
        assert a[key].shape == (2, 3, 130, 64)
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    c = synth.make(w.with_(seed=1))
    assert not torch.equal(a["q"], c["q"])


def test_gain_before_rounding_and_rne():
    w = synth.small(64, 64, 1.5, False, B=1, H=1, gain=3.0)
    out = synth.make(w)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 64, 64), dtype=np.float32) * np.float32(3.0)
    # round-to-nearest-even to bf16 by bit manipulation
    bits = q.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    ref = rounded.astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(out["q"].float().numpy(), ref)


def test_fp32_workload_is_exact():
    w = synth.tiny()
    out = synth.make(w)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 256, 64), dtype=np.float32)
    assert out["q"].dtype == torch.float32
    np.testing.assert_array_equal(out["q"].numpy(), q)
    assert "do" not in out


def test_local_mean_query():
    w = synth.Workload("lm", 1, 1, 600, 8, 1.5, True, gain=1.0, local_mean=True, backward=True)
    out = synth.make(w)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 1, 600, 8), dtype=np.float32)
    v = rng.standard_normal((1, 1, 600, 8), dtype=np.float32)
    eps = rng.standard_normal((1, 1, 600, 8), dtype=np.float32)
    for i in (0, 1, 255, 256, 257, 599):
        lo = max(0, i - 256)
        mean = k[0, 0, lo:i].astype(np.float64).mean(axis=0) if i > 0 else 0.0
        ref = (eps[0, 0, i] + 2.0 * mean).astype(np.float32)
        got = out["q"][0, 0, i].float().numpy()
        np.testing.assert_allclose(got, ref, rtol=2 ** -8, atol=1e-6)
    np.testing.assert_array_equal(out["v"].float().numpy(), torch.from_numpy(v).bfloat16().float().numpy())


def test_sampled_blocks():
    w = synth.sweep16k(1.5)
    rows = synth.sample_query_blocks(w)
    assert rows.size == 512
    blocks = np.unique(rows // 64)
    assert blocks.size == 8
    assert np.array_equal(rows, np.sort(rows))
    assert np.array_equal(synth.sample_query_blocks(w), rows)
    assert synth.sample_query_blocks(synth.tiny()).size == 256

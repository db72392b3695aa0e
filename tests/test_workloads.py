"""Seeded synthetic inputs: determinism, distributions, varlen recipe."""
import numpy as np
import torch

from gated_deltanet_chunked_chunk_amd import workloads as W


def test_seeded_determinism():
    w = W.WORKLOADS["gdn_fwd_1x512_h2x2"]
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[key], b[key])
    assert a["initial_state"] is None


def test_distributions():
    w = W.WORKLOADS["gdn_fwd_1x512_h2x2"]
    x = W.make_inputs(w)
    assert x["q"].dtype == torch.bfloat16 and x["k"].dtype == torch.bfloat16 and x["v"].dtype == torch.bfloat16
    assert x["g"].dtype == torch.float32 and x["beta"].dtype == torch.float32
    for key in ("q", "k"):
        n = x[key].float().norm(dim=-1)
        assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert (x["g"] < 0).all()
    assert ((x["beta"] > 0) & (x["beta"] < 1)).all()
    # logsigmoid(N(2,1)): mean log-decay per token about -0.18
    assert -0.25 < x["g"].mean().item() < -0.12
    assert x["scale"] == 128 ** -0.5


def test_varlen_lengths_recipe():
    w = W.WORKLOADS["gdn_fwd_varlen16_65536_h8x24"]
    rng = np.random.default_rng(w.seed)
    lens = W.varlen_lengths(rng, 16, 65536, 512, 16384)
    assert lens.sum() == 65536 and lens.min() >= 512 and lens.max() <= 16384 and len(lens) == 16
    x = W.make_inputs(w, T=65536)
    cu = x["cu_seqlens"].numpy()
    assert cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) >= 512)
    assert x["initial_state"].shape == (16, 24, 128, 128)


def test_reduced_varlen_shapes():
    w = W.WORKLOADS["gdn_fwd_varlen16_65536_h8x24"]
    x = W.make_inputs(w, T=4096, num_seqs=5)
    cu = x["cu_seqlens"].numpy()
    assert len(cu) == 6 and cu[-1] == 4096
    assert x["q"].shape == (1, 4096, 8, 128)

"""Seeded generators: determinism, subset consistency, bf16 rounding."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(0)
    x = np.concatenate([rs.normal(0, 5, 100000), [0.0, -0.0, 1e-40, -3e38, 65504.5]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.to_bf16_bits(x), ref)


def test_generation_is_deterministic_and_subsettable():
    a = workloads.generate(3, B=6)
    b = workloads.generate(3, B=6, threads=1)
    for name in ("target", "draft", "uniforms", "draft_u"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    sub = workloads.generate(3, seqs=[4, 1])
    assert np.array_equal(sub.target, a.target[[4, 1]])
    assert np.array_equal(sub.draft, a.draft[[4, 1]])
    assert np.array_equal(sub.uniforms, a.uniforms[[4, 1]])
    assert a.target.dtype == np.uint16 and a.target.shape == (6, 6, 151936)
    assert ((a.uniforms >= 0) & (a.uniforms < 1)).all()


def test_branch_fanout_shares_target_per_request():
    w = workloads.generate(5, seqs=[0, 1, 15, 16])
    assert np.array_equal(w.target[0], w.target[1])
    assert np.array_equal(w.target[0], w.target[2])
    assert not np.array_equal(w.target[0], w.target[3])
    assert not np.array_equal(w.draft[0], w.draft[1])


def test_recipes_shapes_and_statistics():
    c1 = workloads.generate(1)
    assert c1.target.shape == (1, 5, 1024) and c1.target.dtype == np.float32
    assert abs(c1.target.std() - 2.0) < 0.1
    c2 = workloads.generate(2)
    t = workloads.bf16_bits_to_f32(c2.target)
    assert t.shape == (1, 9, 151936)
    assert (t.max(axis=2) > 8).all()
    c4 = workloads.generate(4, seqs=[0])
    assert c4.target.shape == (1, 9, 262144)
    # Zipf-ranked bias: early token ids carry higher mean logits.
    assert c4.target[0, :, :100].mean() > c4.target[0, :, -1000:].mean() + 5

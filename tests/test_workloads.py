"""The seeded input generators draw what they claim (CPU only)."""
import numpy as np
import pytest
import torch

from combine_moe_layout_amd import workloads


def test_bf16_rounding_of_inputs_matches_torch():
    f = np.random.default_rng(0).standard_normal(100_000).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (workloads.float32_to_bf16_bits(f) == ref).all()


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_shapes_determinism_and_routing(name):
    T0, H, E, G, k, cap, fp8, kind = workloads.CONFIGS[name]
    T = min(T0, 512)
    a = workloads.make(name, T=T)
    b = workloads.make(name, T=T)
    assert a.x_bits.shape == (T, H) and a.x_bits.dtype == np.uint16
    assert a.topk_idx.shape == (T, k) and a.topk_idx.dtype == np.int64
    assert a.topk_weights.shape == (T, k) and a.topk_weights.dtype == np.float32
    assert (a.x_bits == b.x_bits).all() and (a.topk_idx == b.topk_idx).all()
    c = workloads.make(name, T=T, seed=1)
    assert not (a.topk_idx == c.topk_idx).all()
    assert ((a.topk_idx >= 0) & (a.topk_idx < E)).all()
    assert all(len(set(r)) == k for r in a.topk_idx.tolist())       # distinct experts
    assert (a.topk_weights > 0).all()
    assert np.allclose(a.topk_weights.sum(1), 1.0, atol=1e-6)
    x = workloads.bf16_bits_to_float32(a.x_bits)
    tol = 5 / np.sqrt(x.size)
    assert abs(x.mean()) < tol and abs(x.std() - 1) < tol
    assert a.R == (E * cap if cap else T * k)


def test_shared_expert_recipe():
    wl = workloads.make("large", T=2048)
    assert (wl.topk_idx[:, 0] == 0).all() and (wl.topk_idx[:, 1:] >= 1).all()


def test_skewed_recipe():
    wl = workloads.make("skewed", T=4096)
    cnt = np.bincount(wl.topk_idx.ravel(), minlength=256)
    assert cnt.argmax() == 0 and cnt[0] > 0.8 * 4096
    groups = wl.topk_idx // 32
    assert all(len(set(r)) <= 4 for r in groups.tolist())             # top-4 of 8 groups
    assert cnt.reshape(8, 32).sum(1)[0] > 0.5 * cnt.sum()


def test_uniform_recipe_is_balanced():
    wl = workloads.make("dsv3", T=8192, H=128)
    cnt = np.bincount(wl.topk_idx.ravel(), minlength=256)
    assert cnt.sum() == 65536 and cnt.min() > 180 and cnt.max() < 340

"""Seeded input generator: determinism and the shape/distribution recipe."""
import numpy as np
import pytest

from synth import CONFIGS, Config, generate, expert_rows, bf16_to_f32


def test_deterministic_and_seed_sensitive():
    cfg = CONFIGS["tiny"]
    a, b, c = generate(cfg, 0), generate(cfg, 0), generate(cfg, 1)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])
    assert not np.array_equal(a["topk_idx"], c["topk_idx"])


@pytest.mark.parametrize("name", ["tiny", "decode", "share"])
def test_shapes_and_ranges(name):
    cfg = CONFIGS[name]
    d = generate(cfg, 0)
    T, H, K = cfg.tokens, cfg.hidden, cfg.top_k
    assert d["x"].shape == (T, H) and d["x"].dtype == np.uint16
    assert d["topk_idx"].shape == (T, K) and d["topk_idx"].dtype == np.int32
    assert d["topk_weights"].shape == (T, K) and d["topk_weights"].dtype == np.float32
    idx = d["topk_idx"]
    assert idx.min() >= -1 and idx.max() < cfg.num_experts
    # routing draws K distinct experts per token (masking only adds -1)
    for row in idx:
        v = row[row >= 0]
        assert len(set(v.tolist())) == len(v)
    # router weights are a softmax over the k slots
    np.testing.assert_allclose(d["topk_weights"].sum(1), 1.0, rtol=1e-6)
    xf = bf16_to_f32(d["x"])
    assert abs(float(xf.mean())) < 0.05 and abs(float(xf.std()) - 1.0) < 0.05


def test_share_config_masks_non_local_experts():
    cfg = CONFIGS["share"]
    d = generate(cfg, 0)
    idx = d["topk_idx"]
    valid = idx >= 0
    # 16 of 128 experts are local: about 1/8 of slots survive
    assert abs(valid.mean() - 16 / 128) < 0.01
    assert idx.max() == 15


def test_mask_fraction():
    cfg = CONFIGS["stream"].replace(tokens=4096, hidden=128)
    d = generate(cfg, 0)
    assert abs((d["topk_idx"] == -1).mean() - 0.05) < 0.01


def test_zipf_routing_is_skewed():
    cfg = CONFIGS["prefill"].replace(tokens=4096, hidden=8)
    d = generate(cfg, 0)
    counts = np.bincount(d["topk_idx"].ravel(), minlength=256)
    assert counts.sum() == 4096 * 8
    top = np.sort(counts)[::-1]
    # the most popular experts are hit by nearly every token, the tail rarely
    assert top[0] > 0.8 * 4096 and top[-1] < 0.02 * 4096


def test_expert_rows_deterministic():
    a = expert_rows(5, 3, 16, seed=0)
    b = expert_rows(5, 3, 16, seed=0)
    assert a.shape == (5, 3, 16) and np.array_equal(a, b)


def test_empty_config():
    cfg = Config("empty", 0, 128, 2, 4, 4, 8)
    d = generate(cfg, 0)
    assert d["x"].shape == (0, 128) and d["topk_idx"].shape == (0, 2)

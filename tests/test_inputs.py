"""The seeded generators: reproducible, right shapes/dtypes, distributions as stated."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from memory_bound_rmsnorm_amd import inputs
from tests import exact


def test_workload_table_matches_stated_configs():
    w = inputs.WORKLOADS
    assert (w["fp32_64x2048"].rows, w["fp32_64x2048"].hidden, w["fp32_64x2048"].dtype) == (64, 2048, "f32")
    assert (w["bf16_prefill_4096x2048"].rows, w["bf16_prefill_4096x2048"].hidden) == (4096, 2048)
    d = w["bf16_decode_256x4096"]
    assert (d.rows, d.hidden, d.eps, d.x, d.weight) == (256, 4096, 1e-6, inputs.Dist("normal", 0, 2),
                                                         inputs.Dist("uniform", 0.5, 1.5))
    h = w[inputs.HEADLINE]
    assert (h.rows, h.hidden, h.dtype, len(h.outlier_columns), h.outlier_scale) == (16384, 8192, "bf16", 8, 100.0)
    assert sorted(c % 8 for c in h.outlier_columns) == list(range(8))
    f = w["bf16_residual_12289x5120"]
    assert f.fused and (f.rows, f.hidden) == (12289, 5120)


def test_algorithmic_bytes():
    w = inputs.WORKLOADS
    assert w["fp32_64x2048"].algorithmic_bytes == 1_056_768
    assert w["bf16_prefill_4096x2048"].algorithmic_bytes == 33_558_528
    assert w["bf16_decode_256x4096"].algorithmic_bytes == 4_202_496
    assert w[inputs.HEADLINE].algorithmic_bytes == 536_887_296
    assert w["bf16_residual_12289x5120"].algorithmic_bytes == 503_367_680
    assert w["bf16_shard_2048x8192"].algorithmic_bytes == (2 * 2048 * 8192 + 8192) * 2


def test_quant_workload_bytes():
    q = inputs.QUANT_WORKLOADS
    assert q["bf16_int8_16384x8192"].algorithmic_bytes == (16384 * 8192 + 8192) * 2 + 16384 * 8192 + 4 * 16384
    r, h = 12289, 5120
    assert q["bf16_fp8_residual_12289x5120"].algorithmic_bytes == (2 * r * h + h) * 2 + r * h * 2 + r * h + 4 * r
    assert all(w.quant in ("int8", "fp8") for w in q.values())


def test_reproducible_and_seed_dependent():
    w = inputs.WORKLOADS["bf16_prefill_4096x2048"]
    a = inputs.make(w, seed=0, rows=64)
    b = inputs.make(w, seed=0, rows=64)
    c = inputs.make(w, seed=1, rows=64)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["weight"], b["weight"])
    assert not torch.equal(a["x"], c["x"])


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_shapes_dtypes_and_moments(name):
    w = inputs.WORKLOADS[name]
    rows = min(w.rows, 256)
    t = inputs.make(w, seed=0, rows=rows)
    want = torch.float32 if w.dtype == "f32" else torch.bfloat16
    assert t["x"].shape == (rows, w.hidden) and t["x"].dtype == want
    assert t["weight"].shape == (w.hidden,) and t["weight"].dtype == want
    assert ("residual" in t) == w.fused
    x = t["x"].float().numpy().copy()
    if w.outlier_columns:
        cols = list(w.outlier_columns)
        assert abs(np.std(x[:, cols]) / 100.0 - 1.0) < 0.05
        x = np.delete(x, cols, axis=1)
    assert abs(x.mean() - w.x.a) < 0.02 * max(1.0, w.x.b)
    if w.x.kind == "normal":
        assert abs(x.std() / w.x.b - 1.0) < 0.02
    wt = t["weight"].float().numpy()
    if w.weight.kind == "normal":
        assert abs(wt.mean() - w.weight.a) < 0.01 and abs(wt.std() - w.weight.b) < 0.01
    else:
        assert wt.min() >= w.weight.a and wt.max() <= w.weight.b


def test_bf16_storage_is_nearest_even_of_the_fp32_draws():
    w = inputs.WORKLOADS["bf16_prefill_4096x2048"]
    t = inputs.make(w, seed=0, rows=2)
    rng = np.random.default_rng(0)
    draws = rng.standard_normal((2, w.hidden), dtype=np.float32)
    got = inputs.bits(t["x"]).reshape(-1)[:300]
    for g, d in zip(got, draws.reshape(-1)[:300]):
        assert int(g) == exact.round_bf16_exact(Fraction(float(d)))

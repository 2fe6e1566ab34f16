"""The seeded input generator: determinism, shapes, storage exactness and the
segment-length recipes of the five workloads."""
import numpy as np
import pytest

import gdr_inputs as gi


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, 3.0e-39],
                 dtype=np.float32)
    r = gi.round_to_bf16(x)
    # ties go to the even mantissa; values already in bf16 stay put
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == 1.0
    assert r[4] == -2.5 and r[5] == 0.0
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_matches_torch_bf16_cast():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ours = gi.round_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("name", gi.WORKLOAD_ORDER[:3])
def test_deterministic_and_exact(name):
    w = gi.WORKLOADS[name]
    a = gi.generate(w)
    b = gi.generate(w)
    for key in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(a[key], b[key])
        if w.dtype == "bf16":
            assert np.all((a[key].view(np.uint32) & 0xFFFF) == 0), key
    qn = np.linalg.norm(a["q"].astype(np.float64), axis=-1)
    assert np.allclose(qn, 1.0, atol=1e-2 if w.dtype == "bf16" else 1e-5)
    assert np.all(a["g"] <= 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_varlen_ghost_layout():
    d = gi.generate(gi.WORKLOADS["varlen8_ghost8_H32_d128"])
    cu = d["cu_seqlens"]
    assert cu.dtype == np.int32 and cu.shape == (17,)
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0)
    assert np.all(cu[8:] == cu[8]) and np.all(np.diff(cu[:9]) >= 1)
    assert np.all(np.diff(cu[:9]) <= 512)
    assert d["q"].shape[1] == cu[-1]
    assert d["h0"].shape == (16, 32, 128, 128)


def test_packed64k_lengths_recipe():
    w = gi.WORKLOADS["packed64k_gqa_Hk16_Hv32_d128"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = gi.draw_lengths(rng, w)
    assert sum(lens) == 65536
    assert all(256 <= L <= 8192 for L in lens[:-1]) and 1 <= lens[-1] <= 8192


def test_long_config_tail():
    w = gi.WORKLOADS["long_T20468_H16_d128"]
    assert w.seq_len == 319 * 64 + 52

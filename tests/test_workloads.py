"""The seeded input generator: closed forms of the position feature, bf16
rounding against torch's own conversion, determinism and per-head streams."""
import numpy as np
import torch

import workloads


def test_position_feature_norm_and_split():
    for d in (64, 128):
        phi = workloads.position_feature(3, 4, 5, d)
        assert phi.shape == (60, d)
        np.testing.assert_allclose((phi ** 2).sum(1), d / 2, rtol=1e-12)
    # token order (t, y, x), x fastest: the x block varies with n, the t block is constant in a frame
    phi = workloads.position_feature(2, 3, 4, 64)
    dt = 64 - 4 * (64 // 6)
    assert np.all(phi[:12, :dt] == phi[0, :dt])
    assert not np.allclose(phi[0, -20:], phi[1, -20:])
    # first pair of each axis block is (sin 0, cos 0) = (0, 1) at the origin
    assert phi[0, 0] == 0.0 and phi[0, 1] == 1.0


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # exact ties round to even
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic_and_per_head_streams():
    w = workloads.small_case(H=3, N=256, d=64, block_q=64, block_k=64, seed=11)
    q1, k1, v1 = workloads.make_qkv(w)
    q2, k2, v2 = workloads.make_qkv(w)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(v1, v2)
    only = workloads.make_qkv(w, heads=[2], which=(1,))[0]
    np.testing.assert_array_equal(only[0, 0], k1[0, 2])
    # values are bf16-representable
    np.testing.assert_array_equal(workloads.bf16_round(q1), q1)


def test_workload_table_shapes():
    w = workloads.get("wan14b_n32760")
    assert (w.N, w.nqb, w.nkb, w.rows) == (32760, 512, 512, 20480)
    w = workloads.get("skew_n75600_bq128")
    assert (w.N, w.nqb, w.nkb) == (75600, 591, 1182)
    a = workloads.head_alphas(w)
    assert a.min() >= 0.1 and a.max() <= 6.0

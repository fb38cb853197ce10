"""Seeded input generator: determinism, distributions, formats."""
import numpy as np
import pytest

import moe_inputs as mi


def test_splitmix_reference_values():
    # SplitMix64 seeded with 0: first outputs of the published generator
    h = mi.splitmix_stream(0, 0, 3)
    assert [int(v) for v in h] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert mi.mix64(mi.GAMMA) == 0xE220A8397B1DCDAF


def test_stream_offsets_consistent():
    a = mi.splitmix_stream(12345, 0, 100)
    b = mi.splitmix_stream(12345, 40, 60)
    assert np.array_equal(a[40:], b)
    assert np.array_equal(mi.normal(7, 64, 1.0)[32:], mi.normal(7, 32, 1.0, start=32))


def test_normal_table_shape():
    t = mi.NORMAL_TABLE
    assert t.dtype == np.float32 and t.shape == (65536,)
    assert np.all(np.diff(t) > 0)
    assert np.array_equal(t, -t[::-1])
    assert abs(float(t.astype(np.float64).std()) - 1.0) < 2e-3


def test_normal_moments():
    v = mi.normal(mi.derive_key(1, 2, 3), 1 << 20, 0.02).astype(np.float64)
    assert abs(v.mean()) < 1e-4
    assert abs(v.std() - 0.02) < 1e-4


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = mi.normal(99, 4096, 1.0)
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 0.0]   # ties to even
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mi.bf16_bits_from_f32(x), want)


def test_expert_generation_deterministic_and_distinct():
    wl = mi.WORKLOADS["tiny"]
    a = mi.expert_tensor_host(wl, 0, mi.GATE, 3)
    b = mi.expert_tensor_host(wl, 0, mi.GATE, 3)
    c = mi.expert_tensor_host(wl, 0, mi.GATE, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (128, 8, 2) and a[1].shape == (128, 8)


def test_three_bit_uses_same_draws():
    wl2 = mi.WORKLOADS["decode_48layer"]
    wl3 = mi.WORKLOADS["verify4_3bit"]
    assert mi.expert_key(wl2, 5, mi.UP, 17) == mi.expert_key(wl3, 5, mi.UP, 17)


def test_expert_bytes():
    wl = mi.WORKLOADS["decode_1layer"]
    assert wl.expert_bytes() == 1_474_560
    assert mi.WORKLOADS["verify4_3bit"].expert_bytes() == 2_064_384
    assert mi.WORKLOADS["tiny"].expert_bytes() == 30_720


def test_zipf_bias_skews_routing():
    """The router bias gives a Zipf prior: on sampled prefill tokens the
    hottest expert takes far more than the mean load."""
    import oracle.moe_oracle as O
    wl = mi.WORKLOADS["prefill_8192"]
    w, b = mi.router_host(wl, 0)
    x = mi.activations_host(wl)[:512]
    ids, _, _ = O.route(x, w, b, wl.top_k)
    load = np.bincount(ids.reshape(-1), minlength=wl.n_experts)
    assert load.max() / load.mean() > 10
    ranks = np.sort(-1.1 * np.log(np.arange(1, 513)))
    assert np.allclose(np.sort(b), ranks.astype(np.float32))

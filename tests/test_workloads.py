"""Seeded input generators: shapes, value sets and determinism (CPU)."""
import torch

from workloads import WORKLOADS, make_inputs, sample_positions


def test_small_prefill_inputs():
    w = WORKLOADS["prefill_2k_tiny"]
    a = make_inputs(w)
    b = make_inputs(w)
    assert a["kidx"].shape == (1, 2048, 64) and a["kidx"].dtype == torch.bfloat16
    assert a["q"].shape == (1, 2048, 1, 128)
    for key in a:
        assert torch.equal(a[key], b[key])
    ki = a["kidx"].float()
    assert ki.min() == -8 and ki.max() == 8 and torch.equal(ki, ki.round())
    assert a["q_pos"].tolist() == [list(range(2048))]


def test_mla_view_aliases_latent():
    w = WORKLOADS["prefill_64k_mla"].with_(L=512, nq=512, B=128, m=4, k=64)
    a = make_inputs(w)
    assert a["v"].data_ptr() == a["k"].data_ptr()
    assert a["v"].shape[-1] == 512 and a["k"].shape[-1] == 576
    assert a["v"].stride() == a["k"].stride()


def test_hils_int_twin_values():
    w = WORKLOADS["hils_decode_1m"].with_(L=4096, int_mode=True)
    a = make_inputs(w)
    wp = a["w_proj"].float()
    assert set(wp.unique().tolist()) <= {-1.0, 0.0, 1.0}
    assert a["q_pos"].tolist() == [4095]


def test_sample_positions_has_edges():
    w = WORKLOADS["prefill_16k_mqa"]
    p = sample_positions(w, 40)
    for e in [0, 1, 127, 128, 2047, 2048, 4095, 4096, 16383]:
        assert e in p

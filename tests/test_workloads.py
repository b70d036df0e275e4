"""Input generators: determinism, shapes and the bf16 rounding of the draws (CPU only)."""

import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38], np.float32)])
    # bit patterns just around the bf16 rounding midpoints
    mid = (np.arange(0, 1 << 16, 37, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, mid.view(np.float32)[np.isfinite(mid.view(np.float32))]])
    ours = workloads.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_decode_case_layout():
    c = workloads.decode_case(5, seq_lens=[100, 1, 64, 129], H=16, next_n=2, spare_pages=3)
    P = c["page_size"]
    assert c["k"].shape == (294, 128) and c["k"].dtype == np.uint16
    assert c["q"].shape == (8, 16, 128)
    assert c["w"].shape == (8, 16) and c["w"].dtype == np.float32
    assert c["num_pages"] == 2 + 1 + 1 + 3 + 3
    slots = c["slot_mapping"]
    assert len(np.unique(slots)) == len(slots)
    assert slots.min() >= 0 and slots.max() < c["num_pages"] * P
    # block table entries of used pages are distinct physical pages
    used = np.concatenate([c["block_table"][b, :(L + P - 1) // P] for b, L in enumerate(c["context_lens"])])
    assert len(np.unique(used)) == len(used)


def test_generators_are_deterministic():
    a = workloads.tiny()
    b = workloads.tiny()
    for key in ("k", "q", "w", "slot_mapping", "block_table"):
        assert np.array_equal(a[key], b[key])
    assert a["k"].dtype == np.float32 and a["next_n"] == 4 and a["topk"] == 64


def test_lognormal_block_scales_span():
    rng = np.random.default_rng(1)
    x = workloads.draw_values(rng, (4000, 128), "lognormal")
    amax = np.abs(x.reshape(4000, 4, 32)).max(-1)
    lg = np.log2(amax)
    assert lg.min() < -6 and lg.max() > 8

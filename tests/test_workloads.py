"""Checks of the seeded input generators (shapes, layouts, statistics)."""
import numpy as np
import torch

import workloads as wl
from workloads.generate import _Normal


def test_field_has_unit_variance_and_neighbour_correlation():
    f = wl.correlated_field(_Normal(123), 3000, 16).astype(np.float64)
    assert abs(f.var() - 1.0) < 0.02
    right = np.mean(f[:, :, 1:] * f[:, :, :-1])
    down = np.mean(f[:, 1:, :] * f[:, :-1, :])
    diag = np.mean(f[:, 1:, 1:] * f[:, :-1, :-1])
    assert abs(right - 0.8) < 0.02 and abs(down - 0.8) < 0.02
    assert abs(diag - 0.64) < 0.02


def test_inputs_are_reproducible_and_prefix_stable():
    a = wl.decode_inputs(wl.small_decode("gqa_b64", n_seq=2))
    b = wl.decode_inputs(wl.small_decode("gqa_b64", n_seq=3))
    assert torch.equal(a.k_logical, b.k_logical[:2])
    assert torch.equal(a.pos, b.pos[:2])
    c = wl.decode_inputs(wl.small_decode("gqa_b64", n_seq=2))
    assert torch.equal(a.v_cache, c.v_cache) and torch.equal(a.q, c.q)


def test_paged_layout_holds_the_logical_cache():
    d = wl.decode_inputs(wl.small_decode("paged_b128", n_seq=3))
    ps = d.cfg.page_size
    bt = d.block_table
    assert sorted(bt.reshape(-1).tolist()) == list(range(bt.numel()))
    for s in range(3):
        for j in (0, 17, int(d.pos[s]), d.lmax - 1):
            page = int(bt[s, j // ps])
            assert torch.equal(d.k_cache[page, :, j % ps], d.k_logical[s, :, j])
            assert torch.equal(d.v_cache[page, :, j % ps], d.v_logical[s, :, j])


def test_positions_follow_the_workload_rules():
    c = wl.CONFIGS["llamagen_b16"]
    d = wl.decode_inputs(c)
    P = c.prompt[0]
    assert d.pos.min() >= P + c.W and d.pos.max() < P + c.n_vis
    s = wl.decode_inputs(wl.CONFIGS["sweep_f32"])
    assert s.pos.tolist() == list(range(16, 272))
    p = wl.decode_inputs(wl.small_decode("paged_b128", n_seq=20))
    assert p.prompt_len.min() >= 64 and p.prompt_len.max() <= 300
    assert bool(((p.pos - p.prompt_len) < 48 * 48).all())

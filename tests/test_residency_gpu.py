"""Decode through the ring block table (rows older than the live window
recycled) returns exactly what it returns on the full cache, and matches
the oracle run on the logical (full) cache."""
import pytest
import torch

import ar_image_generation_amd as da
import oracle as O
import workloads as wl
from gpu_helpers import assert_close, dev, run_oracle

pytestmark = pytest.mark.gpu


def ring_cache(inp, m, ps):
    """Fills a ring-paged cache the way generation would: logical pages in
    order, each later page overwriting its slot."""
    cfg = inp.cfg
    k_log, v_log = inp.k_logical, inp.v_logical             # [n_seq, hkv, L, hd]
    n_seq, hkv, L, hd = k_log.shape
    bt, total = da.ring_block_table(m, inp.prompt_len_per_seq, L, ps)
    kc = torch.zeros((total, hkv, ps, hd), dtype=k_log.dtype)
    vc = torch.zeros_like(kc)
    for s in range(n_seq):
        top = int(inp.pos[inp.seq == s].max()) if (inp.seq == s).any() else -1
        for lp in range(top // ps + 1):
            pg = int(bt[s, lp])
            lo, hi = lp * ps, min(L, (lp + 1) * ps)
            kc[pg, :, : hi - lo] = k_log[s, :, lo:hi]
            vc[pg, :, : hi - lo] = v_log[s, :, lo:hi]
    return kc, vc, bt, total


@pytest.mark.parametrize("name,n_seq", [("paged_b128", 6), ("llamagen_b16", 3)])
def test_ring_cache_decode_equals_full_cache(name, n_seq):
    cfg = wl.small_decode(name, n_seq=n_seq)
    inp = wl.decode_inputs(cfg)
    # one query per request here: its prompt length is the request's
    inp.prompt_len_per_seq = [int(inp.prompt_len[inp.seq == s][0]) for s in range(cfg.n_seq)]
    ps = 16
    q = inp.q.to(dev())
    seq, pos, prompt = inp.seq.to(dev()), inp.pos.to(dev()), inp.prompt_len.to(dev())
    for mode in sorted(set(cfg.modes) | {O.DENSE}):
        m = da.mask(mode, cfg.W, cfg.B, cfg.G)
        cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
        kc, vc, bt, total = ring_cache(inp, m, ps)
        full_pages = cfg.n_seq * -(-inp.k_logical.shape[2] // ps)
        assert total <= full_pages
        kc, vc, bt = kc.to(dev()), vc.to(dev()), bt.to(dev())
        ref, ref_lse, _, _ = da.sparse_decode_attn_masked(
            m, q, inp.k_logical.to(dev()), inp.v_logical.to(dev()), seq, pos, prompt,
            cap=cap, split=4096, want_lse=True)
        got, got_lse, _, _ = da.sparse_decode_attn_masked(
            m, q, kc, vc, seq, pos, prompt, cap=cap, split=4096, block_table=bt, want_lse=True)
        count, idx, _, _ = da.keepset_build(m, pos, prompt, cap)
        got2, _ = da.sparse_decode_attn(q, kc, vc, seq, count, idx, split=4096, block_table=bt)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu()), mode
        assert torch.equal(got_lse.cpu(), ref_lse.cpu()), mode
        assert torch.equal(got2.cpu(), ref.cpu()), mode
        # and against the oracle on the logical cache: the ring holds every
        # row the keep-sets read
        ref_o, ref_l = run_oracle(inp, mode)
        assert_close(got.cpu(), got_lse.cpu(), ref_o, ref_l, cfg.dtype)

"""The allocation-free decode entry point (the library's per-GPU scratch
array instead of a caller workspace) against the workspace entry point:
identical outputs, on calls in a row whose sizes shrink, in the
multi-chunk case where the scratch actually holds partials."""
import pytest
import torch

import ar_image_generation_amd as da
import oracle as O
import workloads as wl
from ar_image_generation_amd._native import DiagAttnError

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(n_seq, paged):
    cfg = wl.small_decode("paged_b128" if paged else "gqa_b64", n_seq=n_seq)
    inp = wl.decode_inputs(cfg)
    if paged:
        k, v, bt = inp.k_cache.to(DEV), inp.v_cache.to(DEV), inp.block_table.to(DEV)
    else:
        k, v, bt = inp.k_logical.to(DEV), inp.v_logical.to(DEV), None
    return cfg, inp, k, v, bt


def _both(cfg, inp, k, v, bt, mode, split):
    m = da.mask(mode, cfg.W, cfg.B, cfg.G)
    cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
    q, seq, pos, pr = (inp.q.to(DEV), inp.seq.to(DEV), inp.pos.to(DEV), inp.prompt_len.to(DEV))
    ref, ref_lse, ref_c, ref_i = da.sparse_decode_attn_masked(
        m, q, k, v, seq, pos, pr, cap=cap, split=split, block_table=bt, want_lse=True,
        want_lists=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((inp.n_q, cfg.hq), float("nan"), dtype=torch.float32, device=DEV)
    count = torch.full_like(ref_c, -1)
    idx = torch.full_like(ref_i, -1)
    da.sparse_decode_attn_masked_noalloc(m, q, k, v, seq, pos, pr, cap=cap, split=split, out=out,
                                         block_table=bt, lse=lse, count=count, idx=idx)
    torch.cuda.synchronize()
    return (ref, ref_lse, ref_c, ref_i), (out, lse, count, idx), cap


@pytest.mark.parametrize("paged", [False, True])
def test_noalloc_equals_workspace_entry_on_shrinking_calls(paged):
    for n_seq, mode, split in [(6, O.DENSE, 256), (3, O.DENSE, 256), (5, O.ROWDIAG, 64),
                               (2, O.ROWDIAG, 4096)]:
        cfg, inp, k, v, bt = _inputs(n_seq, paged)
        (ro, rl, rc, ri), (o, l, c, i), cap = _both(cfg, inp, k, v, bt, mode, split)
        assert torch.equal(o, ro), (n_seq, mode, split)
        assert torch.equal(l, rl)
        assert torch.equal(c, rc)
        for qq in range(inp.n_q):
            n = min(int(rc[qq]), cap)
            assert torch.equal(i[qq, :n], ri[qq, :n])
        if mode == O.DENSE and split < cap:
            assert da.decode_workspace_bytes(inp.n_q, cfg.hq, cfg.hd, cap, split) > 0


def test_noalloc_matches_oracle():
    cfg, inp, k, v, bt = _inputs(2, False)
    _, (o, l, _, _), _ = _both(cfg, inp, k, v, bt, O.DENSE, 200)
    ref_o, ref_l = O.decode_attention(inp.q.double().numpy(), inp.k_logical.double().numpy(),
                                      inp.v_logical.double().numpy(), inp.pos.numpy(),
                                      inp.prompt_len.numpy(), inp.seq.numpy(), W=cfg.W, B=cfg.B,
                                      G=cfg.G, mode=O.DENSE)
    assert float((o.double().cpu() - torch.from_numpy(ref_o)).abs().max()) <= 2e-2
    assert float((l.double().cpu() - torch.from_numpy(ref_l)).abs().max()) <= 1e-4 * 10


def test_noalloc_refuses_sizes_beyond_its_scratch():
    cfg, inp, k, v, bt = _inputs(2, False)
    m = da.mask(O.DENSE, 0, 0, cfg.G)
    q, seq, pos, pr = (inp.q.to(DEV), inp.seq.to(DEV), inp.pos.to(DEV), inp.prompt_len.to(DEV))
    # a cap whose chunk partials exceed the scratch: n_q * hq * ceil(cap/split) * (hd + 2) * 4
    cap, split = 4096, 1
    assert da.decode_workspace_bytes(inp.n_q, cfg.hq, cfg.hd, cap, split) > da.decode_scratch_bytes()
    out = torch.empty_like(q)
    with pytest.raises(DiagAttnError) as e:
        da.sparse_decode_attn_masked_noalloc(m, q, k, v, seq, pos, pr, cap=cap, split=split, out=out)
    assert e.value.status == -3

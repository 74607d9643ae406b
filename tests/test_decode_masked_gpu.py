"""GPU decode with the keep-set computed in the kernel (mask form).

It must equal, bit for bit, the list path (keepset_build lists through
sparse_decode_attn): the same kept rows in the same order through the same
tile loop.  The lists it writes must equal keepset_build's exactly.  The
oracle checks it directly as well, to the decode tolerances."""
import numpy as np
import pytest
import torch

import ar_image_generation_amd as da
import oracle as O
import workloads as wl
from gpu_helpers import assert_close, dev, run_oracle

pytestmark = pytest.mark.gpu


def caches(inp, paged=None):
    paged = inp.cfg.page_size > 0 if paged is None else paged
    if paged:
        return inp.k_cache.to(dev()), inp.v_cache.to(dev()), inp.block_table.to(dev())
    return inp.k_logical.to(dev()), inp.v_logical.to(dev()), None


def both_paths(inp, mode, split, cap=None, W=None, B=None, G=None):
    """(list path, mask path) results on the same inputs and cap."""
    cfg = inp.cfg
    m = da.mask(mode, cfg.W if W is None else W, cfg.B if B is None else B, cfg.G if G is None else G)
    pos, prompt = inp.pos.to(dev()), inp.prompt_len.to(dev())
    if cap is None:
        cap = da.keep_cap(m, max(0, int(inp.pos.max())), max(0, int(inp.prompt_len.max())))
    q = inp.q.to(dev())
    k, v, bt = caches(inp)
    seq = inp.seq.to(dev())
    count, idx, _, _ = da.keepset_build(m, pos, prompt, cap)
    o1 = torch.full_like(q, 7.0)
    o1, l1 = da.sparse_decode_attn(q, k, v, seq, count, idx, split=split, block_table=bt, out=o1,
                                   want_lse=True)
    o2 = torch.full_like(q, 7.0)
    o2, l2, c2, i2 = da.sparse_decode_attn_masked(m, q, k, v, seq, pos, prompt, cap=cap, split=split,
                                                  block_table=bt, out=o2, want_lse=True,
                                                  want_lists=True)
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu(), count.cpu(), idx.cpu()), (o2.cpu(), l2.cpu(), c2.cpu(), i2.cpu()), cap


def assert_same(a, b, cap):
    o1, l1, c1, i1 = a
    o2, l2, c2, i2 = b
    assert torch.equal(c1, c2)
    for qi in range(c1.numel()):
        n = min(int(c1[qi]), cap)
        assert torch.equal(i1[qi, :n], i2[qi, :n]), qi
    assert torch.equal(o1, o2)
    valid = c1 > 0
    assert torch.equal(l1[valid], l2[valid])


@pytest.mark.parametrize("split", [8, 37, 256])
def test_fp32_sweep_equals_list_path(split):
    inp = wl.decode_inputs(wl.CONFIGS["sweep_f32"])
    a, b, cap = both_paths(inp, O.ROWDIAG, split)
    assert_same(a, b, cap)


@pytest.mark.parametrize("name,n_seq", [("llamagen_b16", 4), ("gqa_b64", 3), ("paged_b128", 6)])
@pytest.mark.parametrize("split", [32, 136, 4096])
def test_reduced_workloads_equal_list_path(name, n_seq, split):
    cfg = wl.small_decode(name, n_seq=n_seq)
    inp = wl.decode_inputs(cfg)
    for mode in sorted(set(cfg.modes) | {O.DENSE}):
        a, b, cap = both_paths(inp, mode, split)
        assert_same(a, b, cap)


@pytest.mark.parametrize("name,n_seq", [("sweep_f32", None), ("llamagen_b16", 3), ("paged_b128", 4)])
def test_mask_path_vs_oracle(name, n_seq):
    cfg = wl.CONFIGS[name] if n_seq is None else wl.small_decode(name, n_seq=n_seq)
    inp = wl.decode_inputs(cfg)
    for mode in sorted(set(cfg.modes) | {O.DENSE}):
        _, (o, l, _, _), _ = both_paths(inp, mode, 64)
        ref_o, ref_l = run_oracle(inp, mode)
        assert_close(o, l, ref_o, ref_l, cfg.dtype)


def test_edge_positions():
    """Queries inside the prompt, at position 0, with no prompt, with a
    window reaching past the prompt start, and invalid ones (count 0, output
    untouched)."""
    cfg = wl.small_decode("llamagen_b16", n_seq=1)
    inp = wl.decode_inputs(cfg)
    n_q = 8
    g = torch.Generator().manual_seed(3)
    inp.q = torch.randn((n_q,) + tuple(inp.q.shape[1:]), generator=g).to(inp.q.dtype)
    inp.pos = torch.tensor([0, 5, 119, 120, 130, 300, -1, 200], dtype=torch.int32)
    inp.prompt_len = torch.tensor([120, 120, 120, 0, 120, 7, 120, -2], dtype=torch.int32)
    inp.seq = torch.zeros(n_q, dtype=torch.int32)
    for mode in (O.DENSE, O.BAND, O.ROWDIAG):
        for split in (16, 4096):
            a, b, cap = both_paths(inp, mode, split)
            assert_same(a, b, cap)
            o, _, c, _ = b
            assert int(c[6]) == 0 and int(c[7]) == 0
            assert torch.all(o[6:].float() == 7.0)          # no output for invalid queries
            ok = [0, 1, 2, 3, 4, 5]
            ref_o, ref_l = O.decode_attention(
                inp.q.double().numpy(), inp.k_logical.double().numpy(), inp.v_logical.double().numpy(),
                inp.pos.numpy(), inp.prompt_len.numpy(), inp.seq.numpy(),
                W=cfg.W, B=cfg.B, G=cfg.G, mode=mode, queries=ok)
            assert_close(o, b[1], ref_o, ref_l, cfg.dtype, queries=ok)


@pytest.mark.parametrize("W,B,G", [(0, 0, 32), (32, 0, 32), (96, 20, 32), (5, 2, 1)])
def test_mask_parameters(W, B, G):
    """Zero window, zero band, overlapping bands (2B+1 >= G), G = 1."""
    cfg = wl.small_decode("llamagen_b16", n_seq=2)
    inp = wl.decode_inputs(cfg)
    for mode in (O.BAND, O.ROWDIAG):
        a, b, cap = both_paths(inp, mode, 64, W=W, B=B, G=G)
        assert_same(a, b, cap)


@pytest.mark.parametrize("W,B,G", [(2**31 - 1, 3, 64), (96, 2**31 - 1, 32), (2**30, 2**30, 2**31 - 1),
                                   (40, 7, 15), (2**31 - 1, 0, 2**31 - 1)])
def test_extreme_mask_parameters(W, B, G):
    """Window, band and grid width at the int32 limits, and 2B+1 = G: the
    in-kernel keep-set (closed form) equals the list builder's (scan)."""
    cfg = wl.small_decode("llamagen_b16", n_seq=2)
    inp = wl.decode_inputs(cfg)
    for mode in (O.BAND, O.ROWDIAG):
        a, b, cap = both_paths(inp, mode, 4096, W=W, B=B, G=G)
        assert_same(a, b, cap)


def test_truncated_capacity():
    """cap below the keep-set size: both paths attend to the first cap
    entries and report the true count."""
    cfg = wl.small_decode("gqa_b64", n_seq=2)
    inp = wl.decode_inputs(cfg)
    a, b, cap = both_paths(inp, O.ROWDIAG, 64, cap=100)
    assert int(b[2].min()) > 100
    assert_same(a, b, cap)


@pytest.mark.parametrize("name", ["llamagen_b16", "gqa_b64", "paged_b128"])
def test_full_size_equals_list_path(name):
    """The decode workloads at full size in their launch setting (one chunk
    per query and kv head), every mask mode they run plus the dense one:
    the in-kernel keep-set equals the list path bitwise."""
    cfg = wl.CONFIGS[name]
    inp = wl.decode_inputs(cfg)
    for mode in dict.fromkeys(tuple(cfg.modes) + (O.DENSE,)):
        split = cfg.dense_split if mode == O.DENSE else cfg.split
        a, b, cap = both_paths(inp, mode, split)
        assert_same(a, b, cap)
        assert torch.isfinite(b[0].float()).all()


def test_without_lists_same_output():
    cfg = wl.small_decode("paged_b128", n_seq=4)
    inp = wl.decode_inputs(cfg)
    m = da.mask(O.ROWDIAG, cfg.W, cfg.B, cfg.G)
    cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
    k, v, bt = caches(inp)
    args = (m, inp.q.to(dev()), k, v, inp.seq.to(dev()), inp.pos.to(dev()), inp.prompt_len.to(dev()))
    o1, _, c1, _ = da.sparse_decode_attn_masked(*args, cap=cap, split=64, block_table=bt,
                                                want_lists=True)
    o2, _, c2, _ = da.sparse_decode_attn_masked(*args, cap=cap, split=64, block_table=bt)
    torch.cuda.synchronize()
    assert c2 is None and c1 is not None
    assert torch.equal(o1.cpu(), o2.cpu())


@pytest.mark.parametrize("name,n_seq,split", [("llamagen_b16", 4, 4096), ("llamagen_b16", 4, 32),
                                              ("paged_b128", 5, 4096), ("paged_b128", 5, 48)])
def test_kv_append(name, n_seq, split):
    """KV append: on a cache missing each query's own row, the step with
    k_new/v_new equals the step on the complete cache, and leaves the cache
    complete (one query per request)."""
    cfg = wl.small_decode(name, n_seq=n_seq)
    inp = wl.decode_inputs(cfg)
    k_full, v_full, bt = caches(inp)
    s_idx, p_idx = inp.seq.long(), inp.pos.long()
    k_new = inp.k_logical[s_idx, :, p_idx].contiguous().to(dev())      # [n_q, hkv, hd]
    v_new = inp.v_logical[s_idx, :, p_idx].contiguous().to(dev())
    if bt is None:
        rows = (s_idx.to(dev()), slice(None), p_idx.to(dev()))
    else:
        ps = k_full.shape[2]
        pages = bt[s_idx.to(dev()), (p_idx // ps).to(dev())].long()
        rows = (pages, slice(None), (p_idx % ps).to(dev()))
    q, seq, pos, prompt = (inp.q.to(dev()), inp.seq.to(dev()), inp.pos.to(dev()),
                           inp.prompt_len.to(dev()))
    for mode in sorted(set(cfg.modes) | {O.DENSE}):
        m = da.mask(mode, cfg.W, cfg.B, cfg.G)
        cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
        k_miss, v_miss = k_full.clone(), v_full.clone()
        k_miss[rows] = 0
        v_miss[rows] = 0
        assert not torch.equal(k_miss, k_full)
        ref, ref_lse, _, _ = da.sparse_decode_attn_masked(m, q, k_full, v_full, seq, pos, prompt,
                                                          cap=cap, split=split, block_table=bt,
                                                          want_lse=True)
        got, got_lse, _, _ = da.sparse_decode_attn_masked(m, q, k_miss, v_miss, seq, pos, prompt,
                                                          cap=cap, split=split, block_table=bt,
                                                          want_lse=True, k_new=k_new, v_new=v_new)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu()), mode
        assert torch.equal(got_lse.cpu(), ref_lse.cpu()), mode
        assert torch.equal(k_miss, k_full) and torch.equal(v_miss, v_full), mode
        # and against the oracle on the logical cache (contiguous and paged)
        ref_o, ref_l = run_oracle(inp, mode)
        assert_close(got.cpu(), got_lse.cpu(), ref_o, ref_l, cfg.dtype)


@pytest.mark.parametrize("split", [37, 4096])
@pytest.mark.parametrize("mode", [O.ROWDIAG, O.BAND, O.DENSE])
def test_kv_append_query_inside_its_prompt(mode, split):
    """KV append with some queries inside their prompt (pos < prompt_len):
    the query's own row is then a prompt entry, which a short chunk of a
    contiguous cache loads before the keep-set scan, so what that load
    returns must give way to the appended row.  Equal, bit for bit, to the
    plain step on the complete cache (one query per request)."""
    cfg = wl.small_decode("llamagen_b16", n_seq=6)
    inp = wl.decode_inputs(cfg)
    n_q = inp.n_q
    g = torch.Generator().manual_seed(5)
    pos = torch.randint(0, 90, (n_q,), generator=g, dtype=torch.int32)
    r = torch.arange(n_q, dtype=torch.int32)
    prompt = torch.where(r % 2 == 0, pos + 1 + r % 5, pos // 2).to(torch.int32)
    assert bool((prompt > pos).any()) and bool((prompt <= pos).any())
    k_full, v_full, _ = caches(inp, paged=False)
    s_idx, p_idx = inp.seq.long(), pos.long()
    k_new = inp.k_logical[s_idx, :, p_idx].contiguous().to(dev())
    v_new = inp.v_logical[s_idx, :, p_idx].contiguous().to(dev())
    rows = (s_idx.to(dev()), slice(None), p_idx.to(dev()))
    q, seq = inp.q.to(dev()), inp.seq.to(dev())
    pos_d, prompt_d = pos.to(dev()), prompt.to(dev())
    m = da.mask(mode, cfg.W, cfg.B, cfg.G)
    cap = da.keep_cap(m, int(pos.max()), int(prompt.max()))
    k_miss, v_miss = k_full.clone(), v_full.clone()
    k_miss[rows] = 0
    v_miss[rows] = 0
    ref, ref_lse, _, _ = da.sparse_decode_attn_masked(m, q, k_full, v_full, seq, pos_d, prompt_d,
                                                      cap=cap, split=split, want_lse=True)
    got, got_lse, _, _ = da.sparse_decode_attn_masked(m, q, k_miss, v_miss, seq, pos_d, prompt_d,
                                                      cap=cap, split=split, want_lse=True,
                                                      k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), ref.cpu())
    assert torch.equal(got_lse.cpu(), ref_lse.cpu())
    assert torch.equal(k_miss, k_full) and torch.equal(v_miss, v_full)
    ref_o, ref_l = O.decode_attention(
        inp.q.double().numpy(), inp.k_logical.double().numpy(), inp.v_logical.double().numpy(),
        pos.numpy(), prompt.numpy(), inp.seq.numpy(), W=cfg.W, B=cfg.B, G=cfg.G, mode=mode)
    assert_close(got.cpu(), got_lse.cpu(), ref_o, ref_l, cfg.dtype)


def test_mass_share_from_lse_matches_direct_softmax():
    """exp(lse_sparse - lse_dense) is the share of the dense softmax mass on
    the keep-set; compared with that share summed directly in fp64 from the
    oracle's keep-sets (relative 1e-3: two LSEs within 1e-4 each, plus bf16)."""
    cfg = wl.small_decode("llamagen_b16", n_seq=3)
    inp = wl.decode_inputs(cfg)
    k, v, bt = caches(inp)
    args = (inp.q.to(dev()), k, v, inp.seq.to(dev()), inp.pos.to(dev()), inp.prompt_len.to(dev()))
    dense = da.mask(O.DENSE, 0, 0, 1)
    _, lse_d, _, _ = da.sparse_decode_attn_masked(dense, *args, cap=int(inp.pos.max()) + 1,
                                                  split=4096, block_table=bt, want_lse=True)
    q = inp.q.double().numpy()
    K = inp.k_logical.double().numpy()
    for W, B in [(32, 0), (96, 2), (192, 4)]:
        m = da.mask(O.ROWDIAG, W, B, cfg.G)
        cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
        _, lse_s, _, _ = da.sparse_decode_attn_masked(m, *args, cap=cap, split=4096, block_table=bt,
                                                      want_lse=True)
        torch.cuda.synchronize()
        share = torch.exp(lse_s - lse_d).double().cpu().numpy()
        for qi in range(inp.n_q):
            i, P, s = int(inp.pos[qi]), int(inp.prompt_len[qi]), int(inp.seq[qi])
            kept = O.keepset(i, P=P, W=W, B=B, G=cfg.G, mode=O.ROWDIAG)
            for h in range(cfg.hq):
                g = h // (cfg.hq // cfg.hkv)
                sc = K[s, g, : i + 1] @ q[qi, h] / np.sqrt(cfg.hd)
                w = np.exp(sc - sc.max())
                want = w[kept].sum() / w.sum()
                assert abs(share[qi, h] - want) <= 1e-3 * want, (W, B, qi, h, share[qi, h], want)


@pytest.mark.parametrize("seed", range(10))
def test_random_configurations(seed):
    """Seeded random shapes and masks (dtype, head size, GQA ratio, paged or
    contiguous cache, grid, window, band, prompt range, split): the mask
    path against the oracle, and bitwise against the list path."""
    rng = np.random.default_rng(500 + seed)
    hd = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    pmin = int(rng.integers(0, 60))
    cfg = wl.small_decode(
        "paged_b128", n_seq=int(rng.integers(1, 5)), hq=hq, hkv=hkv, hd=hd,
        dtype=str(rng.choice(["f32", "bf16"])), prompt=(pmin, pmin + int(rng.integers(0, 40))),
        G=int(rng.integers(1, 40)), W=int(rng.integers(0, 200)), B=int(rng.integers(0, 8)),
        modes=(O.BAND, O.ROWDIAG), pos_rule="image", page_size=int(rng.choice([0, 4, 16])),
        kv_gen="normal", seed=700 + seed)
    inp = wl.decode_inputs(cfg)
    split = int(rng.choice([16, 48, 4096]))
    for mode in (O.DENSE, O.BAND, O.ROWDIAG):
        a, b, cap = both_paths(inp, mode, split)
        assert_same(a, b, cap)
        ref_o, ref_l = run_oracle(inp, mode)
        assert_close(b[0], b[1], ref_o, ref_l, cfg.dtype)


def _per_head_reference(inp, wb, mode):
    """The oracle once per query head, with that head's (W, B)."""
    cfg = inp.cfg
    grp = cfg.hq // cfg.hkv
    q = inp.q.double().numpy()
    K, V = inp.k_logical.double().numpy(), inp.v_logical.double().numpy()
    ref_o = np.zeros(q.shape)
    ref_l = np.zeros(q.shape[:2])
    for h, (w, b) in enumerate(wb):
        g = h // grp
        o_h, l_h = O.decode_attention(q[:, h:h + 1], K[:, g:g + 1], V[:, g:g + 1], inp.pos.numpy(),
                                      inp.prompt_len.numpy(), inp.seq.numpy(),
                                      W=int(w), B=int(b), G=cfg.G, mode=mode)
        ref_o[:, h:h + 1], ref_l[:, h:h + 1] = o_h, l_h
    return ref_o, ref_l


@pytest.mark.parametrize("name,split", [("gqa_b64", 32), ("gqa_b64", 4096), ("paged_b128", 4096),
                                        ("llamagen_b16", 4096)])
def test_per_head_masks(name, split):
    """A (W, B) per query head (heads of one kv group differ): every head
    against the oracle run with its own mask.  The group reads its widest
    keep-set once and masks per head, so GQA sharing is kept; MHA reads per
    head.  With the same (W, B) everywhere, bitwise the shared-mask call."""
    cfg = wl.small_decode(name, n_seq=3)
    inp = wl.decode_inputs(cfg)
    k, v, bt = caches(inp)
    rng = np.random.default_rng(7)
    wb = np.stack([rng.integers(0, 300, cfg.hq), rng.integers(0, 7, cfg.hq)], axis=1).astype(np.int32)
    head_wb = torch.from_numpy(wb).to(dev())
    args = (inp.q.to(dev()), k, v, inp.seq.to(dev()), inp.pos.to(dev()), inp.prompt_len.to(dev()))
    maxpos, maxp = int(inp.pos.max()), int(inp.prompt_len.max())
    for mode in (O.BAND, O.ROWDIAG):
        m = da.mask(mode, cfg.W, cfg.B, cfg.G)
        cap = da.keep_cap(m, maxpos, maxp, head_wb=wb)
        out, lse, _, _ = da.sparse_decode_attn_masked(m, *args, cap=cap, split=split, block_table=bt,
                                                      want_lse=True, head_wb=head_wb)
        torch.cuda.synchronize()
        ref_o, ref_l = _per_head_reference(inp, wb, mode)
        assert_close(out.cpu(), lse.cpu(), ref_o, ref_l, cfg.dtype)
    same = torch.tensor([[cfg.W, cfg.B]] * cfg.hq, dtype=torch.int32, device=dev())
    m = da.mask(O.ROWDIAG, cfg.W, cfg.B, cfg.G)
    cap = da.keep_cap(m, maxpos, maxp)
    o1, l1, _, _ = da.sparse_decode_attn_masked(m, *args, cap=cap, split=split, block_table=bt,
                                                want_lse=True, head_wb=same)
    o2, l2, _, _ = da.sparse_decode_attn_masked(m, *args, cap=cap, split=split, block_table=bt,
                                                want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())


def test_sink_plus_window_mode():
    """StreamingLLM-style attention sinks plus a recent window is the band
    mode with the sinks as the prompt and B >= W: it keeps exactly keys
    j < P and i - W <= j <= i.  Against the oracle, and the keep-set against
    that closed description."""
    cfg = wl.small_decode("gqa_b64", n_seq=4, prompt=(4, 4), W=200, B=200)
    inp = wl.decode_inputs(cfg)
    for i, P in zip(inp.pos.tolist(), inp.prompt_len.tolist()):
        ks = O.keepset(int(i), P=int(P), W=200, B=200, G=cfg.G, mode=O.BAND)
        want = sorted(set(range(min(P, i + 1))) | set(range(max(0, i - 200), i + 1)))
        assert ks.tolist() == want
    k, v, bt = caches(inp)
    m = da.mask(O.BAND, 200, 200, cfg.G)
    cap = da.keep_cap(m, int(inp.pos.max()), int(inp.prompt_len.max()))
    out, lse, _, _ = da.sparse_decode_attn_masked(m, inp.q.to(dev()), k, v, inp.seq.to(dev()),
                                                  inp.pos.to(dev()), inp.prompt_len.to(dev()), cap=cap,
                                                  split=4096, block_table=bt, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = run_oracle(inp, O.BAND)
    assert_close(out.cpu(), lse.cpu(), ref_o, ref_l, cfg.dtype)


def test_per_head_masks_fp32_groups_not_supported():
    cfg = wl.small_decode("gqa_b64", n_seq=1, dtype="f32")
    inp = wl.decode_inputs(cfg)
    k, v, bt = caches(inp)
    wb = torch.tensor([[cfg.W, cfg.B]] * cfg.hq, dtype=torch.int32, device=dev())
    m = da.mask(O.ROWDIAG, cfg.W, cfg.B, cfg.G)
    with pytest.raises(da.DiagAttnError) as e:
        da.sparse_decode_attn_masked(m, inp.q.to(dev()), k, v, inp.seq.to(dev()), inp.pos.to(dev()),
                                     inp.prompt_len.to(dev()), cap=2000, split=4096, block_table=bt,
                                     head_wb=wb)
    assert e.value.status == -2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_context(dtype):
    """Queries ~100k positions into their request (prompt 2000): the dense
    keep-set spans 25 chunks of the longest split (4096) and the merge; the
    row-diagonal one a single chunk.  Both paths against the oracle, and the
    mask path bitwise against the list path."""
    n_seq, hq, hkv, hd, L = 2, 4, 2, 128, 100_001
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(21)
    k = torch.randn((n_seq, hkv, L, hd), generator=g).to(tdt)
    v = torch.randn((n_seq, hkv, L, hd), generator=g).to(tdt)
    q = torch.randn((3, hq, hd), generator=g).to(tdt)
    pos = torch.tensor([100_000, 99_871, 65_537], dtype=torch.int32)
    prompt = torch.tensor([2000, 2000, 17], dtype=torch.int32)
    seq = torch.tensor([0, 1, 1], dtype=torch.int32)
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    for mode, split in ((O.DENSE, 4096), (O.ROWDIAG, 4096)):
        m = da.mask(mode, 256, 3, 64)
        cap = da.keep_cap(m, int(pos.max()), int(prompt.max()))
        count, idx, _, _ = da.keepset_build(m, pos.to(dev()), prompt.to(dev()), cap)
        o1, l1 = da.sparse_decode_attn(qd, kd, vd, seq.to(dev()), count, idx, split=split, want_lse=True)
        o2, l2, c2, i2 = da.sparse_decode_attn_masked(m, qd, kd, vd, seq.to(dev()), pos.to(dev()),
                                                      prompt.to(dev()), cap=cap, split=split,
                                                      want_lse=True, want_lists=True)
        torch.cuda.synchronize()
        assert torch.equal(count, c2) and torch.equal(o1, o2) and torch.equal(l1, l2)
        for qi in range(3):
            n = int(count[qi])
            assert torch.equal(idx[qi, :n], i2[qi, :n])
        ref_o, ref_l = O.decode_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                          pos.numpy(), prompt.numpy(), seq.numpy(),
                                          W=256, B=3, G=64, mode=mode)
        assert_close(o2.cpu(), l2.cpu(), ref_o, ref_l, dtype)


def test_scheduled_batch_order_moves_only_slots():
    """The batch laid out in da_decode_schedule's order (the serving-layer
    layout the benchmark times) gives every query bit for bit the output,
    LSE and keep-set list it gets in the generated order."""
    cfg = wl.CONFIGS["paged_b128"]
    inp = wl.decode_inputs(cfg)
    m = da.mask(cfg.modes[0], cfg.W, cfg.B, cfg.G)
    cost = [da.keep_count(m, int(p), int(P)) for p, P in zip(inp.pos.tolist(), inp.prompt_len.tolist())]
    perm = da.decode_schedule(cost, cfg.hkv).long()
    assert sorted(perm.tolist()) == list(range(inp.n_q))
    cap = max(cost)
    k, v, bt = caches(inp)
    res = []
    for p in (torch.arange(inp.n_q), perm):
        q = inp.q[p].contiguous().to(dev())
        o, lse, c, i = da.sparse_decode_attn_masked(
            m, q, k, v, inp.seq[p].contiguous().to(dev()), inp.pos[p].contiguous().to(dev()),
            inp.prompt_len[p].contiguous().to(dev()), cap=cap, split=4096, block_table=bt,
            want_lse=True, want_lists=True)
        torch.cuda.synchronize()
        res.append((o.cpu(), lse.cpu(), c.cpu(), i.cpu()))
    (o0, l0, c0, i0), (o1, l1, c1, i1) = res
    assert torch.equal(o1, o0[perm]) and torch.equal(l1, l0[perm]) and torch.equal(c1, c0[perm])
    for slot in range(inp.n_q):
        n = int(c1[slot])
        assert torch.equal(i1[slot, :n], i0[perm[slot], :n])


@pytest.mark.parametrize("name,split", [("gqa_b64", 4096), ("gqa_b64", 37), ("paged_b128", 4096),
                                        ("llamagen_b16", 4096), ("llamagen_b16", 50)])
def test_per_kv_head_lists(name, split):
    """One list per kv head (the builder with a (W, B) per kv head) through
    the list decode: every query head against the oracle run with its kv
    head's mask, and bitwise the mask form with those (W, B) given per
    query head.  Splits below the list lengths exercise the merge, which
    then reads the counts per (query, kv head)."""
    cfg = wl.small_decode(name, n_seq=3)
    inp = wl.decode_inputs(cfg)
    k, v, bt = caches(inp)
    grp = cfg.hq // cfg.hkv
    rng = np.random.default_rng(31)
    wb_kv = np.stack([rng.integers(0, 300, cfg.hkv), rng.integers(0, 7, cfg.hkv)], axis=1).astype(np.int32)
    wb_q = np.repeat(wb_kv, grp, axis=0)
    q, seq = inp.q.to(dev()), inp.seq.to(dev())
    pos, prompt = inp.pos.to(dev()), inp.prompt_len.to(dev())
    maxpos, maxp = int(inp.pos.max()), int(inp.prompt_len.max())
    for mode in (O.BAND, O.ROWDIAG):
        m = da.mask(mode, cfg.W, cfg.B, cfg.G)
        cap = da.keep_cap(m, maxpos, maxp, head_wb=wb_kv)
        count, idx, _, _ = da.keepset_build(m, pos, prompt, cap, head_wb=torch.from_numpy(wb_kv).to(dev()))
        ws = da.decode_workspace(inp.n_q, cfg.hq, cfg.hd, cap, split, dev())
        out, lse = da.sparse_decode_attn(q, k, v, seq, count, idx, split=split, block_table=bt,
                                         want_lse=True, workspace=ws)
        o2, l2, _, _ = da.sparse_decode_attn_masked(m, q, k, v, seq, pos, prompt, cap=cap, split=split,
                                                    block_table=bt, want_lse=True, workspace=ws,
                                                    head_wb=torch.from_numpy(wb_q).to(dev()))
        torch.cuda.synchronize()
        ref_o, ref_l = _per_head_reference(inp, wb_q, mode)
        assert_close(out.cpu(), lse.cpu(), ref_o, ref_l, cfg.dtype)
        assert torch.equal(out.cpu(), o2.cpu()) and torch.equal(lse.cpu(), l2.cpu())

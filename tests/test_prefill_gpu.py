"""GPU band-masked prefill (MFMA) vs the fp64 oracle.

bf16 inputs: max |o - ref| <= 2e-2 with the oracle run on the same
bf16-rounded values; natural-log LSE within 1e-3."""
import numpy as np
import pytest
import torch

import ar_image_generation_amd as da
import oracle as O
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL = 2e-2


def run(q, k, v, prompt, mode, W, B, G):
    m = da.mask(mode, W, B, G)
    out, lse = da.band_prefill_attn(m, q.to(DEV), k.to(DEV), v.to(DEV),
                                    torch.as_tensor(prompt, dtype=torch.int32).to(DEV),
                                    want_lse=True)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_rows(q, k, v, prompt, mode, W, B, G, rows):
    heads, kvh = q.shape[1], k.shape[1]
    rep = heads // kvh
    K = np.repeat(k.double().numpy(), rep, axis=1)
    V = np.repeat(v.double().numpy(), rep, axis=1)
    return O.prefill_attention(q.double().numpy(), K, V, prompt, W=W, B=B, G=G, mode=mode,
                               rows=rows)


def check(out, lse, ref):
    o = out.double().numpy()
    l = lse.double().numpy()
    worst = 0.0
    for (b, h, i), (ro, rl) in ref.items():
        err = np.abs(o[b, h, i] - ro).max()
        worst = max(worst, err)
        assert err <= ATOL, ((b, h, i), err)
        assert abs(l[b, h, i] - rl) <= 1e-3 * max(1.0, abs(rl)), ((b, h, i), l[b, h, i], rl)
    return worst


def randn(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("mode", [O.ROWDIAG, O.BAND, O.DENSE])
@pytest.mark.parametrize("hd,heads,kvh", [(128, 2, 2), (64, 4, 2)])
def test_small_all_rows(mode, hd, heads, kvh):
    """Ragged length (not a tile multiple), window crossing the prompt,
    GQA heads: every row against the oracle."""
    P, G, rows_w, B = 20, 16, 4, 3
    W = rows_w * G
    n = P + G * G + 7
    q, k, v = randn((2, heads, n, hd), 1), randn((2, kvh, n, hd), 2), randn((2, kvh, n, hd), 3)
    prompt = [P, 3]
    out, lse = run(q, k, v, prompt, mode, W, B, G)
    rows = [(b, h, i) for b in range(2) for h in range(heads) for i in range(n)]
    check(out, lse, oracle_rows(q, k, v, prompt, mode, W, B, G, rows))


@pytest.mark.parametrize("n,P,W,B,G", [(1, 0, 4, 1, 4), (5, 9, 4, 1, 4), (63, 0, 0, 0, 8),
                                       (65, 64, 8, 2, 8), (130, 7, 40, 9, 10)])
def test_edge_shapes(n, P, W, B, G):
    q, k, v = randn((1, 2, n, 128), 4), randn((1, 2, n, 128), 5), randn((1, 2, n, 128), 6)
    for mode in (O.ROWDIAG, O.BAND):
        out, lse = run(q, k, v, [P], mode, W, B, G)
        rows = [(0, h, i) for h in range(2) for i in range(n)]
        check(out, lse, oracle_rows(q, k, v, [P], mode, W, B, G, rows))


def test_single_kept_key_rows_return_their_value():
    """P = 0, W = 0, B = 0: each row keeps only its own key."""
    n = 70
    q, k, v = randn((1, 2, n, 128), 7), randn((1, 2, n, 128), 8), randn((1, 2, n, 128), 9)
    out, _ = run(q, k, v, [0], O.BAND, 0, 0, 4)
    assert torch.equal(out, v)


def test_full_prefill_workload_sampled_rows():
    """The full prefill workload (2 x 32 heads x 4352 tokens, head_dim 128):
    a seeded sample of rows, including the prompt boundary, the first rows
    past the window and the last row."""
    cfg = wl.PREFILL_CONFIGS["prefill_b2"]
    inp = wl.prefill_inputs(cfg)
    out, lse = run(inp.q, inp.k, inp.v, inp.prompt_len.tolist(), cfg.mode, cfg.W, cfg.B, cfg.G)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(0)
    fixed = [0, 1, 63, 64, cfg.P - 1, cfg.P, cfg.P + 1, cfg.P + cfg.W, cfg.P + cfg.W + 1,
             cfg.n - 1]
    rows = []
    for b in range(cfg.batch):
        for h in rng.choice(cfg.heads, size=6, replace=False):
            for i in fixed + rng.choice(cfg.n, size=8, replace=False).tolist():
                rows.append((b, int(h), int(i)))
    check(out, lse, oracle_rows(inp.q, inp.k, inp.v, inp.prompt_len.tolist(), cfg.mode, cfg.W,
                                cfg.B, cfg.G, rows))


def test_prefill_row_matches_decode_at_that_position():
    """Row i of prefill and a decode query at position i over the same cache
    agree (two different kernels, same keep-set)."""
    P, G, W, B, n = 16, 16, 64, 2, 16 + 256
    q, k, v = randn((1, 4, n, 128), 10), randn((1, 4, n, 128), 11), randn((1, 4, n, 128), 12)
    out, _ = run(q, k, v, [P], O.ROWDIAG, W, B, G)
    pos = torch.arange(n, dtype=torch.int32)
    m = da.mask(O.ROWDIAG, W, B, G)
    count, idx, _, _ = da.keepset_build(m, pos.to(DEV), torch.full((n,), P, dtype=torch.int32).to(DEV),
                                        da.keep_cap(m, n - 1, P))
    qd = q[0].permute(1, 0, 2).contiguous().to(DEV)          # [n, heads, hd]
    dec, _ = da.sparse_decode_attn(qd, k.to(DEV), v.to(DEV), torch.zeros(n, dtype=torch.int32).to(DEV),
                                   count, idx, split=4096)
    torch.cuda.synchronize()
    diff = (dec.cpu().float().permute(1, 0, 2) - out[0].float()).abs().max().item()
    assert diff <= ATOL


@pytest.mark.parametrize("seed", range(10))
def test_random_masks_and_shapes(seed):
    """Seeded random masks (any mode, overlapping bands, G = 1, W = 0,
    prompts longer than the sequence), ragged lengths, both head sizes and
    GQA ratios: every row against the oracle."""
    rng = np.random.default_rng(100 + seed)
    mode = int(rng.choice([O.DENSE, O.BAND, O.ROWDIAG]))
    hd = int(rng.choice([64, 128]))
    kvh, rep = int(rng.choice([1, 2])), int(rng.choice([1, 2]))
    heads = kvh * rep
    n = int(rng.integers(1, 600))
    batch = int(rng.integers(1, 3))
    G = int(rng.integers(1, 80))
    W, B = int(rng.integers(0, 300)), int(rng.integers(0, 12))
    prompt = [int(rng.integers(0, n + 6)) for _ in range(batch)]
    q = randn((batch, heads, n, hd), 200 + seed)
    k = randn((batch, kvh, n, hd), 300 + seed)
    v = randn((batch, kvh, n, hd), 400 + seed)
    out, lse = run(q, k, v, prompt, mode, W, B, G)
    rows = [(b, h, i) for b in range(batch) for h in range(heads) for i in range(n)]
    check(out, lse, oracle_rows(q, k, v, prompt, mode, W, B, G, rows))


@pytest.mark.parametrize("n,P,W,B,G,hd", [(300, 17, 96, 2, 32, 128), (300, 0, 96, 8, 48, 128),
                                          (129, 5, 40, 8, 32, 64), (500, 64, 144, 2, 48, 128),
                                          (77, 100, 30, 0, 16, 64), (513, 3, 1000, 7, 16, 128),
                                          (1, 0, 4, 1, 16, 128), (1100, 256, 256, 3, 64, 128),
                                          (260, 260, 64, 3, 32, 64), (700, 31, 2**31 - 1, 8, 64, 128),
                                          (1030, 0, 160, 5, 80, 128), (1100, 5, 2100, 3, 1016, 128)])
def test_row_diagonal_shapes(n, P, W, B, G, hd):
    """Row-diagonal masks at raster widths of 16 to 80 with bands up to 8:
    ragged lengths, prompts longer than the sequence, windows past the
    sequence, a group of query heads per kv head.  Every row against the
    oracle."""
    q = randn((2, 4, n, hd), 31)
    k, v = randn((2, 2, n, hd), 32), randn((2, 2, n, hd), 33)
    prompt = [P, n // 3]
    out, lse = run(q, k, v, prompt, O.ROWDIAG, W, B, G)
    rows = [(b, h, i) for b in range(2) for h in range(4) for i in range(n)]
    check(out, lse, oracle_rows(q, k, v, prompt, O.ROWDIAG, min(W, n), B, G, rows))


@pytest.mark.parametrize("mode", [O.ROWDIAG, O.DENSE])
def test_longest_sequence_sampled_rows(mode):
    """The longest sequence the prefill takes (65536 tokens, its whole tile
    list in LDS): sampled rows -- the first and last query tiles, tile
    boundaries and seeded random rows -- against the oracle."""
    n, P, W, B, G = 65536, 256, 256, 3, 64
    q = randn((1, 1, n, 128), 11)
    k = randn((1, 1, n, 128), 12)
    v = randn((1, 1, n, 128), 13)
    out, lse = run(q, k, v, [P], mode, W, B, G)
    rng = np.random.default_rng(14)
    pick = {0, 1, 127, 128, 255, 256, 257, n - 129, n - 128, n - 2, n - 1}
    pick |= {int(x) for x in rng.integers(0, n, 16)}
    check(out, lse, oracle_rows(q, k, v, [P], mode, W, B, G, [(0, 0, i) for i in sorted(pick)]))


@pytest.mark.parametrize("W,B,G", [(2**31 - 1, 2**31 - 1, 1), (2**31 - 1, 2**31 - 1, 7),
                                   (40, 2**31 - 1, 5), (2**31 - 1, 2**30, 9),
                                   (2**31 - 1, 3, 9), (100, 2**30, 64)])
def test_window_and_band_at_the_int32_limit(W, B, G):
    """W and B up to INT32_MAX: a window or band wider than the sequence
    keeps what an unbounded one keeps, with no overflow in the band
    pattern or the range tests (rows with P = 0 and with a prompt)."""
    n = 150
    q, k, v = randn((2, 2, n, 128), 21), randn((2, 2, n, 128), 22), randn((2, 2, n, 128), 23)
    prompt = [0, 17]
    # The oracle's vectorised rows loop over the diagonals a window can
    # reach, so it is run with W, B cut to n; the pairwise definition
    # (O.keep, no such loop) confirms the cut changes no pair.
    Wr, Br = min(W, n), min(B, n)
    for mode in (O.ROWDIAG, O.BAND):
        for P in prompt:
            for i in range(0, n, 7):
                want = [O.keep(i, j, P=P, W=W, B=B, G=G, mode=mode) for j in range(n)]
                assert O.keep_row(i, n, P=P, W=Wr, B=Br, G=G, mode=mode).tolist() == want
        out, lse = run(q, k, v, prompt, mode, W, B, G)
        rows = [(b, h, i) for b in range(2) for h in range(2) for i in range(n)]
        check(out, lse, oracle_rows(q, k, v, prompt, mode, Wr, Br, G, rows))


def _parse_tiles(tiles, batch, n):
    n_qt = (n + 127) // 128
    max_tiles = (n + 63) // 64 + 3
    raw = tiles.cpu().numpy().view(np.int32)
    counts = raw[:batch * n_qt].reshape(batch, n_qt)
    off = ((batch * n_qt * 4 + 15) // 16 * 16) // 4
    ent = raw[off:off + batch * n_qt * max_tiles * 8].reshape(batch, n_qt, max_tiles, 8)
    return counts, ent, max_tiles


@pytest.mark.parametrize("mode,n,P,W,B,G", [(O.ROWDIAG, 600, 256, 256, 3, 64), (O.ROWDIAG, 300, 17, 96, 2, 32),
                                            (O.ROWDIAG, 283, 3, 64, 3, 16), (O.BAND, 283, 20, 64, 3, 16),
                                            (O.DENSE, 283, 20, 64, 3, 16), (O.ROWDIAG, 130, 7, 40, 9, 10),
                                            (O.ROWDIAG, 700, 31, 2**31 - 1, 8, 64)])
def test_tile_lists_hold_every_kept_pair_once(mode, n, P, W, B, G):
    """The prefill tile lists against the oracle's keep rule: every kept
    (row, key) pair lies in exactly one listed (tile, 16-key block) marked as
    holding a kept pair -- prompt tiles counting keys below the prompt end,
    window tiles keys at or past it -- every block marked wholly kept is, in
    a half tile each wave (row blocks w and w + 4 of the query tile) marks at
    most two blocks, and whole tiles come first."""
    prompt = [P, min(P, n) // 2]
    m = da.mask(mode, W, B, G)
    tiles = da.prefill_tiles_build(m, torch.as_tensor(prompt, dtype=torch.int32).to(DEV), n)
    torch.cuda.synchronize()
    counts, ent, max_tiles = _parse_tiles(tiles, len(prompt), n)
    for b, Pb in enumerate(prompt):
        Pc = min(Pb, n)
        keep = np.stack([O.keep_row(i, n, P=Pc, W=min(W, n), B=min(B, n), G=G, mode=mode) for i in range(n)])
        seen = np.zeros((n, n), dtype=np.int32)
        for qt in range(counts.shape[1]):
            cnt, n_whole = int(counts[b, qt]) & 0xffff, int(counts[b, qt]) >> 16
            assert 0 < cnt <= max_tiles and n_whole <= cnt

            i0 = 128 * qt
            for e in range(cnt):
                j0, nlo, nhi, win, flo, fhi = (int(x) for x in ent[b, qt, e, :6])
                need = (nlo & 0xffffffff) | ((nhi & 0xffffffff) << 32)
                full = (flo & 0xffffffff) | ((fhi & 0xffffffff) << 32)
                assert -15 <= j0 < n and need != 0
                for w in range(4):
                    if e >= n_whole:
                        union = ((need >> (8 * w)) | (need >> (8 * w + 4))) & 0xf
                        assert bin(union).count("1") <= 2, (b, qt, e, w)
                    for rb in range(2):
                        r0 = i0 + 16 * w + 64 * rb
                        bits = (need >> (8 * w + 4 * rb)) & 0xf
                        for kq in range(4):
                            if not (bits >> kq) & 1:
                                continue
                            jl = j0 + 16 * kq
                            for i in range(r0, min(r0 + 16, n)):
                                js = np.arange(max(jl, 0), min(jl + 16, n))
                                js = js[(js >= Pc) if win else (js < Pc) if mode != O.DENSE else js >= 0]
                                kept = keep[i, js]
                                seen[i, js[kept]] += 1
                                if (full >> (8 * w + 4 * rb + kq)) & 1:
                                    assert kept.all() and len(js) == 16
        assert np.array_equal(seen > 0, keep), b
        assert seen.max() <= 1, b

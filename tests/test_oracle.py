"""Pins for the CPU oracle: what the pages and plain mathematics fix.

Each test checks the oracle against something other than itself: the
numbers printed by the worked example, the sparsity closed form, the
per-query count closed forms, a library attention routine, or closed-form
special cases.  Together they fail on a dropped mask term, a wrong sign or
offset in the keep rule, a transposed operand or a wrong head mapping.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))


def ex_mask(mode=O.BAND):
    return dict(P=0, W=GOLD["W"], B=GOLD["B"], G=1, mode=mode)


# ------------------------------------------------ worked example (summary page)

def test_worked_example_matrix_form_keeps_printed_keys():
    i, N = GOLD["i"], GOLD["N"]
    ks = O.keepset(i, N, causal=False, **ex_mask())
    assert ks.tolist() == GOLD["kept_matrix_form"]
    assert O.keepset_loop(i, N, causal=False, **ex_mask()) == GOLD["kept_matrix_form"]
    for j in GOLD["skipped_named"]:
        assert not O.keep(i, j, causal=False, **ex_mask())
    dense = O.keepset(i, N, causal=False, **ex_mask(O.DENSE))
    assert len(dense) == GOLD["kv_reads_dense"]
    assert len(ks) == GOLD["kv_reads_sparse"]


def test_worked_example_decode_form_is_causal_prefix():
    i = GOLD["i"]
    ks = O.keepset(i, **ex_mask())            # causal: keys 0..i
    assert ks.tolist() == [j for j in GOLD["kept_matrix_form"] if j <= i]


def test_worked_example_softmax_of_printed_scores():
    """Scores 0.1, 0.2, 0.5, 0.2 on the kept keys 4..7; the masked keys get
    a large score that would dominate if the mask were dropped."""
    N, i = GOLD["N"], GOLD["i"]
    kept = O.keep_row(i, N, causal=False, **ex_mask())
    s = dict(zip(GOLD["kept_matrix_form"], GOLD["scores_kept"]))
    K = np.array([[s.get(j, 100.0)] for j in range(N)])
    V = np.eye(N)
    o, lse = O.attend(np.array([1.0]), K, V, kept, scale=1.0)
    z = sum(math.exp(x) for x in GOLD["scores_kept"])
    want = [math.exp(s[j]) / z if j in s else 0.0 for j in range(N)]
    assert np.all(o[~kept] == 0.0)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-15)
    assert lse == pytest.approx(math.log(z), abs=1e-15)
    # the printed weights need an unstated temperature: not reproduced
    assert not np.allclose(o[kept], GOLD["printed_weights_not_pinned"], atol=1e-2)


# ------------------------------------------------ sparsity closed form

def sum_M_closed_form(N, W, B):
    """sum_ij M_ij of the printed N x N mask (P = 0, non-causal, N > B):
    (B+1) diagonals on and above the main one, min(B, W) below it."""
    b2 = min(B, W)
    return N * (1 + B + b2) - B * (B + 1) // 2 - b2 * (b2 + 1) // 2


@pytest.mark.parametrize("N,W,B", [(8, 4, 2), (8, 1, 2), (16, 3, 3), (100, 5, 2),
                                   (64, 0, 0), (33, 7, 7), (20, 2, 5), (9, 8, 8)])
def test_sparsity_closed_form(N, W, B):
    M = O.mask_matrix(N, P=0, W=W, B=B, G=1, mode=O.BAND)
    assert int(M.sum()) == sum_M_closed_form(N, W, B)
    assert O.sparsity(M) == pytest.approx(1 - sum_M_closed_form(N, W, B) / N**2, abs=0)


def test_sparsity_worked_example_value():
    M = O.mask_matrix(GOLD["N"], **ex_mask())
    assert int(M.sum()) == 34
    assert O.sparsity(M) == 0.46875


def test_speedup_definition():
    assert O.speedup(3.1, 1.0) == 3.1


# ------------------------------------------------ per-query count closed forms

def band_count(i, P, W, B):
    if i < P:
        return i + 1
    return P + min(B, W, i - P) + 1


def rowdiag_count(i, P, W, B, G):
    """Distances 0..min(W, i-P) covered by the union of the intervals
    [kG - B, kG + B] (enumerated as ranges, not via the predicate)."""
    if i < P:
        return i + 1
    D = min(W, i - P)
    cover = set()
    for k in range(0, D // G + 2):
        cover.update(range(max(0, k * G - B), min(D, k * G + B) + 1))
    return P + len(cover)


@pytest.mark.parametrize("P,W,B,G", [(0, 4, 2, 3), (5, 12, 1, 4), (3, 20, 2, 4),
                                     (16, 64, 2, 16), (7, 9, 0, 5), (2, 30, 4, 6)])
def test_counts_closed_forms(P, W, B, G):
    for i in range(0, P + 3 * W + 5):
        m = dict(P=P, W=W, B=B, G=G)
        assert len(O.keepset(i, mode=O.DENSE, **m)) == i + 1
        assert len(O.keepset(i, mode=O.BAND, **m)) == band_count(i, P, W, B)
        assert len(O.keepset(i, mode=O.ROWDIAG, **m)) == rowdiag_count(i, P, W, B, G)


@pytest.mark.parametrize("P,G,rows,B,want", [(16, 16, 4, 2, 37),   # fp32 sweep
                                              (120, 32, 3, 2, 136),  # LlamaGen-like
                                              (256, 64, 4, 3, 285)])  # GQA
def test_steady_state_counts_of_the_workloads(P, G, rows, B, want):
    """Once the window lies past the prompt: P + rows*(2B+1) + 1."""
    W = rows * G
    assert P + rows * (2 * B + 1) + 1 == want
    for i in (P + W, P + W + 1, P + G * G - 1):
        assert len(O.keepset(i, P=P, W=W, B=B, G=G, mode=O.ROWDIAG)) == want


def test_scalar_and_vectorised_rules_agree():
    rng = np.random.default_rng(0)
    for _ in range(60):
        P, W, B, G = (int(rng.integers(0, 6)), int(rng.integers(0, 14)),
                      int(rng.integers(0, 4)), int(rng.integers(1, 7)))
        N = int(rng.integers(1, 30))
        for mode in (O.DENSE, O.BAND, O.ROWDIAG):
            for causal in (True, False):
                m = dict(P=P, W=W, B=B, G=G, mode=mode, causal=causal)
                for i in range(N):
                    assert O.keepset_loop(i, N, **m) == O.keepset(i, N, **m).tolist()


def test_rowdiag_keeps_spatial_neighbours_rows_above():
    """In raster order the key k rows above and delta columns over sits
    k*G - delta positions back: every such key with |delta| <= B inside the
    window is kept, and visual keys outside the window are not."""
    P, G, B, rows = 3, 8, 2, 3
    W = rows * G
    N = P + G * G
    for i in range(P, N):
        r, c = divmod(i - P, G)
        kept = set(O.keepset(i, P=P, W=W, B=B, G=G, mode=O.ROWDIAG).tolist())
        for k in range(0, rows + 1):
            for dc in range(-B, B + 1):
                rr, cc = r - k, c + dc
                if rr < 0 or not (0 <= cc < G):
                    continue
                j = P + rr * G + cc
                if j > i or i - j > W:
                    continue
                assert j in kept, (i, j)
        assert all(j < P or i - j <= W for j in kept)
        assert set(range(P)) <= kept


def test_prompt_rows_keep_all_earlier_keys():
    for mode in (O.BAND, O.ROWDIAG):
        for i in range(10):
            assert O.keepset(i, P=10, W=3, B=1, G=4, mode=mode).tolist() == list(range(i + 1))


# ------------------------------------------------ runs / tiles

def test_runs_literal():
    assert O.runs([0, 1, 2, 5, 6, 9]).tolist() == [[0, 3], [5, 2], [9, 1]]
    assert O.runs([]).shape == (0, 2)


def test_tiles_literal():
    assert O.tiles([5, 0, 3], 2).tolist() == [[0, 0], [0, 2], [0, 4], [2, 0], [2, 2]]


# ------------------------------------------------ attention

def sdpa(q, k, v, mask=None, is_causal=False, gqa=False):
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, is_causal=is_causal, enable_gqa=gqa)


@pytest.mark.parametrize("mode", [O.DENSE, O.BAND, O.ROWDIAG])
def test_decode_matches_library_sdpa_gqa(mode):
    """Against torch's fp64 scaled_dot_product_attention with a boolean
    mask and its own GQA head mapping."""
    rng = np.random.default_rng(1)
    hq, hkv, hd, L = 6, 2, 8, 41
    P, W, B, G = 5, 12, 1, 4
    K = rng.standard_normal((1, hkv, L, hd))
    V = rng.standard_normal((1, hkv, L, hd))
    pos = np.arange(0, L)
    q = rng.standard_normal((L, hq, hd))
    o, lse = O.decode_attention(q, K, V, pos, np.full(L, P), np.zeros(L, int),
                                W=W, B=B, G=G, mode=mode)
    for i in pos:
        kept = torch.from_numpy(O.keep_row(int(i), L, P=P, W=W, B=B, G=G, mode=mode))
        ref = sdpa(torch.from_numpy(q[i][None, :, None, :]), torch.from_numpy(K),
                   torch.from_numpy(V), mask=kept[None, None, None, :], gqa=True)
        np.testing.assert_allclose(o[i], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def test_dense_mode_is_causal_attention():
    rng = np.random.default_rng(2)
    H, N, hd = 3, 37, 16
    Q, K, V = (rng.standard_normal((1, H, N, hd)) for _ in range(3))
    out = O.prefill_attention(Q, K, V, [4], W=5, B=1, G=3, mode=O.DENSE)
    ref = sdpa(*(torch.from_numpy(x) for x in (Q, K, V)), is_causal=True).numpy()
    for (b, h, i), (o, _) in out.items():
        np.testing.assert_allclose(o, ref[b, h, i], rtol=1e-12, atol=1e-12)


def test_single_kept_key_returns_its_value():
    """P = 0, B = 0, W = 0: the only key is the query's own."""
    rng = np.random.default_rng(3)
    L, hd = 12, 8
    K, V = rng.standard_normal((1, 1, L, hd)), rng.standard_normal((1, 1, L, hd))
    q = rng.standard_normal((L, 1, hd))
    for mode in (O.BAND, O.ROWDIAG):
        o, lse = O.decode_attention(q, K, V, np.arange(L), np.zeros(L, int),
                                    np.zeros(L, int), W=0, B=0, G=3, mode=mode)
        for i in range(L):
            assert np.array_equal(o[i, 0], V[0, 0, i])
            assert lse[i, 0] == pytest.approx(float(q[i, 0] @ K[0, 0, i]) / math.sqrt(hd),
                                              abs=1e-12)


def test_zero_query_gives_mean_of_kept_values():
    rng = np.random.default_rng(4)
    L, hd, P, W, B, G = 50, 4, 6, 20, 1, 5
    K, V = rng.standard_normal((1, 1, L, hd)), rng.standard_normal((1, 1, L, hd))
    q = np.zeros((L, 1, hd))
    o, lse = O.decode_attention(q, K, V, np.arange(L), np.full(L, P), np.zeros(L, int),
                                W=W, B=B, G=G, mode=O.ROWDIAG)
    for i in range(L):
        ks = O.keepset(i, P=P, W=W, B=B, G=G, mode=O.ROWDIAG)
        np.testing.assert_allclose(o[i, 0], V[0, 0, ks].mean(axis=0), atol=1e-13)
        assert lse[i, 0] == pytest.approx(math.log(len(ks)), abs=1e-13)


def test_two_keys_weights_are_logistic():
    """Two kept keys with score gap g get weights 1/(1+e^-g) and 1/(1+e^g)."""
    for gap in (-3.0, -0.5, 0.0, 0.7, 5.0):
        K = np.array([[gap], [0.0], [50.0]])   # third key masked
        kept = np.array([True, True, False])
        o, _ = O.attend(np.array([1.0]), K, np.eye(3), kept, scale=1.0)
        assert o[0] == pytest.approx(1 / (1 + math.exp(-gap)), abs=1e-15)
        assert o[1] == pytest.approx(1 / (1 + math.exp(gap)), abs=1e-15)
        assert o[2] == 0.0


def test_affine_values_and_key_permutation():
    rng = np.random.default_rng(5)
    L, hd = 30, 6
    q, K, V = rng.standard_normal(hd), rng.standard_normal((L, hd)), rng.standard_normal((L, hd))
    kept = rng.random(L) < 0.5
    kept[3] = True
    o, lse = O.attend(q, K, V, kept, 0.4)
    o2, _ = O.attend(q, K, 2.5 * V - 1.0, kept, 0.4)
    np.testing.assert_allclose(o2, 2.5 * o - 1.0, atol=1e-13)
    p = rng.permutation(L)
    o3, lse3 = O.attend(q, K[p], V[p], kept[p], 0.4)
    np.testing.assert_allclose(o3, o, atol=1e-14)
    assert lse3 == pytest.approx(lse, abs=1e-13)


def test_prefill_row_equals_decode_at_that_position():
    rng = np.random.default_rng(6)
    H, N, hd, P, W, B, G = 2, 40, 8, 4, 12, 1, 4
    Q, K, V = (rng.standard_normal((1, H, N, hd)) for _ in range(3))
    pre = O.prefill_attention(Q, K, V, [P], W=W, B=B, G=G, mode=O.ROWDIAG)
    q = Q[0].transpose(1, 0, 2)                         # (N, H, hd)
    dec, _ = O.decode_attention(q, K, V, np.arange(N), np.full(N, P), np.zeros(N, int),
                                W=W, B=B, G=G, mode=O.ROWDIAG)
    for (b, h, i), (o, _) in pre.items():
        np.testing.assert_allclose(o, dec[i, h], atol=1e-14)


def test_prefill_kept_pairs_matches_count_closed_form():
    N, P, W, B, G = 60, 7, 12, 1, 4
    want = sum(rowdiag_count(i, P, W, B, G) for i in range(N))
    assert O.prefill_kept_pairs(N, P, W=W, B=B, G=G, mode=O.ROWDIAG) == want

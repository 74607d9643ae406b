"""Plain fp64 CPU oracle for diagonal-aware sparse attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, nothing else.  It is slow on
purpose: the keep rule is evaluated per (query, key) pair by brute force,
every key up to the sequence end is scored, masked keys get a -inf logit,
and the softmax is taken over the whole row in float64.

Sources.  All pages describe "Understanding and Exploiting Diagonal
Attention Sparsity in Autoregressive Image Generation" (arXiv 2609.19702):
  [abstract] the arXiv abstract on the mlsanity.com index page, section
             "Abstract (arXiv)": decode is bound by KV-cache reads;
             attention concentrates on prompt and local tokens; a diagonal
             pattern follows from the spatial locality of visual tokens;
             the method skips KV entries along the diagonal direction inside
             a recent window.
  [how]      the paper-daily summary page (vsvnakers.github.io), section
             "技术方法详解" (How), items 2 (diagonal pattern from raster-scan
             order) and 3 (the sparse mechanism: a recent window W, a
             diagonal band width B, skipped entries are zeroed or skipped).
  [formula]  same summary, section "核心公式与算法" (core formulas):
             attention = softmax(Q K^T / sqrt(d) (.) M) V with
             M_ij = 1 when |i-j| <= B and j >= i-W, else 0;
             sparsity = 1 - sum_ij M_ij / N^2;  speedup = T_dense / T_sparse.
  [example]  same summary, section "具体技术细节示例" (worked example):
             N = 8, W = 4, B = 2, query i = 6 keeps keys 4..7; KV reads drop
             from 8 to 4.

Readings taken where the pages are silent or garbled (each is restated in
the design notes with its reason):
  * "(.) M" excludes masked keys: their logit is -inf, so they get zero
    weight and the softmax normalises over the kept keys only ([how] item
    3 lets masked entries be skipped; [example] normalises over the four
    kept keys and counts 4 KV reads, not 8).
  * the band test is |i-j| <= B, inclusive ([formula]; [example] keeps
    j = 4 at distance exactly B); the window test j >= i-W is inclusive.
  * prompt tokens j < P are always kept in the sparse modes ([abstract]:
    attention concentrates on the prompt); P = 0 gives the printed M.
  * ROWDIAG: in raster order the token k rows above sits k*G positions
    back, so besides the main band the window also keeps a band of
    half-width B around every offset k*G (k >= 1) that lies inside the
    window ([how] item 2).  Distances are plain sequence distances (no
    correction where a band wraps past a row end).
  * decode is causal: a query at position i reads keys j <= i, its own
    key included.  The printed worked example keeps j = 7 > i = 6, which
    is the full N x N matrix form; ``causal=False`` reproduces it.
  * scale = 1/sqrt(head_dim); query head h reads kv head h // (Hq/Hkv).
"""
from __future__ import annotations

import math

import numpy as np

DENSE, BAND, ROWDIAG = 0, 1, 2


# ---------------------------------------------------------------- keep rule

def keep(i: int, j: int, *, P: int, W: int, B: int, G: int, mode: int,
         causal: bool = True) -> bool:
    """Is key j in the keep-set of query i?  One pair at a time, by the
    definition ([formula] mask M, extended by the prompt and row-offset
    readings in the module header)."""
    if causal and j > i:
        return False
    if mode == DENSE:
        return True
    if j < P:
        return True
    d = i - j
    if mode == BAND:
        return abs(d) <= B and j >= i - W
    if mode == ROWDIAG:
        if d < 0:                       # future keys (matrix form only)
            return -d <= B
        if j < i - W:                   # outside the recent window
            return False
        k = 0
        while k * G <= d + B:           # every diagonal k*G that could reach d
            if abs(d - k * G) <= B:
                return True
            k += 1
        return False
    raise ValueError(f"unknown mode {mode}")


def keep_row(i: int, n_keys: int, *, P: int, W: int, B: int, G: int,
             mode: int, causal: bool = True) -> np.ndarray:
    """keep(i, j) for every j in [0, n_keys), vectorised over j."""
    j = np.arange(n_keys, dtype=np.int64)
    out = np.ones(n_keys, dtype=bool)
    if causal:
        out &= j <= i
    if mode == DENSE:
        return out
    d = i - j
    if mode == BAND:
        rule = (np.abs(d) <= B) & (j >= i - W)
    elif mode == ROWDIAG:
        inwin = (d >= 0) & (j >= i - W)
        near = np.zeros(n_keys, dtype=bool)
        for k in range(0, (W + B) // G + 1):
            near |= np.abs(d - k * G) <= B
        rule = (inwin & near) | ((d < 0) & (-d <= B))
    else:
        raise ValueError(f"unknown mode {mode}")
    return out & ((j < P) | rule)


def keepset(i: int, n_keys: int | None = None, **mask) -> np.ndarray:
    """Ascending key positions kept for query i among [0, n_keys);
    decode (causal) default n_keys = i + 1."""
    if n_keys is None:
        n_keys = i + 1
    return np.nonzero(keep_row(i, n_keys, **mask))[0].astype(np.int64)


def keepset_loop(i: int, n_keys: int | None = None, **mask) -> list:
    """Same as ``keepset`` through the scalar predicate (small cases)."""
    if n_keys is None:
        n_keys = i + 1
    return [j for j in range(n_keys) if keep(i, j, **mask)]


def runs(ks) -> np.ndarray:
    """Maximal runs of consecutive positions in an ascending list, as
    (start, length) rows."""
    out = []
    for j in ks:
        j = int(j)
        if out and out[-1][0] + out[-1][1] == j:
            out[-1][1] += 1
        else:
            out.append([j, 1])
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def tiles(counts, tile: int) -> np.ndarray:
    """Split-KV work list: each query's keep-set cut into consecutive chunks
    of ``tile`` entries, in query order, as (query, first entry) rows."""
    out = []
    for q, c in enumerate(counts):
        for b in range(0, int(c), tile):
            out.append((q, b))
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def mask_matrix(N: int, *, causal: bool = False, **mask) -> np.ndarray:
    """The N x N matrix M of [formula] (non-causal by default, as printed)."""
    return np.stack([keep_row(i, N, causal=causal, **mask) for i in range(N)])


def sparsity(M: np.ndarray) -> float:
    """[formula]: 1 - sum(M) / N^2 for an N x N mask."""
    n = M.shape[0]
    return 1.0 - float(M.sum()) / float(n * n)


def speedup(t_dense: float, t_sparse: float) -> float:
    """[formula]: T_dense / T_sparse."""
    return t_dense / t_sparse


# ---------------------------------------------------------------- attention

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, kept: np.ndarray,
           scale: float):
    """Masked softmax attention of one query row, in float64.

    q: (hd,), K and V: (L, hd), kept: bool (L,).  Every key is scored;
    masked keys get a -inf logit ([formula] with the exclusion reading).
    Returns (o (hd,), lse) where lse = log sum_j exp(s_j) over kept keys.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = (K @ q) * scale
    s = np.where(kept, s, -np.inf)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    o = (w @ V) / z
    return o, m + math.log(z)


def decode_attention(q, K, V, pos, prompt_len, seq, *, W, B, G, mode,
                     scale=None, queries=None):
    """Decode attention for a batch of queries over a logical cache.

    q: (n_q, hq, hd); K, V: (n_seq, hkv, Lmax, hd) in logical position
    order; pos, prompt_len, seq: (n_q,).  Query q of request seq[q] sits at
    position pos[q] and sees keys 0..pos[q] (causal), kept per the mask.
    Returns o (n_q, hq, hd) float64 and lse (n_q, hq); ``queries`` limits
    the work to a subset of query indices (others are left NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, hq, hd = q.shape
    hkv = K.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    o = np.full((n_q, hq, hd), np.nan)
    lse = np.full((n_q, hq), np.nan)
    for qi in (range(n_q) if queries is None else queries):
        i, P, s = int(pos[qi]), int(prompt_len[qi]), int(seq[qi])
        kept = keep_row(i, i + 1, P=P, W=W, B=B, G=G, mode=mode, causal=True)
        for h in range(hq):
            g = h // group
            Kg = np.asarray(K[s, g, :i + 1], dtype=np.float64)
            Vg = np.asarray(V[s, g, :i + 1], dtype=np.float64)
            o[qi, h], lse[qi, h] = attend(q[qi, h], Kg, Vg, kept, scale)
    return o, lse


def prefill_attention(Q, K, V, prompt_len, *, W, B, G, mode, scale=None,
                      rows=None):
    """Causal masked attention of full sequences (prefill).

    Q, K, V: (batch, heads, N, hd).  Row i of (b, h) attends to keys
    j <= i kept for a query at position i with prompt_len[b].  ``rows`` is
    a list of (b, h, i) to compute (default: all); returns a dict mapping
    (b, h, i) to (o, lse).
    """
    bsz, H, N, hd = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    if rows is None:
        rows = [(b, h, i) for b in range(bsz) for h in range(H) for i in range(N)]
    out = {}
    for b, h, i in rows:
        kept = keep_row(i, N, P=int(prompt_len[b]), W=W, B=B, G=G, mode=mode,
                        causal=True)
        out[(b, h, i)] = attend(Q[b, h, i], K[b, h], V[b, h], kept, scale)
    return out


def prefill_kept_pairs(N: int, P: int, *, W, B, G, mode) -> int:
    """Number of kept (i, j) pairs of one causal N x N prefill mask."""
    return int(sum(int(keep_row(i, N, P=P, W=W, B=B, G=G, mode=mode,
                                causal=True).sum()) for i in range(N)))

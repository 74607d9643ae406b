"""Seeded synthetic inputs (CPU tensors) for the decode and prefill workloads.

Nothing here implements the attention method: these are random numbers,
query positions and cache layouts only.  Every draw comes from a random
stream keyed by (seed, purpose, index), so a reduced workload with
fewer requests reproduces the first requests of the full one.

Key/value recipe for the image workloads (the configs describe it only in
words): each (request, kv head, channel) gets an independent zero-mean,
unit-variance separable AR(1) field on the G x G raster grid with
correlation rho = 0.8 to the left and to the upper neighbour.  It is
X = L E L^T with E iid N(0,1) and L the lower-triangular Cholesky factor
of the AR(1) correlation matrix rho^|a-b|, i.e. L[a,b] = rho^(a-b) for
b = 0 and sqrt(1-rho^2) rho^(a-b) for 0 < b <= a.  0.3 * N(0,1) noise is
added on top.  Prompt keys are 2 * N(0,1) (twice the norm of the visual
keys), prompt values N(0,1), queries N(0,1).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import DecodeConfig, PrefillConfig

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


class _Normal:
    """Stream of float32 N(0,1) draws keyed by (seed, purpose, index).

    torch's CPU generator (mt19937) is used because it fills normals about
    3x faster than numpy's; its output depends only on the key."""

    def __init__(self, *key: int):
        state = np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint64)[0]
        self.g = torch.Generator().manual_seed(int(state) & 0x7FFF_FFFF_FFFF_FFFF)

    def __call__(self, shape) -> np.ndarray:
        return torch.randn(tuple(shape), generator=self.g, dtype=torch.float32).numpy()


def _ar1_cholesky(G: int, rho: float) -> np.ndarray:
    a = np.arange(G)
    diff = a[:, None] - a[None, :]
    L = np.where(diff >= 0, rho ** np.clip(diff, 0, None), 0.0)
    L[:, 1:] *= np.sqrt(1.0 - rho * rho)
    return L


def correlated_field(normal: "_Normal", n: int, G: int,
                     rho: float = 0.8) -> np.ndarray:
    """n independent G x G unit-variance fields, float32, shape (n, G, G)."""
    L = _ar1_cholesky(G, rho).astype(np.float32)
    eps = normal((n, G, G))
    return np.matmul(np.matmul(L, eps), L.T)


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q: torch.Tensor                  # [n_q, hq, hd]
    k_logical: torch.Tensor          # [n_seq, hkv, Lmax, hd]
    v_logical: torch.Tensor
    k_cache: torch.Tensor            # layout the library reads (contiguous or paged)
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]   # int32 [n_seq, pages_per_seq] or None
    pos: torch.Tensor                # int32 [n_q]
    prompt_len: torch.Tensor         # int32 [n_q]
    seq: torch.Tensor                # int32 [n_q]

    @property
    def n_q(self) -> int:
        return int(self.pos.numel())

    @property
    def lmax(self) -> int:
        return int(self.k_logical.shape[2])


def _positions(cfg: DecodeConfig, seed: int):
    Pmin, Pmax = cfg.prompt
    r = _rng(seed, 1)
    prompt_s = r.integers(Pmin, Pmax + 1, size=cfg.n_seq) if Pmax > Pmin \
        else np.full(cfg.n_seq, Pmin)
    rp = _rng(seed, 2)
    if cfg.pos_rule == "sweep":
        # every position of the image after the prompt, on every request
        pos = np.concatenate([np.arange(p, p + cfg.n_vis) for p in prompt_s])
        seq = np.repeat(np.arange(cfg.n_seq), cfg.n_vis)
    elif cfg.pos_rule == "after_window":
        # uniform over [P + W, P + n_vis)
        pos = np.array([rp.integers(p + cfg.W, p + cfg.n_vis) for p in prompt_s])
        seq = np.arange(cfg.n_seq)
    elif cfg.pos_rule == "image":
        # uniform over the whole image, [P, P + n_vis)
        pos = np.array([rp.integers(p, p + cfg.n_vis) for p in prompt_s])
        seq = np.arange(cfg.n_seq)
    else:
        raise ValueError(cfg.pos_rule)
    return (prompt_s.astype(np.int64), pos.astype(np.int64),
            seq.astype(np.int64))


def positions(cfg: DecodeConfig, seed: Optional[int] = None):
    """(pos, prompt_len, seq) int32 tensors of a decode workload, without
    generating its cache."""
    seed = cfg.seed if seed is None else seed
    prompt_s, pos, seq = _positions(cfg, seed)
    return (torch.from_numpy(pos.astype(np.int32)),
            torch.from_numpy(prompt_s[seq].astype(np.int32)),
            torch.from_numpy(seq.astype(np.int32)))


def _fill_sequence(cfg: DecodeConfig, seed: int, s: int, P: int, lmax: int,
                   which: int) -> np.ndarray:
    """Logical K (which=0) or V (which=1) rows of request s, float32
    [hkv, lmax, hd]."""
    r = _Normal(seed, 10 + which, s)
    out = np.zeros((cfg.hkv, lmax, cfg.hd), dtype=np.float32)
    if cfg.kv_gen == "normal":
        out[:] = r(out.shape)
        return out
    n_vis = cfg.n_vis
    prompt = r((cfg.hkv, P, cfg.hd))
    if which == 0:
        prompt *= 2.0
    out[:, :P, :] = prompt
    f = correlated_field(r, cfg.hkv * cfg.hd, cfg.G)          # (hkv*hd, G, G)
    f = f.reshape(cfg.hkv, cfg.hd, n_vis).transpose(0, 2, 1)  # (hkv, n_vis, hd)
    noise = r((cfg.hkv, n_vis, cfg.hd))
    out[:, P:P + n_vis, :] = f + np.float32(0.3) * noise
    return out


def decode_inputs(cfg: DecodeConfig, seed: Optional[int] = None) -> DecodeInputs:
    seed = cfg.seed if seed is None else seed
    tdt = _TORCH_DTYPE[cfg.dtype]
    prompt_s, pos, seq = _positions(cfg, seed)
    Pmax = cfg.prompt[1]
    ps = cfg.page_size
    lmax = Pmax + cfg.n_vis
    if ps:
        pages_per_seq = -(-lmax // ps)
        lmax = pages_per_seq * ps
    k_log = torch.empty((cfg.n_seq, cfg.hkv, lmax, cfg.hd), dtype=tdt)
    v_log = torch.empty_like(k_log)
    for s in range(cfg.n_seq):
        P = int(prompt_s[s])
        k_log[s] = torch.from_numpy(_fill_sequence(cfg, seed, s, P, lmax, 0)).to(tdt)
        v_log[s] = torch.from_numpy(_fill_sequence(cfg, seed, s, P, lmax, 1)).to(tdt)
    n_q = int(pos.size)
    q = torch.from_numpy(_Normal(seed, 3)((n_q, cfg.hq, cfg.hd))).to(tdt)

    block_table = None
    k_cache, v_cache = k_log, v_log
    if ps:
        n_pages = cfg.n_seq * pages_per_seq
        perm = _rng(seed, 4).permutation(n_pages).astype(np.int32)
        block_table = torch.from_numpy(perm.reshape(cfg.n_seq, pages_per_seq).copy())
        flat = block_table.reshape(-1).long()

        def to_pages(x):
            pg = x.view(cfg.n_seq, cfg.hkv, pages_per_seq, ps, cfg.hd)
            pg = pg.permute(0, 2, 1, 3, 4).reshape(n_pages, cfg.hkv, ps, cfg.hd)
            out = torch.empty_like(pg)
            out[flat] = pg
            return out

        k_cache, v_cache = to_pages(k_log), to_pages(v_log)

    return DecodeInputs(
        cfg=cfg, q=q, k_logical=k_log, v_logical=v_log,
        k_cache=k_cache, v_cache=v_cache, block_table=block_table,
        pos=torch.from_numpy(pos.astype(np.int32)),
        prompt_len=torch.from_numpy(prompt_s[seq].astype(np.int32)),
        seq=torch.from_numpy(seq.astype(np.int32)))


@dataclass
class PrefillInputs:
    cfg: PrefillConfig
    q: torch.Tensor   # [batch, heads, n, hd]
    k: torch.Tensor
    v: torch.Tensor
    prompt_len: torch.Tensor  # int32 [batch]


def prefill_inputs(cfg: PrefillConfig, seed: Optional[int] = None,
                   n: Optional[int] = None) -> PrefillInputs:
    """Q, K, V ~ N(0,1).  ``n`` overrides the sequence length (for reduced
    cases); the prompt length stays cfg.P."""
    seed = cfg.seed if seed is None else seed
    n = cfg.n if n is None else n
    tdt = _TORCH_DTYPE[cfg.dtype]
    shape = (cfg.batch, cfg.heads, n, cfg.hd)
    out = []
    for which in range(3):
        x = _Normal(seed, 20 + which)(shape)
        out.append(torch.from_numpy(x).to(tdt))
    return PrefillInputs(cfg=cfg, q=out[0], k=out[1], v=out[2],
                         prompt_len=torch.full((cfg.batch,), cfg.P, dtype=torch.int32))

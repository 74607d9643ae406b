"""The five workloads: shapes and mask parameters, nothing else.

Sequence lengths follow the visual-token counts the summary page of
"Understanding and Exploiting Diagonal Attention Sparsity in
Autoregressive Image Generation" lists in its results section
(1024 / 2048 / 4096 visual tokens; a 48x48 grid of 2304 tokens stands in
for 2048, which is not a square).  W is given in tokens (rows x G).

Mode numbers match the C header: 0 = DENSE, 1 = BAND, 2 = ROWDIAG.
"""
from __future__ import annotations

from dataclasses import dataclass, field

DENSE, BAND, ROWDIAG = 0, 1, 2
MODE_NAMES = {DENSE: "dense", BAND: "band", ROWDIAG: "rowdiag"}


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_seq: int              # requests in the batch
    hq: int                 # query heads
    hkv: int                # key/value heads (hq % hkv == 0)
    hd: int                 # head dim
    dtype: str              # "f32" or "bf16" (q, k, v and output)
    prompt: tuple           # (Pmin, Pmax) prompt tokens, inclusive range
    G: int                  # raster grid width (= height)
    W: int                  # recent window, tokens
    B: int                  # diagonal half-width
    modes: tuple            # masks this workload runs
    pos_rule: str           # "sweep" | "after_window" | "image"
    page_size: int = 0      # 0 = contiguous cache, else paged
    kv_gen: str = "normal"  # "normal" | "field"
    seed: int = 0
    queries_per_seq: int = 1
    split: int = 4096       # listed keys per decode workgroup, sparse masks (launch setting)
    dense_split: int = 512  # the same for the dense all-keep run

    @property
    def n_vis(self) -> int:
        return self.G * self.G

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    heads: int
    hd: int
    dtype: str
    P: int
    G: int
    W: int
    B: int
    mode: int
    seed: int = 0

    @property
    def n(self) -> int:
        return self.P + self.G * self.G


CONFIGS = {
    # 1: fp32 correctness sweep, one head, one shared cache, one query per
    #    position 16..271.
    "sweep_f32": DecodeConfig(
        name="sweep_f32", n_seq=1, hq=1, hkv=1, hd=64, dtype="f32",
        prompt=(16, 16), G=16, W=64, B=2, modes=(ROWDIAG,),
        pos_rule="sweep", kv_gen="normal", seed=1, queries_per_seq=256),
    # 2: LlamaGen-like decode step, MHA.
    "llamagen_b16": DecodeConfig(
        name="llamagen_b16", n_seq=16, hq=32, hkv=32, hd=128, dtype="bf16",
        prompt=(120, 120), G=32, W=96, B=2, modes=(ROWDIAG,),
        pos_rule="after_window", kv_gen="field", seed=2),
    # 3: Llama-3-8B-shaped GQA decode, with the dense run at the same shape.
    "gqa_b64": DecodeConfig(
        name="gqa_b64", n_seq=64, hq=32, hkv=8, hd=128, dtype="bf16",
        prompt=(256, 256), G=64, W=256, B=3, modes=(ROWDIAG, DENSE),
        pos_rule="after_window", kv_gen="field", seed=3),
    # 4: paged KV decode, random block table, both sparse modes (row-diagonal
    #    first: the headline step of the benchmark).
    "paged_b128": DecodeConfig(
        name="paged_b128", n_seq=128, hq=32, hkv=8, hd=128, dtype="bf16",
        prompt=(64, 300), G=48, W=96, B=2, modes=(ROWDIAG, BAND),
        pos_rule="image", page_size=16, kv_gen="field", seed=4),
}

PREFILL_CONFIGS = {
    # 5: band-masked prefill on the MFMA path.
    "prefill_b2": PrefillConfig(
        name="prefill_b2", batch=2, heads=32, hd=128, dtype="bf16",
        P=256, G=64, W=256, B=3, mode=ROWDIAG, seed=5),
}


def get(name: str):
    if name in CONFIGS:
        return CONFIGS[name]
    return PREFILL_CONFIGS[name]


def small_decode(name: str, **over) -> DecodeConfig:
    """A reduced copy of a decode workload (same structure, fewer requests)."""
    base = CONFIGS[name]
    d = dict(base.__dict__)
    d.update(over)
    return DecodeConfig(**d)

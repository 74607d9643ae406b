"""Shared pieces of the GPU parity tests: run the library through its
binding, run the oracle on the same inputs, compare."""
import math

import numpy as np
import torch

import ar_image_generation_amd as da
import oracle as O

FP32_RTOL = 1e-5      # per output row: max|o - ref| / max|ref|
BF16_ATOL = 2e-2      # max |o - ref| over all elements
LSE_ATOL = 1e-4


def dev():
    return torch.device("cuda:0")


def build_lists(cfg, pos, prompt_len, mode, cap=None):
    """Keep-set lists on the GPU for one workload and mask mode."""
    m = da.mask(mode, cfg.W, cfg.B, cfg.G)
    if cap is None:
        cap = da.keep_cap(m, int(pos.max()), int(prompt_len.max()))
    count, idx, _, _ = da.keepset_build(m, pos.to(dev()), prompt_len.to(dev()), cap)
    return count, idx


def run_decode(inp, mode, split, paged=None, want_lse=True):
    """Keep-set build + sparse decode for a DecodeInputs on cuda:0."""
    cfg = inp.cfg
    paged = cfg.page_size > 0 if paged is None else paged
    count, idx = build_lists(cfg, inp.pos, inp.prompt_len, mode)
    q = inp.q.to(dev())
    if paged:
        k, v, bt = inp.k_cache.to(dev()), inp.v_cache.to(dev()), inp.block_table.to(dev())
    else:
        k, v, bt = inp.k_logical.to(dev()), inp.v_logical.to(dev()), None
    out, lse = da.sparse_decode_attn(q, k, v, inp.seq.to(dev()), count, idx, split=split,
                                     block_table=bt, want_lse=want_lse)
    torch.cuda.synchronize()
    return out.cpu(), (lse.cpu() if lse is not None else None), count.cpu(), idx.cpu()


def run_oracle(inp, mode, queries=None):
    cfg = inp.cfg
    return O.decode_attention(
        inp.q.double().numpy(), inp.k_logical.double().numpy(), inp.v_logical.double().numpy(),
        inp.pos.numpy(), inp.prompt_len.numpy(), inp.seq.numpy(),
        W=cfg.W, B=cfg.B, G=cfg.G, mode=mode, queries=queries)


def assert_close(out, lse, ref_o, ref_lse, dtype, queries=None):
    o = out.double().numpy()
    l = lse.double().numpy() if lse is not None else None
    qs = range(o.shape[0]) if queries is None else queries
    for qi in qs:
        for h in range(o.shape[1]):
            ref = ref_o[qi, h]
            err = np.abs(o[qi, h] - ref).max()
            if dtype == "f32":
                assert err <= FP32_RTOL * np.abs(ref).max(), (qi, h, err)
            else:
                assert err <= BF16_ATOL, (qi, h, err)
            if l is not None:
                assert abs(l[qi, h] - ref_lse[qi, h]) <= LSE_ATOL * max(1.0, abs(ref_lse[qi, h])), \
                    (qi, h, l[qi, h], ref_lse[qi, h])

"""GPU: the measurement probes read exactly what they claim to read.

The gather probe, at the row offsets ``kept_row_offsets`` resolves from the
oracle's keep-sets, must XOR to the XOR of every 32-bit word of the kept K
and V rows gathered on the host from the logical caches: a probe or an
offset that skipped, repeated or misaddressed a row would give a different
word (bit-exact check)."""
import functools

import numpy as np
import pytest
import torch

import ar_image_generation_amd as da
import oracle as O
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def xor_all(t: torch.Tensor) -> int:
    a = t.contiguous().cpu().view(torch.int32).numpy().ravel()
    return int(np.bitwise_xor.reduce(a.astype(np.uint32))) if a.size else 0


@functools.lru_cache(maxsize=None)
def _case(name):
    """Inputs of a decode workload, the oracle's keep-sets as lists, and the
    XOR of every kept K and V word (every kv head) gathered on the host."""
    cfg = wl.CONFIGS[name]
    inp = wl.decode_inputs(cfg)
    mode = cfg.modes[0]
    ks = [O.keepset(int(p), P=int(P), W=cfg.W, B=cfg.B, G=cfg.G, mode=mode)
          for p, P in zip(inp.pos.tolist(), inp.prompt_len.tolist())]
    cap = max(len(k) for k in ks)
    idx = np.zeros((inp.n_q, cap), dtype=np.int32)
    for q, k in enumerate(ks):
        idx[q, :len(k)] = k
    count = torch.tensor([len(k) for k in ks], dtype=torch.int32)
    want = 0
    for q, k in enumerate(ks):
        s = int(inp.seq[q])
        rows = torch.as_tensor(k, dtype=torch.long)
        want ^= xor_all(inp.k_logical[s, :, rows]) ^ xor_all(inp.v_logical[s, :, rows])
    return cfg, inp, count, torch.from_numpy(idx), want


@pytest.mark.parametrize("name", ["paged_b128", "llamagen_b16", "sweep_f32"])
@pytest.mark.parametrize("grid,loads", [(64, 1), (2048, 2), (300, 4)])
def test_gather_probe_reads_exactly_the_kept_rows(name, grid, loads):
    cfg, inp, count, idx, want = _case(name)
    paged = cfg.page_size > 0
    kc = (inp.k_cache if paged else inp.k_logical).to(DEV).contiguous()
    vc = (inp.v_cache if paged else inp.v_logical).to(DEV).contiguous()
    bt = inp.block_table.to(DEV).contiguous() if paged else None
    offs = da.kept_row_offsets(kc, inp.seq.to(DEV), count.to(DEV), idx.to(DEV), bt)
    assert offs.numel() == int(count.sum()) * cfg.hkv
    sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
    da.gather_read_probe(kc, vc, offs, sink, grid, loads_in_flight=loads)
    torch.cuda.synchronize()
    assert xor_all(sink) == want


def test_read_probe_reads_the_whole_buffer():
    g = torch.Generator().manual_seed(3)
    buf = torch.randint(-2**31, 2**31 - 1, (1 << 20,), generator=g, dtype=torch.int32)
    want = xor_all(buf)
    for grid, loads in ((64, 1), (2048, 8), (300, 16)):
        sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
        da.hbm_read_probe(buf.to(DEV), sink, grid, loads_in_flight=loads)
        torch.cuda.synchronize()
        assert xor_all(sink) == want

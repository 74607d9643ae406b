"""Benchmark of the sparse decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = keep-set build + sparse decode attention (plus the chunk merge
when a keep-set spans several chunks) for one batch of a decode workload, by
default the largest one: paged KV decode of 128 requests x 32 query / 8 kv
heads, head_dim 128, bf16, 16-slot pages behind a seeded random block
table, prompts of 64..300 tokens, a 48x48 raster grid, W = 2 rows, B = 2,
row-diagonal mode (the band mode is reported beside it) -- as one launch
(sparse_decode_attn_masked, which also writes the keep-set lists).  The same
step as two launches (keepset_build, sparse_decode_attn) is reported beside
it, with the dense run at the same shape, the other decode workloads, a
streaming-read probe of the same byte count, a KV append run, the ring-cache
(KV residency) run, a B x W mask sweep and the band prefill.  Inputs are
seeded synthetic tensors, resident in HBM before timing starts.

Cold-cache timing: the KV cache is replicated on the device and step k reads
copy k mod n, with n chosen so that at least 1 GiB of other kept rows is
read between two uses of a copy; the kept rows are then not served from the
4 MB L2s or the 256 MB Infinity Cache, and the reported GB/s is HBM
bandwidth.  A warm (single copy) figure is reported beside it.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD public spec
METRIC = "sparse decode-attn tokens/s + kept-KV GB/s vs HBM peak; speedup vs dense"
ROTATE_BYTES = 1 << 30          # distinct kept bytes between reuses of a copy
MAX_COPY_BYTES = 48 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_key(cfg):
    esz = 2 if cfg.dtype == "bf16" else 4
    return cfg.hkv * 2 * cfg.hd * esz        # K and V rows of every kv head


def ring_inputs(inp, m, page_size=16):
    """Replaces the cache of `inp` by a ring-paged one (rows older than the
    live window recycled, da.ring_block_table), filled the way generation
    would fill it: each request's logical pages in order, later pages
    overwriting their slot.  One query per request."""
    import torch
    import ar_image_generation_amd as da
    k_log, v_log = inp.k_logical, inp.v_logical
    n_seq, hkv, L, hd = k_log.shape
    prompt = [int(inp.prompt_len[inp.seq == s][0]) for s in range(n_seq)]
    bt, total = da.ring_block_table(m, prompt, L, page_size)
    kc = torch.zeros((total, hkv, page_size, hd), dtype=k_log.dtype)
    vc = torch.zeros_like(kc)
    for s in range(n_seq):
        top = int(inp.pos[inp.seq == s].max())
        for lp in range(top // page_size + 1):
            pg = int(bt[s, lp])
            lo, hi = lp * page_size, min(L, (lp + 1) * page_size)
            kc[pg, :, : hi - lo] = k_log[s, :, lo:hi]
            vc[pg, :, : hi - lo] = v_log[s, :, lo:hi]
    inp.k_cache, inp.v_cache, inp.block_table = kc, vc, bt
    return total, n_seq * -(-L // page_size)


class DecodeBench:
    """Device-resident inputs of one decode workload plus rotation copies."""

    def __init__(self, cfg, n_copies=None, split=None, ring=False, order="given"):
        import torch
        import ar_image_generation_amd as da
        import workloads as wl
        self.torch, self.da = torch, da
        self.cfg = cfg
        self.split = split or cfg.split
        t0 = time.time()
        self.inp = wl.decode_inputs(cfg)
        log(f"[bench] {cfg.name}: inputs generated in {time.time() - t0:.1f}s")
        self.order = order
        if order == "balanced":
            # the serving layer's batch layout: queries placed by
            # da_decode_schedule from their host-side keep-set sizes
            inp = self.inp
            m0 = da.mask(cfg.modes[0], cfg.W, cfg.B, cfg.G)
            cost = [da.keep_count(m0, int(p), int(P)) for p, P in zip(inp.pos.tolist(), inp.prompt_len.tolist())]
            perm = da.decode_schedule(cost, cfg.hkv).long()
            inp.q, inp.pos = inp.q[perm].contiguous(), inp.pos[perm].contiguous()
            inp.prompt_len, inp.seq = inp.prompt_len[perm].contiguous(), inp.seq[perm].contiguous()
        dev = torch.device("cuda:0")
        self.dev = dev
        inp = self.inp
        self.q = inp.q.to(dev)
        self.pos = inp.pos.to(dev)
        self.prompt = inp.prompt_len.to(dev)
        self.paged = cfg.page_size > 0 or ring
        self.ring_pages = None
        if ring:
            self.ring_pages = ring_inputs(inp, da.mask(cfg.modes[0], cfg.W, cfg.B, cfg.G))
        k = (inp.k_cache if self.paged else inp.k_logical)
        v = (inp.v_cache if self.paged else inp.v_logical)
        copy_bytes = 2 * k.numel() * k.element_size()
        self.copy_bytes = copy_bytes
        self.n_q = inp.n_q
        self.hosts = (inp.pos.numpy(), inp.prompt_len.numpy())
        self.lists = {}
        self.kept = {}
        for mode in set(cfg.modes) | {da.DENSE}:
            m = da.mask(mode, cfg.W, cfg.B, cfg.G)
            counts = [da.keep_count(m, int(p), int(P)) for p, P in zip(*self.hosts)]
            cap = max(counts)
            count = torch.empty(self.n_q, dtype=torch.int32, device=dev)
            idx = torch.empty((self.n_q, cap), dtype=torch.int32, device=dev)
            self.lists[mode] = (m, cap, count, idx)
            self.kept[mode] = sum(counts)
        sparse_mode = cfg.modes[0]
        if n_copies is None:
            kept_b = self.kept[sparse_mode] * kv_bytes_per_key(cfg)
            n_copies = max(2, math.ceil(ROTATE_BYTES / kept_b))
            n_copies = min(n_copies, max(2, MAX_COPY_BYTES // copy_bytes))
        self.n_copies = n_copies
        t0 = time.time()
        kd, vd = k.to(dev), v.to(dev)
        self.k = kd.repeat(n_copies, 1, 1, 1)
        self.v = vd.repeat(n_copies, 1, 1, 1)
        del kd, vd
        seq = inp.seq.to(dev)
        self.seqs, self.bts = [], []
        for c in range(n_copies):
            if self.paged:
                n_pages = k.shape[0]
                self.seqs.append(seq)
                self.bts.append((inp.block_table + c * n_pages).to(dev).contiguous())
            else:
                self.seqs.append(seq + c * cfg.n_seq)
                self.bts.append(None)
        self.out = torch.empty_like(self.q)
        s_idx, p_idx = inp.seq.long(), inp.pos.long()
        self.k_new = inp.k_logical[s_idx, :, p_idx].contiguous().to(dev)
        self.v_new = inp.v_logical[s_idx, :, p_idx].contiguous().to(dev)
        self.ws = {}
        self.splits = {mode: (cfg.dense_split if mode == da.DENSE else self.split)
                       for mode in self.lists}
        for mode, (m, cap, count, idx) in self.lists.items():
            self.ws[mode] = da.decode_workspace(self.n_q, cfg.hq, cfg.hd, cap, self.splits[mode], dev)
            self.build(mode)            # lists are valid from construction on
        torch.cuda.synchronize()
        log(f"[bench] {cfg.name}: {n_copies} cache copies ({n_copies * copy_bytes / 2**30:.1f} GiB) "
            f"on device in {time.time() - t0:.1f}s")

    def build(self, mode):
        m, cap, count, idx = self.lists[mode]
        self.da.keepset_build(m, self.pos, self.prompt, cap, count=count, idx=idx)

    def decode(self, mode, c):
        m, cap, count, idx = self.lists[mode]
        self.da.sparse_decode_attn(self.q, self.k, self.v, self.seqs[c], count, idx,
                                   split=self.splits[mode], block_table=self.bts[c],
                                   out=self.out, workspace=self.ws[mode])

    def decode_masked(self, mode, c, append=False):
        """Keep-set build and attention in one launch; the lists are written
        too (the same count/idx keepset_build writes).  append=True also
        writes each query's own K/V row (the values already there)."""
        m, cap, count, idx = self.lists[mode]
        kn, vn = (self.k_new, self.v_new) if append else (None, None)
        self.da.sparse_decode_attn_masked(m, self.q, self.k, self.v, self.seqs[c], self.pos,
                                          self.prompt, cap=cap, split=self.splits[mode],
                                          block_table=self.bts[c], out=self.out,
                                          workspace=self.ws[mode], count=count, idx=idx,
                                          k_new=kn, v_new=vn)

    def kept_bytes(self, mode):
        return self.kept[mode] * kv_bytes_per_key(self.cfg)

    def step(self, mode, c, path):
        """One step: 'fused' = decode_masked; 'lists' = keepset_build then
        sparse_decode_attn; 'decode' = sparse_decode_attn on built lists."""
        if path in ("fused", "append"):
            self.decode_masked(mode, c, append=path == "append")
            return
        if path == "lists":
            self.build(mode)
        self.decode(mode, c)

    def gather_us(self, mode, steps, warmup):
        """The gather probe on this step's rows: every kept K/V row read once
        at its byte offset (resolved beforehand through the lists and the
        block table of each cache copy) and nothing else, cold (rotating
        over the cache copies), best over GATHER_SHAPES.  Returns
        (microseconds, (grid, loads in flight))."""
        torch, da = self.torch, self.da
        m, cap, count, idx = self.lists[mode]
        self.build(mode)
        offs = [da.kept_row_offsets(self.k, self.seqs[c], count, idx, self.bts[c]) for c in range(self.n_copies)]
        sink = torch.empty(8192, dtype=torch.int32, device=self.dev)
        best = None
        for grid, loads in GATHER_SHAPES:
            def run(c, grid=grid, loads=loads):
                da.gather_read_probe(self.k, self.v, offs[c], sink, grid, loads_in_flight=loads)
            us = graph_us(torch, run, self.n_copies, steps, warmup)
            if best is None or us < best[0]:
                best = (us, (grid, loads))
        del offs
        return best

    def burn(self, mode, seconds, path="fused"):
        """Replays graphs of back-to-back steps for `seconds`, untimed: the
        first ~0.1 s of decode steps after the streaming burn-in run up to
        ~5 % slower than the steady state they settle to."""
        t0 = time.time()
        while time.time() - t0 < seconds:
            self.time_graph(mode, 50, 2, path=path)

    def time_graph(self, mode, steps, warmup, with_build=True, rotate=True, path=None):
        """Runs `warmup` eager steps, captures `steps` steps in one HIP graph,
        replays it once untimed and once timed (events on the capture
        stream).  Returns microseconds per step.  with_build=False captures
        decode launches only (the decode kernel's average duration); `path`
        overrides with 'fused', 'append' (fused with KV append), 'lists' or 'decode'."""
        torch = self.torch
        n = self.n_copies if rotate else 1
        path = path or ("lists" if with_build else "decode")
        for w in range(warmup):
            self.step(mode, w % n, path)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(steps):
                self.step(mode, (warmup + s) % n, path)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        del g
        return us

    def time_eager(self, mode, steps, warmup):
        """Steps launched one by one from Python (includes host dispatch)."""
        torch = self.torch
        n = self.n_copies
        for w in range(warmup):
            self.build(mode)
            self.decode(mode, w % n)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.build(mode)
            self.decode(mode, s % n)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / steps


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16, AMD public spec


class PrefillBench:
    """The band-masked prefill workload on the device, with rotation copies
    so that each timed launch reads Q, K, V cold from HBM."""

    def __init__(self, cfg, n_copies=4):
        import torch
        import ar_image_generation_amd as da
        import workloads as wl
        self.torch, self.da, self.cfg = torch, da, cfg
        t0 = time.time()
        inp = wl.prefill_inputs(cfg)
        dev = torch.device("cuda:0")
        self.q = [inp.q.to(dev)]
        self.k = [inp.k.to(dev)]
        self.v = [inp.v.to(dev)]
        for _ in range(n_copies - 1):
            self.q.append(self.q[0].clone())
            self.k.append(self.k[0].clone())
            self.v.append(self.v[0].clone())
        self.o = [torch.empty_like(self.q[0]) for _ in range(n_copies)]
        self.prompt = inp.prompt_len.to(dev)
        self.tiles = {md: da.prefill_tiles_build(da.mask(md, cfg.W, cfg.B, cfg.G), self.prompt, cfg.n)
                      for md in (cfg.mode, da.DENSE)}
        self.n_copies = n_copies
        self.bytes = 4 * self.q[0].numel() * 2          # Q, K, V read once, O written once
        per_head = {}
        for mode in (cfg.mode, da.DENSE):
            m = da.mask(mode, cfg.W, cfg.B, cfg.G)
            per_head[mode] = sum(da.keep_count(m, i, cfg.P) for i in range(cfg.n))
        self.kept_pairs = {md: c * cfg.batch * cfg.heads for md, c in per_head.items()}
        torch.cuda.synchronize()
        log(f"[bench] {cfg.name}: inputs + {n_copies} copies in {time.time() - t0:.1f}s, "
            f"kept pairs/head {per_head[cfg.mode]} (dense causal {per_head[da.DENSE]})")

    def run(self, mode, c):
        cfg = self.cfg
        self.da.band_prefill_attn(self.da.mask(mode, cfg.W, cfg.B, cfg.G), self.q[c], self.k[c],
                                  self.v[c], self.prompt, tiles=self.tiles[mode], out=self.o[c])

    def time_graph(self, mode, steps, warmup):
        torch = self.torch
        for w in range(warmup):
            self.run(mode, w % self.n_copies)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(steps):
                self.run(mode, s % self.n_copies)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / steps

    def burn(self, seconds):
        """Replays a graph of back-to-back sparse prefills for `seconds`, so
        the timed launches see the steady state of sustained matrix work:
        after idle time or memory-only work the first ~0.1 s of back-to-back
        launches run up to ~25 % slower (and launches with idle gaps between
        them ~5 % faster) than a long run."""
        torch = self.torch
        for c in range(self.n_copies):
            self.run(self.cfg.mode, c)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(16):
                self.run(self.cfg.mode, s % self.n_copies)
        t0 = time.time()
        while time.time() - t0 < seconds:
            g.replay()
            g.replay()
            torch.cuda.synchronize()
        del g

    def report(self, steps, warmup, burn_s=0.5):
        """Times the sparse and the dense prefill after `burn_s` seconds of
        the sparse kernel itself."""
        cfg, da = self.cfg, self.da
        self.burn(burn_s)
        us = self.time_graph(cfg.mode, steps, warmup)
        us_d = self.time_graph(da.DENSE, max(4, steps // 2), warmup)
        flops = 4.0 * cfg.hd * self.kept_pairs[cfg.mode]
        flops_d = 4.0 * cfg.hd * self.kept_pairs[da.DENSE]
        hbm_floor = self.bytes / (HBM_PEAK_GBPS * 1e3)            # us
        mfma_floor = flops / (MFMA_BF16_PEAK_TFLOPS * 1e6)       # us
        rec = {
            "workload": cfg.name, "us": round(us, 2),
            "bytes_MB": round(self.bytes / 1e6, 2), "kept_pairs": self.kept_pairs[cfg.mode],
            "algorithmic_GFLOP": round(flops / 1e9, 3),
            "achieved_GBps": round(self.bytes / (us * 1e-6) / 1e9, 1),
            "achieved_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
            "hbm_floor_us": round(hbm_floor, 2), "mfma_floor_us": round(mfma_floor, 2),
            "bound": "hbm" if hbm_floor >= mfma_floor else "mfma",
            "roofline_frac": round(max(hbm_floor, mfma_floor) / us, 4),
            "dense_causal_us": round(us_d, 2),
            "dense_causal_TFLOPs": round(flops_d / (us_d * 1e-6) / 1e12, 2),
            "speedup_vs_dense": round(us_d / us, 3),
        }
        log(f"[bench] {cfg.name}: {us:.2f} us ({rec['achieved_TFLOPs']} TFLOP/s, "
            f"{rec['achieved_GBps']} GB/s), dense causal {us_d:.2f} us")
        return rec


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, budget_s=12.0):
    """The oracle, as it stands, on the same workload: queries of the batch
    taken in order, one at a time, until about `budget_s` seconds of CPU work
    (the sample).  The oracle is plain per-(query, head) numpy; its BLAS is
    held to one thread, which is the parallelism it actually has (small
    matrix-vector products), so `cores` is 1."""
    import numpy as np
    import oracle as O
    import workloads as wl
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    inp = wl.decode_inputs(cfg)
    # float32 copies hold the bf16 values exactly; the oracle takes each
    # slice it reads to float64 itself
    q = inp.q.float().numpy()
    K = inp.k_logical.float().numpy()
    V = inp.v_logical.float().numpy()
    pos, prompt, seq = inp.pos.numpy(), inp.prompt_len.numpy(), inp.seq.numpy()
    mode = cfg.modes[0]
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    done, t0 = 0, time.time()
    try:
        if ctx is not None:
            ctx.__enter__()
        while time.time() - t0 < budget_s:
            O.decode_attention(q, K, V, pos, prompt, seq, W=cfg.W, B=cfg.B, G=cfg.G, mode=mode,
                               queries=[done % inp.n_q])
            done += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.time() - t0
    return {"value": round(done / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{done} queries (all {cfg.hq} heads each) of {cfg.name}, "
                      f"{wl.MODE_NAMES[mode]} mask, taken in order, {dt:.1f}s wall; "
                      f"{O.__name__} fp64 numpy, BLAS held to one thread"}


def traffic_from_profile(workload):
    """HBM bytes per launch of the decode kernel from the committed
    rocprofv3 counter summary, or None when there is none or the kernel
    source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sha256") != kernel_sha(DECODE_SRC):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


DECODE_SRC = [os.path.join(ROOT, "ar_image_generation_amd", "csrc", f)
              for f in ("decode.hip", "common.h")]
PROBE_BYTES = 1 << 30


def graph_us(torch, fn, n, steps, warmup):
    """Microseconds per call of fn(c) for c cycling over n copies: `warmup`
    eager calls, then `steps` calls captured in one HIP graph, replayed once
    untimed and once timed with events on the capture stream."""
    for w in range(warmup):
        fn(w % n)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(steps):
            fn((warmup + s) % n)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del g
    return us


def mask_sweep(b, steps, warmup, w_rows=(1, 2, 3, 6), bands=(0, 1, 2, 4)):
    """Row-diagonal masks over a B x W grid at the benchmark shape: the
    one-launch step's time and kept bytes, and the share of the dense
    attention mass each keep-set captures, exp(lse_sparse - lse_dense), per
    (query, head).  The inputs are synthetic (random queries), so the share
    is a proxy of the quality side, not image quality."""
    torch, da = b.torch, b.da
    cfg = b.cfg
    maxpos, maxp = int(b.inp.pos.max()), int(b.inp.prompt_len.max())
    dense = da.mask(da.DENSE, 0, 0, 1)
    capd = da.keep_cap(dense, maxpos, maxp)
    _, lse_d, _, _ = da.sparse_decode_attn_masked(
        dense, b.q, b.k, b.v, b.seqs[0], b.pos, b.prompt, cap=capd, split=cfg.dense_split,
        block_table=b.bts[0], want_lse=True)
    rows = []
    for wr in w_rows:
        for bw in bands:
            m = da.mask(da.ROWDIAG, wr * cfg.G, bw, cfg.G)
            cap = da.keep_cap(m, maxpos, maxp)
            split = max(cap, 1)
            out = torch.empty_like(b.q)
            lse = torch.empty((b.n_q, cfg.hq), dtype=torch.float32, device=b.q.device)

            def run(c, m=m, cap=cap, split=split, out=out, lse=lse):
                da.sparse_decode_attn_masked(m, b.q, b.k, b.v, b.seqs[c], b.pos, b.prompt, cap=cap,
                                             split=split, block_table=b.bts[c], out=out, lse=lse)
            us = graph_us(torch, run, b.n_copies, steps, warmup)
            run(0)
            torch.cuda.synchronize()
            share = torch.exp(lse - lse_d)
            kept = sum(da.keep_count(m, int(p), int(P)) for p, P in zip(*b.hosts))
            kb = kept * kv_bytes_per_key(cfg)
            rows.append({"W_rows": wr, "W": wr * cfg.G, "B": bw,
                         "kept_per_query": round(kept / b.n_q, 2), "us_per_step": round(us, 2),
                         "kept_GBps": round(kb / (us * 1e-6) / 1e9, 1),
                         "mass_share_mean": round(share.mean().item(), 4),
                         "mass_share_min": round(share.min().item(), 4)})
            log(f"[bench] sweep W={wr}x{cfg.G} B={bw}: {kept / b.n_q:.0f} kept/query, {us:.2f} us, "
                f"mass share {share.mean().item():.3f} (min {share.min().item():.3f})")
    return rows


def per_head_run(b, steps, warmup):
    """Per-query-head windows at the benchmark shape: query heads alternate
    between a window of one raster row and of three (B unchanged), as a
    per-head budget would set them.  A kv group reads its widest keep-set
    once and masks per head, so the bytes read are those of each group's
    widest mask.  Returns the step time, the bytes read and, for reference,
    the bytes of the per-head keep-sets themselves."""
    torch, da = b.torch, b.da
    cfg = b.cfg
    wb = [[cfg.G * (1 if h % 2 == 0 else 3), cfg.B] for h in range(cfg.hq)]
    head_wb = torch.tensor(wb, dtype=torch.int32, device=b.q.device)
    m = da.mask(cfg.modes[0], cfg.W, cfg.B, cfg.G)
    maxpos, maxp = int(b.inp.pos.max()), int(b.inp.prompt_len.max())
    cap = da.keep_cap(m, maxpos, maxp, head_wb=wb)
    out = torch.empty_like(b.q)

    def run(c):
        da.sparse_decode_attn_masked(m, b.q, b.k, b.v, b.seqs[c], b.pos, b.prompt, cap=cap,
                                     split=max(cap, 1), block_table=b.bts[c], out=out,
                                     head_wb=head_wb)
    us = graph_us(torch, run, b.n_copies, steps, warmup)
    row = 2 * cfg.hd * (2 if cfg.dtype == "bf16" else 4)
    grp = cfg.hq // cfg.hkv

    def count(w, bb):
        return sum(da.keep_count(da.mask(cfg.modes[0], w, bb, cfg.G), int(p), int(P))
                   for p, P in zip(*b.hosts))
    read = sum(count(max(w for w, _ in wb[g * grp:(g + 1) * grp]),
                     max(bb for _, bb in wb[g * grp:(g + 1) * grp])) for g in range(cfg.hkv)) * row
    own = sum(count(w, bb) for w, bb in wb) * row / grp
    return {"head_W": [w for w, _ in wb], "us_per_step": round(us, 2),
            "read_MB": round(read / 1e6, 3), "per_head_keepset_MB": round(own / 1e6, 3),
            "read_GBps": round(read / (us * 1e-6) / 1e9, 1)}


def kv_budget_run(steps, warmup, base_requests=128, max_requests=2048, page_size=16, order="given"):
    """KV residency turned into batch size.  The HBM that a full paged cache
    of `base_requests` requests of the paged workload takes (one page per 16
    positions of each request's whole sequence) is the budget.  Under the
    row-diagonal keep-set a request needs only its prompt pages plus a ring
    of window pages (da.ring_pages), so the same budget holds many more
    requests: the largest batch whose ring pages fit is decoded through the
    ring block table (one query per request, position uniform over the
    image as in the workload), and its step time and tokens/s are reported
    beside the full-cache batch's.  Values are random: time depends only on
    the keep-sets.  Returns the record."""
    import numpy as np
    import torch
    import ar_image_generation_amd as da
    import workloads as wl
    base = wl.CONFIGS["paged_b128"]
    md = base.modes[0]
    m = da.mask(md, base.W, base.B, base.G)
    lmax = base.prompt[1] + base.n_vis
    full_pages_per_req = -(-lmax // page_size)
    budget = base_requests * full_pages_per_req
    cfg = wl.small_decode("paged_b128", n_seq=max_requests)
    pos, prompt, seq = wl.positions(cfg)
    need = np.array([da.ring_pages(m, int(P), lmax, page_size) for P in prompt.tolist()])
    n = int(np.searchsorted(np.cumsum(need), budget, side="right"))
    pos, prompt, seq = pos[:n], prompt[:n], seq[:n]
    if order == "balanced":
        cost = [da.keep_count(m, int(p), int(P)) for p, P in zip(pos.tolist(), prompt.tolist())]
        perm = da.decode_schedule(cost, base.hkv).long()
        pos, seq = pos[perm].contiguous(), seq[perm].contiguous()
    bt, total = da.ring_block_table(m, prompt.tolist(), lmax, page_size)
    prompt = prompt[perm].contiguous() if order == "balanced" else prompt
    assert total <= budget
    dev = torch.device("cuda:0")
    kept = sum(da.keep_count(m, int(p), int(P)) for p, P in zip(pos.tolist(), prompt.tolist()))
    kept_b = kept * kv_bytes_per_key(base)
    n_copies = max(2, math.ceil(ROTATE_BYTES / kept_b))
    kc = torch.randn((n_copies * total, base.hkv, page_size, base.hd), dtype=torch.bfloat16, device=dev)
    vc = torch.randn_like(kc)
    bts = [(bt + c * total).to(dev).contiguous() for c in range(n_copies)]
    q = torch.randn((n, base.hq, base.hd), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    pos_d, prompt_d, seq_d = pos.to(dev), prompt.to(dev), seq.to(dev)
    cap = da.keep_cap(m, int(pos.max()), int(prompt.max()))

    def run(c):
        da.sparse_decode_attn_masked(m, q, kc, vc, seq_d, pos_d, prompt_d, cap=cap, split=max(cap, 1),
                                     block_table=bts[c], out=out)
    burn_in([kc, vc], 0.3)
    us = graph_us(torch, run, n_copies, steps, warmup)
    del kc, vc
    torch.cuda.empty_cache()
    return {"mode": wl.MODE_NAMES[md], "kv_budget_pages": budget,
            "kv_budget_GB": round(budget * 2 * base.hkv * page_size * base.hd * 2 / 1e9, 3),
            "full_cache_requests": base_requests, "ring_requests": n, "ring_pages": total,
            "kept_MB": round(kept_b / 1e6, 2),
            "us_per_step": round(us, 2), "tokens_per_s": round(n / (us * 1e-6), 1),
            "kept_GBps": round(kept_b / (us * 1e-6) / 1e9, 1)}


def burn_in(bufs, seconds):
    """Streams the given device tensors until `seconds` have passed, so the
    memory and core clocks have left their idle states before anything is
    timed (the first tens of milliseconds of a fresh process otherwise run
    measurably slower).  Returns the number of passes."""
    import torch
    import ar_image_generation_amd as da
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for t in bufs:
            da.hbm_read_probe(t, sink, 2048)
        torch.cuda.synchronize()
        n += 1
    return n


PROBE_SHAPES = ((2048, 1), (4096, 1), (1024, 2), (512, 4), (256, 8), (2048, 2), (512, 8))
GATHER_SHAPES = ((1024, 1), (2048, 1), (4096, 1), (8192, 1), (1024, 2), (2048, 2), (1024, 4))


def attainable_read(nbytes, steps=50, warmup=10):
    """Streaming-read probe of `nbytes` (rounded down to 16), cold: a HIP
    graph of `steps` reads, each of a different buffer, with >= 1 GiB read
    between two uses of a buffer; the best over (grid, loads in flight per
    thread) shapes.  Returns (microseconds per read, (grid, loads))."""
    import torch
    import ar_image_generation_amd as da
    nb = max(2, math.ceil(ROTATE_BYTES / nbytes))
    size = nbytes // 16 * 16
    bufs = [torch.ones(size // 4, dtype=torch.int32, device="cuda") for _ in range(nb)]
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    best = None
    for grid, depth in PROBE_SHAPES:
        def run(c, grid=grid, depth=depth):
            da.hbm_read_probe(bufs[c % nb], sink, grid, loads_in_flight=depth)
        us = graph_us(torch, run, nb, steps, warmup)
        if best is None or us < best[0]:
            best = (us, (grid, depth))
    del bufs
    torch.cuda.empty_cache()
    return best


def profile_run(args):
    """Only the timed launches (for rocprofv3): K cold steps of the headline
    workload, then one streaming-read probe of PROBE_BYTES (the counter
    calibration: a read of known size).  With --prefill: K launches of the
    band prefill instead."""
    import torch
    import workloads as wl
    if args.prefill:
        pb = PrefillBench(wl.PREFILL_CONFIGS["prefill_b2"], n_copies=2)
        pb.burn(0.5)
        us = pb.time_graph(pb.cfg.mode, args.steps, args.warmup)
        del pb
        torch.cuda.empty_cache()
        counter_calibration()
        log(f"[bench] prefill profile run: {us:.2f} us per launch")
        return
    cfg = wl.CONFIGS[args.workload]
    b = DecodeBench(cfg, split=args.split, order="balanced")
    burn_in([b.k, b.v], 0.5)
    b.burn(cfg.modes[0], 0.3)
    us = b.time_graph(cfg.modes[0], args.steps, args.warmup, path="fused")
    counter_calibration()
    log(f"[bench] profile run: {us:.2f} us/step; probe {PROBE_BYTES} bytes")


def counter_calibration():
    """Kernels of known traffic for scaling the memory counters: a fill of
    PROBE_BYTES, then a streaming read of PROBE_BYTES that are in no cache
    -- written, then pushed out of the L2s and the Infinity Cache by writing
    as many other bytes -- read once."""
    import torch
    import ar_image_generation_amd as da
    buf = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    evict = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    del evict
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    da.hbm_read_probe(buf, sink, 2048)
    torch.cuda.synchronize()


def is_decode_kernel(name):
    """The decode step's kernel: the vector form or the matrix-core form."""
    return "decode_kernel" in name or "decode_mfma_kernel" in name


def summarize(args):
    """Writes profiles/decode_<workload>.txt from three rocprofv3 runs of
    `bench.py --profile-run`: --kernel-trace, --pmc FETCH_SIZE, --pmc WRITE_SIZE."""
    import csv
    import workloads as wl
    import ar_image_generation_amd as da
    cfg = wl.CONFIGS[args.workload]
    trace_dir, fetch_dir, write_dir = args.summarize

    def rows(d, suffix):
        import glob
        out = []
        for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def decode_rows(rs):
        return [r for r in rs if is_decode_kernel(r.get("Kernel_Name", ""))]

    tr = decode_rows(rows(trace_dir, "kernel_trace.csv"))
    durs = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr)
    kname = tr[0]["Kernel_Name"] if tr else "?"
    ks = [r for r in rows(trace_dir, "kernel_trace.csv") if "keepset_kernel" in r["Kernel_Name"]]
    kdur = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in ks)

    def counter(d, name):
        per = {}
        for r in rows(d, "counter_collection.csv"):
            if r.get("Counter_Name") != name:
                continue
            per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), 0.0)
            per[(r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
        dec = [v for (k, _), v in per.items() if is_decode_kernel(k)]
        probe = [v for (k, _), v in per.items() if "read_probe_kernel" in k]
        # the probe buffer's fill: a plain write kernel of PROBE_BYTES
        fill = [v for (k, _), v in per.items() if "FillFunctor<int>" in k]
        return (sum(dec) / len(dec) if dec else None, probe[-1] if probe else None,
                max(fill) if fill else None)

    f_dec, f_probe, _ = counter(fetch_dir, "FETCH_SIZE")
    w_dec, _, w_fill = counter(write_dir, "WRITE_SIZE")
    scale = (PROBE_BYTES / 1024.0) / f_probe if f_probe else None
    wscale = (PROBE_BYTES / 1024.0) / w_fill if w_fill else None
    m = da.mask(cfg.modes[0], cfg.W, cfg.B, cfg.G)
    pos, prompt, _ = wl.positions(cfg)
    kept = sum(da.keep_count(m, int(p), int(P)) for p, P in zip(pos.tolist(), prompt.tolist()))
    kept_bytes = kept * kv_bytes_per_key(cfg)
    hbm = None
    if f_dec is not None and scale is not None and w_dec is not None and wscale is not None:
        hbm = (f_dec * scale + w_dec * wscale) * 1024.0
    avg = sum(durs) / len(durs) if durs else float("nan")
    lines = [
        f"# rocprofv3 summary: decode kernel of the benchmark step (keep-set computed in the "
        f"kernel, lists written, attention), workload {cfg.name}, batch in the slots "
        f"da_decode_schedule gives its queries",
        "# commands (repo root, TMPDIR=/tmp):",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} -o run -- python3 bench.py --profile-run --workload {cfg.name} --steps {args.steps} --warmup {args.warmup}",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o run -- python3 bench.py --profile-run --workload {cfg.name} --steps {args.steps} --warmup {args.warmup}",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o run -- python3 bench.py --profile-run --workload {cfg.name} --steps {args.steps} --warmup {args.warmup}",
        f"#   python3 bench.py --summarize {trace_dir} {fetch_dir} {write_dir} --workload {cfg.name}",
        f"kernel = {kname}",
        f"dispatches = {len(durs)}",
        f"avg_duration_us = {avg / 1e3:.3f}",
        f"median_duration_us = {durs[len(durs) // 2] / 1e3 if durs else float('nan'):.3f}",
        f"min_duration_us = {durs[0] / 1e3 if durs else float('nan'):.3f}",
        f"keepset_kernel_dispatches = {len(kdur)} (the step has no separate keep-set launch)",
        f"kept_bytes_per_launch = {kept_bytes}",
        f"achieved_GBps_from_avg = {kept_bytes / avg if durs else float('nan'):.1f}",
        f"fetch_kib_per_dispatch = {f_dec}",
        f"write_kib_per_dispatch = {w_dec}",
        f"probe_fetch_kib = {f_probe} (cold read of {PROBE_BYTES} bytes, written then evicted by "
        f"another {PROBE_BYTES} bytes of writes)",
        f"fetch_scale = {scale}",
        f"write_calibration_kib = {w_fill} (fill of {PROBE_BYTES} bytes)",
        f"write_scale = {wscale}",
        f"hbm_bytes_per_launch = {hbm}",
        f"traffic_over_kept = {hbm / kept_bytes if hbm else None}",
        f"kernel_sha256 = {kernel_sha(DECODE_SRC)}",
    ]
    out = os.path.join(ROOT, "profiles", f"decode_{cfg.name}_traffic.txt")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))

    stats = [r for r in rows(trace_dir, "kernel_stats.csv") if "da::" in r.get("Name", "")]
    slines = [
        f"# rocprofv3 --kernel-trace --stats summary: benchmark step (keep-set build, lists and "
        f"attention in one launch), workload {cfg.name}",
        f"# ({cfg.n_seq} requests x {cfg.hq}/{cfg.hkv} heads, head_dim {cfg.hd}, {cfg.dtype}, P={cfg.prompt}, "
        f"{cfg.G}x{cfg.G} grid, W={cfg.W}, B={cfg.B}, {wl.MODE_NAMES[cfg.modes[0]]}; cold cache copies)",
        "# command (repo root, TMPDIR=/tmp):",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} -o run -- python3 bench.py "
        f"--profile-run --workload {cfg.name} --steps {args.steps} --warmup {args.warmup}",
        "# columns: name | calls | avg_ns | min_ns | max_ns   (library kernels only)",
    ] + [f"{r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']}"
         for r in stats]
    open(os.path.join(ROOT, "profiles", f"decode_{cfg.name}_kernel_stats.txt"), "w").write(
        "\n".join(slines) + "\n")


def is_prefill_kernel(name):
    """The band prefill's attention kernel (not its tile-list builder)."""
    return "prefill_kernel" in name


def summarize_prefill(args):
    """Writes profiles/prefill_<workload>.txt from rocprofv3 runs of
    `bench.py --profile-run --prefill`: a --kernel-trace folder, then --pmc
    folders (matrix-core busy cycles with GRBM_GUI_ACTIVE, instruction mix,
    the LDS bank-conflict counter on its own, FETCH_SIZE, WRITE_SIZE).
    FETCH_SIZE and WRITE_SIZE are scaled by what they read for the cold
    streaming read and the fill of PROBE_BYTES in the same run."""
    import csv
    import glob
    import workloads as wl
    import ar_image_generation_amd as da
    cfg = wl.PREFILL_CONFIGS["prefill_b2"]
    trace_dir, pmc_dirs = args.summarize[0], args.summarize[1:]

    def rows(d, suffix):
        out = []
        for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    tr = [r for r in rows(trace_dir, "kernel_trace.csv") if is_prefill_kernel(r["Kernel_Name"])]
    durs = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr)
    avg = sum(durs) / len(durs) if durs else float("nan")

    def per_dispatch(d, match):
        acc = {}
        for r in rows(d, "counter_collection.csv"):
            if not match(r["Kernel_Name"]):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        names = sorted({k[1] for k in acc})
        disp = sorted({k[0] for k in acc})
        return {nm: sum(acc[(dd, nm)] for dd in disp if (dd, nm) in acc) / max(1, len(disp))
                for nm in names}

    counters, dirs_of = {}, {}
    for d in pmc_dirs:
        for k, v in per_dispatch(d, is_prefill_kernel).items():
            counters[k] = v
            dirs_of[k] = d
    probe = {}
    for d in pmc_dirs:
        probe.update(per_dispatch(d, lambda k: "read_probe_kernel" in k))
    # the probe buffer's fill: the largest int32 fill kernel of the run
    fill = {}
    for d in pmc_dirs:
        for r in rows(d, "counter_collection.csv"):
            if "FillFunctor<int>" in r["Kernel_Name"]:
                nm = r["Counter_Name"]
                acc = fill.setdefault(nm, {})
                acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    fill = {nm: max(v.values()) for nm, v in fill.items()}
    n_xcd, n_simd = 8, 1024
    util = None
    if counters.get("GRBM_GUI_ACTIVE") and counters.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        cycles = counters["GRBM_GUI_ACTIVE"] / n_xcd          # per-XCD counter, summed over XCDs
        util = counters["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * cycles)
    m = da.mask(cfg.mode, cfg.W, cfg.B, cfg.G)
    kept = sum(da.keep_count(m, i, cfg.P) for i in range(cfg.n)) * cfg.batch * cfg.heads
    flops = 4.0 * cfg.hd * kept
    bytes_ = 4 * cfg.batch * cfg.heads * cfg.n * cfg.hd * 2
    extra = []
    if counters.get("SQ_INSTS_MFMA"):
        # v_mfma_f32_16x16x32_bf16: 16 * 16 * 32 multiply-adds
        executed = counters["SQ_INSTS_MFMA"] * 2 * 16 * 16 * 32
        extra.append(f"executed_mfma_GFLOP = {executed / 1e9:.3f} ({executed / flops:.2f} x algorithmic)")
    if counters.get("FETCH_SIZE") and probe.get("FETCH_SIZE"):
        fscale = (PROBE_BYTES / 1024.0) / probe["FETCH_SIZE"]
        extra.append(f"fetch_scale = {fscale:.4f} (cold read of {PROBE_BYTES} bytes)")
        hbm = counters["FETCH_SIZE"] * fscale * 1024
        if counters.get("WRITE_SIZE") and fill.get("WRITE_SIZE"):
            wscale = (PROBE_BYTES / 1024.0) / fill["WRITE_SIZE"]
            extra.append(f"write_scale = {wscale:.4f} (fill of {PROBE_BYTES} bytes)")
            hbm += counters["WRITE_SIZE"] * wscale * 1024
        extra.append(f"hbm_bytes_per_launch = {hbm:.6g} ({hbm / bytes_:.3f} x Q, K, V, O once)")
    cmd = f"python3 bench.py --profile-run --prefill --steps {args.steps} --warmup {args.warmup}"
    lines = [
        f"# rocprofv3 summary: band prefill kernel, workload {cfg.name}",
        f"# (batch {cfg.batch} x {cfg.heads} heads x {cfg.n} tokens, head_dim {cfg.hd}, bf16; causal and "
        f"prompt {cfg.P} + row-diagonal W={cfg.W} B={cfg.B} G={cfg.G})",
        "# commands (repo root, TMPDIR=/tmp):",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} -o run -- {cmd}",
    ]
    for d in pmc_dirs:
        names = " ".join(sorted(k for k in counters if dirs_of[k] == d))
        lines.append(f"#   rocprofv3 --pmc {names} -f csv -d {d} -o run -- {cmd}")
    lines += [
        f"#   python3 bench.py --summarize {trace_dir} {' '.join(pmc_dirs)} --prefill",
        "# mfma_utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)",
        f"kernel = {tr[0]['Kernel_Name'] if tr else '?'}",
        f"dispatches = {len(durs)}",
        f"avg_duration_us = {avg / 1e3:.3f}",
        f"median_duration_us = {durs[len(durs) // 2] / 1e3 if durs else float('nan'):.3f}",
        f"algorithmic_GFLOP = {flops / 1e9:.3f}",
        f"achieved_TFLOPs_from_avg = {flops / avg / 1e3 if durs else float('nan'):.2f}",
        f"hbm_bytes_QKVO = {bytes_}",
        f"mfma_utilisation = {util}",
    ] + extra + [f"{k} = {v:.6g}" for k, v in sorted(counters.items())]
    out = os.path.join(ROOT, "profiles", f"prefill_{cfg.name}.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="paged_b128",
                    help="headline decode workload (default: the largest, paged_b128)")
    ap.add_argument("--split", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip everything but the headline step, its dense run and the probe")
    ap.add_argument("--profile-run", action="store_true",
                    help="run only the timed decode launches and one probe (for rocprofv3)")
    ap.add_argument("--prefill", action="store_true",
                    help="with --profile-run / --summarize: the band prefill kernel")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="write the profiles/ summary from rocprofv3 output folders: decode "
                         "TRACE_DIR FETCH_DIR WRITE_DIR; with --prefill TRACE_DIR PMC_DIR...")
    args = ap.parse_args()
    if args.summarize:
        if args.prefill:
            summarize_prefill(args)
        elif len(args.summarize) != 3:
            ap.error("decode --summarize takes TRACE_DIR FETCH_DIR WRITE_DIR")
        else:
            summarize(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path is data-parallel over requests "
              "and heads with no exchange, so a GPU's throughput is its share of the batch; "
              "multi-GPU runs are not part of this benchmark. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.profile_run:
        profile_run(args)
        return

    import torch
    import workloads as wl
    import ar_image_generation_amd as da
    da.load()
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device: {props.name} {getattr(props, 'gcnArchName', '')} "
        f"CUs={props.multi_processor_count}")

    cfg = wl.CONFIGS[args.workload]
    # the batch laid out as the serving layer would: queries in the slots
    # da_decode_schedule gives them (the given order is timed further down)
    b = DecodeBench(cfg, split=args.split, order="balanced")
    passes = burn_in([b.k, b.v], 1.0)
    mode = cfg.modes[0]
    b.burn(mode, 0.3)
    log(f"[bench] burn-in: {passes} streaming passes over the cache copies, then 0.3 s of steps")
    K, W = args.steps, args.warmup
    # the step: keep-set build and attention in one launch (lists written too)
    us_step = b.time_graph(mode, K, W, path="fused")
    us_step_warm = b.time_graph(mode, K, W, rotate=False, path="fused")
    # the same step as two launches, and its decode kernel alone
    us_step_l = b.time_graph(mode, K, W, path="lists")
    us_step_a = b.time_graph(mode, K, W, path="append")
    us_dec = b.time_graph(mode, K, W, path="decode")
    us_step_d = b.time_graph(da.DENSE, K, W, path="fused")
    us_dec_d = b.time_graph(da.DENSE, K, W, path="decode")
    us_eager = b.time_eager(mode, K, W)
    log(f"[bench] {cfg.name} sparse: fused step {us_step:.2f} us cold / {us_step_warm:.2f} us warm; "
        f"with KV append {us_step_a:.2f} us; "
        f"list path {us_step_l:.2f} us/step (decode kernel {us_dec:.2f} us), {us_eager:.2f} us/step "
        f"eager; dense fused {us_step_d:.2f} us/step, dense decode {us_dec_d:.2f} us")

    kept = b.kept_bytes(mode)
    achieved = kept / (us_step * 1e-6) / 1e9       # the fused kernel is the whole step
    probe_us, probe_grid = attainable_read(kept, K, W)
    log(f"[bench] attainable: a streaming read of the same {kept / 1e6:.1f} MB takes {probe_us:.2f} us "
        f"cold ({kept / probe_us / 1e3:.0f} GB/s, grid/loads {probe_grid})")
    gather_us, gather_shape = b.gather_us(mode, K, W)
    log(f"[bench] attainable for the access pattern: a gather of exactly the kept rows takes {gather_us:.2f} us "
        f"cold ({kept / gather_us / 1e3:.0f} GB/s, grid/loads {gather_shape})")
    value = b.n_q / (us_step * 1e-6)
    traffic = traffic_from_profile(cfg.name)

    sweep = mask_sweep(b, K, W) if not args.no_extra else None
    per_head = per_head_run(b, K, W) if not args.no_extra else None
    if per_head:
        log(f"[bench] per-head windows {per_head['head_W'][:4]}...: {per_head['us_per_step']:.2f} us, "
            f"{per_head['read_MB']:.1f} MB read, {per_head['read_GBps']:.0f} GB/s")

    # the same batch in the order it was generated (no scheduling)
    gb = DecodeBench(cfg, split=args.split, order="given")
    burn_in([gb.k, gb.v], 0.3)
    gb.burn(mode, 0.3)
    us_given = gb.time_graph(mode, K, W, path="fused")
    given_order = {"us_per_step": round(us_given, 2), "tokens_per_s": round(gb.n_q / (us_given * 1e-6), 1),
                   "kept_GBps": round(kept / (us_given * 1e-6) / 1e9, 1),
                   "frac_hbm_peak": round(kept / (us_given * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    log(f"[bench] {cfg.name} in the generated batch order: fused {us_given:.2f} us/step")
    del gb
    torch.cuda.empty_cache()

    # keep-set-aware KV residency: the same step through a ring block table
    residency = {}
    if not args.no_extra:
        b.decode_masked(mode, 0)
        torch.cuda.synchronize()
        ref_out = b.out.clone()
        for name in ("llamagen_b16", "paged_b128"):
            c = wl.CONFIGS[name]
            rb = DecodeBench(c, ring=True, order="balanced" if name == cfg.name else "given")
            md = c.modes[0]
            st = rb.time_graph(md, K, W, path="fused")
            total, full = rb.ring_pages
            rec = {"mode": wl.MODE_NAMES[md], "pages_full": full, "pages_ring": total,
                   "kv_bytes_ratio": round(total / full, 4), "us_per_step": round(st, 2),
                   "kept_GBps": round(rb.kept_bytes(md) / (st * 1e-6) / 1e9, 1)}
            if name == cfg.name:
                rb.decode_masked(md, 0)
                torch.cuda.synchronize()
                rec["output_equals_full_cache"] = bool(torch.equal(rb.out, ref_out))
            residency[name] = rec
            log(f"[bench] {name} ring cache: {total} of {full} pages ({total / full:.3f}), "
                f"fused step {st:.2f} us")
            del rb
            torch.cuda.empty_cache()
        # the large batch outnumbers the resident workgroups, so it is timed
        # in its generated order and compared with the full-cache batch in
        # its generated order
        budget = kv_budget_run(K, W, order="given")
        if cfg.name == "paged_b128":
            budget["full_cache_us_per_step"] = round(us_given, 2)
            budget["full_cache_tokens_per_s"] = round(b.n_q / (us_given * 1e-6), 1)
            budget["tokens_per_s_ratio"] = round(budget["tokens_per_s"] / budget["full_cache_tokens_per_s"], 3)
            budget["full_cache_balanced_tokens_per_s"] = round(b.n_q / (us_step * 1e-6), 1)
        residency["same_kv_budget"] = budget
        log(f"[bench] same KV budget: {budget['ring_requests']} requests through ring tables vs "
            f"{budget['full_cache_requests']} on full caches: {budget['us_per_step']:.2f} us/step, "
            f"{budget['tokens_per_s']:.0f} tokens/s")

    # the headline workload's other sparse mode(s)
    other_modes = {}
    for md in cfg.modes[1:]:
        if md == da.DENSE:
            continue
        st = b.time_graph(md, K, W, path="fused")
        gb = b.kept_bytes(md) / (st * 1e-6) / 1e9
        other_modes[wl.MODE_NAMES[md]] = {
            "us_per_step": round(st, 2), "tokens_per_s": round(b.n_q / (st * 1e-6), 1),
            "kept_MB": round(b.kept_bytes(md) / 1e6, 2), "kept_GBps": round(gb, 1),
            "frac_hbm_peak": round(gb / HBM_PEAK_GBPS, 4),
            "speedup_vs_dense": round(us_step_d / st, 3)}
        log(f"[bench] {cfg.name} {wl.MODE_NAMES[md]}: fused {st:.2f} us/step ({gb:.0f} GB/s)")

    extra = {}
    if not args.no_extra:
        for name in [n for n in ("llamagen_b16", "gqa_b64", "paged_b128") if n != cfg.name]:
            c = wl.CONFIGS[name]
            eb = DecodeBench(c)
            burn_in([eb.k, eb.v], 0.3)
            eb.burn(c.modes[0], 0.2)
            rec = {}
            for md in list(dict.fromkeys(list(c.modes) + [da.DENSE])):
                st = eb.time_graph(md, K, W, path="fused")
                sl = eb.time_graph(md, K, W, path="lists")
                dk = eb.time_graph(md, K, W, path="decode")
                gbps = eb.kept_bytes(md) / (st * 1e-6) / 1e9
                rec[wl.MODE_NAMES[md]] = {
                    "us_per_step": round(st, 2), "list_path_us_per_step": round(sl, 2),
                    "list_decode_us": round(dk, 2),
                    "tokens_per_s": round(eb.n_q / (st * 1e-6), 1),
                    "kept_MB": round(eb.kept_bytes(md) / 1e6, 2),
                    "kept_GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
                log(f"[bench] {name} {wl.MODE_NAMES[md]}: fused {st:.2f} us/step ({gbps:.0f} GB/s), "
                    f"list path {sl:.2f} us/step, decode kernel {dk:.2f} us")
            dense_us = rec["dense"]["us_per_step"]
            for md in c.modes:
                r = rec[wl.MODE_NAMES[md]]
                r["speedup_vs_dense"] = round(dense_us / r["us_per_step"], 3)
            pu, _ = attainable_read(eb.kept_bytes(c.modes[0]), K, W)
            rec["attainable"] = {"us": round(pu, 3),
                                 "GBps": round(eb.kept_bytes(c.modes[0]) / pu / 1e3, 1),
                                 "step_frac_of_attainable": round(
                                     pu / rec[wl.MODE_NAMES[c.modes[0]]]["us_per_step"], 4)}
            gu, gs = eb.gather_us(c.modes[0], K, W)
            rec["attainable_gather"] = {"us": round(gu, 3), "grid_loads": list(gs),
                                        "GBps": round(eb.kept_bytes(c.modes[0]) / gu / 1e3, 1),
                                        "step_frac_of_attainable": round(
                                            gu / rec[wl.MODE_NAMES[c.modes[0]]]["us_per_step"], 4)}
            extra[name] = rec
            del eb
            torch.cuda.empty_cache()

    prefill = None
    if not args.no_extra:
        pb = PrefillBench(wl.PREFILL_CONFIGS["prefill_b2"])
        prefill = pb.report(max(8, K // 4), 2)
        del pb
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(cfg)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded correlated-field K/V, random positions; paged caches use a "
                "seeded random block table)",
        "config": {"workload": cfg.name, "requests": cfg.n_seq, "q_heads": cfg.hq,
                   "kv_heads": cfg.hkv, "head_dim": cfg.hd, "prompt": list(cfg.prompt),
                   "page_size": cfg.page_size,
                   "grid": cfg.G, "W": cfg.W, "B": cfg.B, "mode": wl.MODE_NAMES[mode],
                   "split": b.split, "dense_split": cfg.dense_split, "cache_copies": b.n_copies,
                   "step": "sparse_decode_attn_masked (keep-set build, lists written, and "
                           "attention in one launch), HIP graph of K steps",
                   "batch_order": "balanced: queries in the batch slots da_decode_schedule gives "
                                  "them from their host-side keep-set sizes (given_order: as generated)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "attainable": {"what": "streaming-read probe (nontemporal 16-byte loads) of the kept byte "
                               "count, cold, best (grid, loads in flight) shape",
                       "bytes": kept, "us": round(probe_us, 3), "grid_loads": list(probe_grid),
                       "GBps": round(kept / probe_us / 1e3, 1),
                       "frac_of_peak": round(kept / probe_us / 1e3 / HBM_PEAK_GBPS, 4),
                       "step_frac_of_attainable": round(probe_us / us_step, 4)},
        "attainable_gather": {"what": "gather probe: exactly the kept K/V rows of the step at byte offsets "
                                      "resolved beforehand (no address chain, no arithmetic); cold, best "
                                      "(grid, loads in flight) shape",
                              "us": round(gather_us, 3), "grid_loads": list(gather_shape),
                              "GBps": round(kept / gather_us / 1e3, 1),
                              "frac_of_peak": round(kept / gather_us / 1e3 / HBM_PEAK_GBPS, 4),
                              "step_frac_of_attainable": round(gather_us / us_step, 4)},
        "cpu_baseline": cpu,
        "device": f"{torch.cuda.get_device_properties(0).name} "
                  f"{getattr(torch.cuda.get_device_properties(0), 'gcnArchName', '')}".strip(),
        "kept_MB_per_step": round(kept / 1e6, 3),
        "list_path": {"us_per_step": round(us_step_l, 2),
                      "tokens_per_s": round(b.n_q / (us_step_l * 1e-6), 1),
                      "decode_us": round(us_dec, 3),
                      "decode_kept_GBps": round(kept / (us_dec * 1e-6) / 1e9, 1),
                      "eager_us_per_step": round(us_eager, 2)},
        "with_kv_append": {"us_per_step": round(us_step_a, 2),
                           "tokens_per_s": round(b.n_q / (us_step_a * 1e-6), 1)},
        "warm": {"us_per_step": round(us_step_warm, 2),
                 "kept_GBps": round(kept / (us_step_warm * 1e-6) / 1e9, 1)},
        "given_order": given_order,
        "dense": {"us_per_step": round(us_step_d, 2), "decode_us": round(us_dec_d, 2),
                  "kept_MB": round(b.kept_bytes(da.DENSE) / 1e6, 2),
                  "speedup_step": round(us_step_d / us_step, 3),
                  "speedup_decode": round(us_dec_d / us_dec, 3)},
        "other_modes": other_modes,
        "extra": extra,
        "kv_residency": residency,
        "mask_sweep": sweep,
        "per_head_masks": per_head,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

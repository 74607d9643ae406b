"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and its host-side paths (sizing, argument checks) behave as documented.
No kernel is launched here."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import ar_image_generation_amd as da
from ar_image_generation_amd import _native
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(da_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = da.load()
    names = declared_symbols()
    assert {"da_keepset_build", "da_sparse_decode_attn", "da_keep_count"} <= names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _native.SIGNATURES, n


def test_version_and_error_text():
    assert da.load().da_version() >= 100
    with pytest.raises(da.DiagAttnError, match="mode 7"):
        da.keep_count(da.mask(7, 1, 1, 1), 0, 0)


@pytest.mark.parametrize("mode", [O.DENSE, O.BAND, O.ROWDIAG])
def test_keep_count_matches_oracle(mode):
    rng = np.random.default_rng(11)
    for _ in range(300):
        P, W, B, G = (int(rng.integers(0, 40)), int(rng.integers(0, 70)),
                      int(rng.integers(0, 6)), int(rng.integers(1, 20)))
        causal = bool(rng.integers(0, 2))
        n_keys = int(rng.integers(1, 200))
        i = int(rng.integers(0, n_keys if not causal else 300))
        m = da.mask(mode, W, B, G, causal)
        want = len(O.keepset(i, n_keys if not causal else None, P=P, W=W, B=B, G=G,
                             mode=mode, causal=causal))
        assert da.keep_count(m, i, P, n_keys) == want, (mode, P, W, B, G, causal, i, n_keys)
        assert da.keep_cap(m, i, P, n_keys) >= want


def test_keep_cap_bounds_the_workloads():
    for (P, W, B, G, mode, maxpos) in [(16, 64, 2, 16, O.ROWDIAG, 271), (120, 96, 2, 32, O.ROWDIAG, 1143),
                                       (300, 96, 2, 48, O.BAND, 2603), (256, 256, 3, 64, O.DENSE, 4351)]:
        m = da.mask(mode, W, B, G)
        cap = da.keep_cap(m, maxpos, P)
        for i in range(0, maxpos + 1, 7):
            assert da.keep_count(m, i, P) <= cap


def test_argument_errors_are_reported_before_launch():
    lib = da.load()
    m = da.mask(O.ROWDIAG, 4, 1, 3)
    dummy = ctypes.c_void_p(16)   # never dereferenced: checks fail first
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 1, None, 0, dummy, dummy, 0, None, None, 0, None, 0, None, None)
    assert rc == -1 and "cap" in _native.last_error()
    rc = lib.da_keepset_build(m, -1, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 0, None, 0, None, None)
    assert rc == -1
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 1, None, 4, dummy, dummy, 2, None, dummy, 0, None, 0, None, None)
    assert rc == -1 and "both" in _native.last_error()
    bad = da.mask(O.BAND, -1, 1, 3)
    assert lib.da_keepset_build(bad, 1, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 0, None, 0, None, None) == -1
    nc = da.mask(O.BAND, 1, 1, 3, causal=False)
    assert lib.da_keepset_build(nc, 1, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 0, None, 0, None, None) == -1
    # zero queries is a valid no-op
    assert lib.da_keepset_build(m, 0, None, None, 0, 1, None, 4, None, None, 0, None, None, 0, None, 0, None, None) == 0
    # tile list: both pointers or neither, tile >= 1, cap_tiles >= 0
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 8, dummy, 4, None, None)
    assert rc == -1 and "both" in _native.last_error()
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 0, dummy, 4, dummy, None)
    assert rc == -1 and "tile" in _native.last_error()
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 1, None, 4, dummy, dummy, 0, None, None, 8, dummy, -1, dummy, None)
    assert rc == -1 and "cap_tiles" in _native.last_error()
    # per-head lists: n_heads >= 1, n_q * n_heads within int32, head_wb aligned
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 0, dummy, 4, dummy, dummy, 0, None, None, 0, None, 0, None, None)
    assert rc == -1 and "n_heads" in _native.last_error()
    rc = lib.da_keepset_build(m, 1 << 20, dummy, dummy, 0, 1 << 12, dummy, 4, dummy, dummy, 0, None, None, 0, None, 0,
                              None, None)
    assert rc == -1 and "INT32_MAX" in _native.last_error()
    rc = lib.da_keepset_build(m, 4, dummy, dummy, 0, 2, ctypes.c_void_p(18), 4, dummy, dummy, 0, None, None, 0, None, 0,
                              None, None)
    assert rc == -1 and "head_wb" in _native.last_error()

    kv = _native.DaKvCache(16, 16, 0, 0, 0, 0, 0, None, 1, 1, 8)

    def dec(dtype=1, n_q=1, hq=8, hkv=2, hd=128, cap=64, split=64, ws=None, wsb=0, kvd=kv, q=dummy, lh=1):
        return lib.da_sparse_decode_attn(q, dtype, n_q, hq, hkv, hd, 0.1, kvd, dummy, dummy,
                                         dummy, cap, lh, split, dummy, None, ws, wsb, None)
    assert dec(hq=6, hkv=4) == -1
    assert dec(hd=96) == -2
    assert dec(dtype=3) == -2
    assert dec(hq=48, hkv=3) == -2          # group 16
    assert dec(split=0) == -1
    assert dec(split=5000) == -2
    assert dec(cap=200, split=64) == -3     # needs a workspace
    assert "workspace" in _native.last_error()
    paged = _native.DaKvCache(16, 16, 0, 0, 0, 12, 4, 16, 1, 4, 48)
    assert dec(kvd=paged) == -1 and "power of two" in _native.last_error()
    paged = _native.DaKvCache(16, 16, 0, 0, 0, 16, 4, 16, 1, 4, 65)
    assert dec(kvd=paged) == -1 and "max_len" in _native.last_error()
    assert dec(kvd=_native.DaKvCache(16, 16, 0, 0, 0, 0, 0, None, 1, 1, 0)) == -1
    assert dec(kvd=_native.DaKvCache(16, 16, 0, 0, 0, 0, 0, None, 3, 2, 8)) == -1
    assert dec(q=ctypes.c_void_p(8)) == -1   # misaligned q
    assert dec(lh=3) == -1 and "list_heads" in _native.last_error()   # lists: one a query or one a kv head
    assert dec(lh=2, n_q=0) == 0

    def dec_m(mk=m, n_q=1, hq=8, hkv=2, hd=128, cap=64, split=64, pos=dummy, count=None, idx=None,
              k_new=None, v_new=None, head_wb=None):
        return lib.da_sparse_decode_attn_masked(mk, dummy, 1, n_q, hq, hkv, hd, 0.1, kv, dummy, pos,
                                                dummy, head_wb, k_new, v_new, cap, split, count, idx,
                                                dummy, None, None, 0, None)
    assert dec_m(mk=bad) == -1
    assert dec_m(mk=nc) == -2 and "causal" in _native.last_error()
    assert dec_m(pos=None) == -1 and "pos" in _native.last_error()
    assert dec_m(count=dummy) == -1 and "both" in _native.last_error()
    assert dec_m(hd=96) == -2
    assert dec_m(cap=200, split=64) == -3
    assert dec_m(k_new=dummy) == -1 and "k_new" in _native.last_error()
    assert dec_m(head_wb=dummy, count=dummy, idx=dummy) == -1 and "per-head" in _native.last_error()
    assert dec_m(k_new=ctypes.c_void_p(8), v_new=dummy) == -1      # misaligned
    assert dec_m(n_q=0, pos=None) == 0     # nothing to do, nothing read


def test_prefill_limits_are_reported_before_launch():
    lib = da.load()
    dummy = ctypes.c_void_p(256)   # never dereferenced: checks fail first
    strides = (ctypes.c_int64 * 12)(*([128 * 1024, 128 * 1024, 128] * 4))

    def pf(mk, n=1024, hd=128, dtype=1):
        return lib.da_band_prefill_attn(mk, dtype, 1, 2, 2, n, hd, dummy, dummy, dummy, dummy,
                                        strides, dummy, dummy, 1 << 30, 0.1, None, None)
    rd = da.mask(O.ROWDIAG, 64, 1, 32)
    assert pf(rd, n=70000) == -2 and "65536" in _native.last_error()
    assert pf(da.mask(O.ROWDIAG, 64, 1, 2048)) == -2 and "G <=" in _native.last_error()
    assert pf(da.mask(O.BAND, 64, 1, 2048), n=0) == 0          # G only matters for ROWDIAG
    assert pf(rd, hd=96) == -2
    assert pf(rd, dtype=0) == -2
    assert pf(da.mask(O.ROWDIAG, 64, 1, 32, causal=False)) == -2
    assert pf(rd, n=0) == 0
    big = (ctypes.c_int64 * 12)(*([128 * 1024, 128 * 1024, 128] * 4))
    big[5] = 34088000                  # k position stride: a 64-row tile spans > 4 GiB
    assert lib.da_band_prefill_attn(rd, 1, 1, 2, 2, 1024, 128, dummy, dummy, dummy, dummy, big,
                                    dummy, dummy, 1 << 30, 0.1, None, None) == -2
    assert "stride too large" in _native.last_error()
    # a tile-list buffer smaller than the sizes need is refused
    need = lib.da_prefill_tiles_bytes(1, 1024)
    assert lib.da_band_prefill_attn(rd, 1, 1, 2, 2, 1024, 128, dummy, dummy, dummy, dummy, strides,
                                    dummy, dummy, need - 1, 0.1, None, None) == -3
    assert "tiles buffer" in _native.last_error()
    # the scale must be positive and finite (masked scores are -inf before it)
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        assert lib.da_band_prefill_attn(rd, 1, 1, 2, 2, 1024, 128, dummy, dummy, dummy, dummy, strides,
                                        dummy, dummy, 1 << 30, bad, None, None) == -1
        assert "scale" in _native.last_error()


def test_decode_workspace_size():
    assert da.decode_workspace_bytes(4, 8, 128, 64, 64) == 0
    b = da.decode_workspace_bytes(4, 8, 128, 200, 64)
    rows = 4 * 8 * 4
    assert b >= rows * (128 + 2) * 4


def test_product_path_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", "/nonexistent/libdiagattn.so")
    with pytest.raises(RuntimeError, match="missing"):
        _native.load()


def test_gather_probe_arguments_are_checked_before_launch():
    lib = da.load()
    dummy = ctypes.c_void_p(256)   # never dereferenced: checks fail first

    def gp(row=256, n=10, span=1 << 20, grid=64, loads=2, k=dummy):
        return lib.da_gather_read_probe(k, dummy, dummy, n, row, span, dummy, grid, loads, None)
    assert gp(row=192) == -2 and "row" in _native.last_error()
    assert gp(n=-1) == -1
    assert gp(grid=0) == -1
    assert gp(loads=3) == -1 and "loads_in_flight" in _native.last_error()
    assert gp(span=100) == -1 and "span" in _native.last_error()
    assert gp(k=ctypes.c_void_p(264)) == -1 and "aligned" in _native.last_error()
    assert gp(k=None) == -1
    assert gp(n=0) == 0                  # nothing to read

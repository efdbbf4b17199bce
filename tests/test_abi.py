"""The C-ABI library loads, exports every symbol include/fathom.h declares, and
validates arguments on the host (no GPU needed: every call here fails
validation before any HIP call)."""

import ctypes
import os
import re

import pytest

from oracle import fathom_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "fathom.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_top_query_amd import build, fathom
    if not os.path.exists(fathom.LIB_PATH):
        build.build()
    return fathom.load()


def test_header_declares_the_entry_points():
    names = header_functions()
    for fn in ("pack_bitplanes", "allocate_depths", "scan_topk", "fathom_workspace_bytes",
               "fathom_scan_scores", "fathom_last_error", "fathom_record_bytes", "attend_topk",
               "fathom_attend_workspace_bytes", "pack_blocks", "scan_topk_append"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_record_geometry_matches_layout_definition(lib):
    for n in (0, 1, 127, 128, 129, 1000, 1024, 4096, 131072, 262144, 1 << 20, 3 * 1024 + 300):
        _, _, _, r = O.record_layout(n)
        assert lib.fathom_record_bytes(n) == r
        for t in range(5):
            assert lib.fathom_prefix_bytes(n, t) == O.prefix_bytes(n, t)


def test_workspace_bytes_monotone(lib):
    a = lib.fathom_workspace_bytes(32, 8, 1 << 20, 128, 2048, 0)
    b = lib.fathom_workspace_bytes(32, 8, 1 << 17, 128, 2048, 0)
    assert a > b > 0
    assert a >= 32 * (1 << 20) * 4       # holds the fp32 scores of every head
    staged = lib.fathom_workspace_bytes(32, 8, 1 << 20, 128, 2048, 2)
    r = O.record_layout(1 << 20)[3]
    # plus a ring of two KV heads' records (not a mirror of all eight)
    assert 2 * 128 * r <= staged - a < 2 * 128 * r + 256
    assert lib.fathom_workspace_bytes(4, 1, 1 << 20, 128, 2048, 2) - lib.fathom_workspace_bytes(
        4, 1, 1 << 20, 128, 2048, 0) < 128 * r + 256                 # one KV head: one slot
    assert lib.fathom_workspace_bytes(32, 8, 0, 128, 0, 0) == 0


def _err(lib):
    return lib.fathom_last_error().decode()


def test_host_validation_errors(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: validation fails first
    # pack: bad d / h_kv
    assert lib.pack_bitplanes(fake, 1, 128, 0, fake, None, None) == -2
    assert "d=0" in _err(lib)
    assert lib.pack_bitplanes(fake, 0, 128, 4, fake, None, None) == -2
    assert lib.pack_bitplanes(None, 1, 128, 4, fake, None, None) == -1
    # allocate: budget, mode, group size
    assert lib.allocate_depths(fake, fake, 4, 1, 8, 0, 33, fake, fake, None, None) == -3
    assert lib.allocate_depths(fake, fake, 4, 1, 8, 1, 6, fake, fake, None, None) == -3
    assert lib.allocate_depths(fake, fake, 4, 1, 8, 7, 6, fake, fake, None, None) == -1
    assert lib.allocate_depths(fake, fake, 3, 1, 8, 0, 6, fake, fake, None, None) == -2
    assert lib.allocate_depths(fake, fake, 6, 4, 8, 0, 6, fake, fake, None, None) == -2
    assert lib.allocate_depths(fake, fake, 4, 1, 300, 0, 6, fake, fake, None, None) == -2
    # scan: shape checks come before any pointer query
    assert lib.scan_topk(fake, 0, fake, fake, fake, 4, 3, 128, 8, 4, fake, None, fake, 1 << 20, None) == -2
    assert lib.scan_topk(fake, 0, fake, fake, fake, 4, 1, -1, 8, 4, fake, None, fake, 1 << 20, None) == -2
    # at most 65535 query heads (G = 16 over 4096 KV heads is one too many)
    assert lib.scan_topk(fake, 0, fake, fake, fake, 65536, 4096, 128, 8, 4, fake, None, fake, 1 << 20, None) == -2
    assert "65535" in _err(lib)
    assert lib.allocate_depths(fake, fake, 65536, 4096, 8, 0, 6, fake, fake, None, None) == -2
    assert lib.fathom_scan_scores(fake, 0, None, fake, fake, 4, 1, 128, 8, fake, 128, None, 0, None) == -1


def test_noalloc_validation(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    assert lib.fathom_noalloc_scratch_bytes() == 32 << 20
    # shapes whose workspace exceeds the fixed scratch are refused before any HIP call
    assert lib.scan_topk_noalloc(fake, 0, fake, fake, fake, 32, 8, 1 << 20, 128, 2048, fake, None, None) == -5
    assert "scratch" in _err(lib)
    assert lib.scan_topk_noalloc(fake, 2, fake, fake, fake, 4, 1, 4096, 128, 64, fake, None, None) == -7
    assert lib.scan_topk_noalloc(fake, 0, fake, fake, fake, 6, 4, 4096, 128, 64, fake, None, None) == -2
    # 32 query heads of 131072 keys fit
    assert lib.fathom_workspace_bytes(32, 8, 1 << 17, 128, 2048, 0) <= lib.fathom_noalloc_scratch_bytes()


def test_attend_workspace_and_validation(lib):
    P = ctypes.c_void_p
    f = ctypes.c_float
    fake = P(0x1000)
    # one split of 256 keys per query head at d = 128: (d + 2) floats + a flag word, 256-byte padded
    assert lib.fathom_attend_workspace_bytes(32, 128, 256) == 32 * 130 * 4 + 256   # 16640 is 65 x 256
    assert lib.fathom_attend_workspace_bytes(32, 128, 2048) > lib.fathom_attend_workspace_bytes(32, 128, 256)
    assert lib.fathom_attend_workspace_bytes(0, 128, 64) == 0
    ws = 1 << 20

    def call(kc=fake, vc=fake, res=0, q=fake, idx=fake, h_q=4, h_kv=1, n=1000, d=128, k=64, scale=0.1,
             out=fake, wsp=fake, wsb=ws):
        return lib.attend_topk(kc, vc, res, q, idx, h_q, h_kv, n, d, k, f(scale), out, None, None, wsp, wsb, None)
    assert call(d=100) == -2 and "d in" in _err(lib)
    assert call(d=512) == -2
    assert call(h_q=6, h_kv=4) == -2
    assert call(k=0) == -2
    assert call(n=0) == -2
    assert call(scale=float("nan")) == -1
    assert call(kc=None) == -1
    assert call(out=None) == -1
    assert call(q=P(0x1004)) == -1 and "aligned" in _err(lib)
    assert call(res=2) == -7
    assert call(wsb=16) == -5


def test_append_validation(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    # pack_blocks: the range must lie inside the capacity's blocks (5000 keys -> 40 blocks)
    assert lib.pack_blocks(fake, 2, 5000, 39, 2, 64, fake, None, None) == -2
    assert lib.pack_blocks(fake, 2, 5000, -1, 1, 64, fake, None, None) == -2
    assert lib.pack_blocks(fake, 2, 0, 0, 0, 64, fake, None, None) == -2
    assert lib.pack_blocks(None, 2, 5000, 0, 3, 64, fake, None, None) == -1
    assert lib.pack_blocks(fake, 2, 5000, 0, 3, 300, fake, None, None) == -2

    def app(n_cap=8192, n_sealed=4096, tail=fake, n_tail=10, k=64, res=0, h_q=8, h_kv=2, ws=1 << 30):
        return lib.scan_topk_append(fake, res, n_cap, n_sealed, tail, n_tail, fake, fake, fake, h_q, h_kv, 128, k,
                                    fake, None, fake, ws, None)
    assert app(n_sealed=4000) == -2 and "multiple of 128" in _err(lib)
    assert app(n_sealed=9000) == -2
    assert app(n_tail=-1) == -2
    assert app(k=4096 + 11) == -2
    assert app(res=2) == -7
    assert app(tail=None) == -1
    assert app(h_q=6, h_kv=4) == -2


def test_size_limits_keep_grids_valid(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    f = ctypes.c_float
    assert lib.pack_bitplanes(fake, 1, (1 << 30) + 1, 8, fake, None, None) == -2
    assert lib.pack_bitplanes(fake, 16, 1 << 30, 8, fake, None, None) == -2          # n * h_kv > 2^33
    assert lib.scan_topk(fake, 0, fake, fake, fake, 64, 16, 1 << 30, 8, 4, fake, None, fake, 1 << 20, None) == -2
    assert "2^33" in _err(lib)
    assert lib.scan_topk_append(fake, 0, 4096, 4096, fake, (1 << 20) + 1, fake, fake, fake, 4, 1, 128, 8, fake, None,
                                fake, 1 << 30, None) == -2
    # attention: h_q * ceil(k / 256) workgroups at most 2^23
    assert lib.attend_topk(fake, fake, 0, fake, fake, 65536, 1, 1 << 20, 128, 1 << 16, f(0.1), fake, None, None,
                           fake, 1 << 40, None) == -2


def test_binding_refuses_cpu_tensors(lib):
    import torch
    from sparse_attention_top_query_amd import fathom
    k = torch.zeros((1, 128, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        fathom.pack(k)
    with pytest.raises(TypeError):
        fathom.pack(k.double())


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "sparse_attention_top_query_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, f

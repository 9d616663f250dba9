"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/dsa.h declares, sizes workspaces, and rejects bad arguments before launching anything.
Rejected calls never touch device memory, so fake (never dereferenced) pointers are safe here."""
import ctypes
import os
import re

import pytest

import sparse_attention_15_amd as dsa
from sparse_attention_15_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libdsa.so not built")

FAKE = 0x7000_0000_0000   # 256-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"dsa_indexer_topk", "dsa_sparse_attn", "dsa_indexer_workspace_size",
            "dsa_sparse_attn_workspace_size", "dsa_last_error", "dsa_version"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)
    assert dsa.lib().dsa_version() == 4


def _layout(B=2, max_pages=4, max_len=256, num_pages=9, page=64):
    return L.Layout(FAKE, FAKE + 256, B, max_pages, page, num_pages, max_len)


def _ishape(T=1, H=64, D=128, K=64, dt=0):
    return L.IndexerShape(T, H, D, K, dt)


def _ashape(T=1, H=128, K=64, scale=0.05):
    return L.AttnShape(T, H, 576, 512, K, scale)


def test_workspace_sizes():
    lib = dsa.lib()
    ws = dsa.dsa_indexer_workspace_size(_layout(), _ishape())
    assert ws > 0 and ws % 256 == 0
    # bigger context -> bigger workspace; invalid shape -> 0
    assert dsa.dsa_indexer_workspace_size(_layout(max_pages=128, max_len=8192), _ishape()) > ws
    assert dsa.dsa_indexer_workspace_size(_layout(), _ishape(H=12)) == 0
    assert dsa.dsa_indexer_workspace_size(_layout(page=32), _ishape()) == 0
    assert lib.dsa_sparse_attn_workspace_size(ctypes.byref(_layout()), ctypes.byref(_ashape(K=2048))) > 0
    assert dsa.dsa_sparse_attn_workspace_size(_layout(), _ashape(H=100)) == 0


def _idx_call(q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, layout=None, shape=None, out=FAKE,
              ws=FAKE, wsb=1 << 40):
    lib = dsa.lib()
    layout = layout or _layout()
    shape = shape or _ishape()
    return lib.dsa_indexer_topk(q, qs, w, k, ks, ctypes.byref(layout), ctypes.byref(shape), out,
                                ws, wsb, None)


def _attn_call(q=FAKE, kv=FAKE, idx=FAKE, layout=None, shape=None, out=FAKE, lse=None, ws=FAKE,
               wsb=1 << 40):
    lib = dsa.lib()
    layout = layout or _layout()
    shape = shape or _ashape()
    return lib.dsa_sparse_attn(q, kv, idx, ctypes.byref(layout), ctypes.byref(shape), out, lse, ws,
                               wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(w=None), 1), (dict(k=None), 1), (dict(out=None), 1),
    (dict(q=FAKE + 8), 3), (dict(k=FAKE + 4), 3), (dict(w=FAKE + 2), 3),
    (dict(shape=_ishape(H=12)), 4), (dict(shape=_ishape(D=96)), 4), (dict(shape=_ishape(K=0)), 4),
    (dict(shape=_ishape(K=4096)), 4), (dict(shape=_ishape(T=0)), 2),
    (dict(shape=_ishape(dt=1)), 1),                       # fp8 without scales
    (dict(shape=_ishape(dt=2)), 1),                       # MXFP8 without scales
    (dict(shape=_ishape(dt=2), qs=FAKE, ks=FAKE + 4), 3),    # MXFP8 k scales need 16 bytes
    (dict(shape=_ishape(dt=3)), 4),                       # unknown dtype
    (dict(qs=FAKE, ks=FAKE), 2),                          # scales given for bf16
    (dict(layout=_layout(page=128)), 4), (dict(layout=_layout(B=0)), 2),
    (dict(layout=_layout(max_pages=2, max_len=256)), 2),  # table too short for max_len
    (dict(layout=_layout(max_len=0)), 2),                 # max_len < T
    (dict(ws=None), 5), (dict(wsb=16), 5), (dict(ws=FAKE + 64), 3),
])
def test_indexer_rejects(kw, status):
    assert _idx_call(**kw) == status
    assert dsa.lib().dsa_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(q=FAKE + 2), 3), (dict(out=FAKE + 8), 3), (dict(lse=FAKE + 2), 3),
    (dict(shape=_ashape(H=100)), 4), (dict(shape=_ashape(H=256)), 4),
    (dict(shape=L.AttnShape(1, 128, 512, 512, 64, 0.1)), 4),
    (dict(shape=_ashape(K=0)), 4), (dict(shape=_ashape(scale=0.0)), 2),
    (dict(shape=_ashape(scale=float("nan"))), 2),
    (dict(layout=_layout(num_pages=0)), 2),
    (dict(shape=_ashape(K=2048), ws=None), 5),
])
def test_attn_rejects(kw, status):
    assert _attn_call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(q=FAKE + 2), 3), (dict(lse=FAKE + 2), 3), (dict(shape=_ashape(H=100)), 4),
    (dict(layout=_layout(num_pages=0)), 2),
])
def test_attn_noalloc_rejects(kw, status):
    kw = {k: v for k, v in kw.items() if k not in ("ws", "wsb")}
    layout = kw.pop("layout", None) or _layout()
    shape = kw.pop("shape", None) or _ashape(K=2048)
    a = dict(q=FAKE, kv=FAKE, idx=FAKE, out=FAKE, lse=None)
    a.update(kw)
    st = dsa.lib().dsa_sparse_attn_noalloc(a["q"], a["kv"], a["idx"], ctypes.byref(layout),
                                           ctypes.byref(shape), a["out"], a["lse"], None)
    assert st == status
    assert dsa.lib().dsa_last_error().decode() != ""


def test_noalloc_scratch_covers_every_supported_attention_shape():
    """The static scratch of the no-alloc entry point holds the workspace of every shape the
    attention plan accepts (heads 16..128, K up to 2048, any row count)."""
    limit = 72 << 20
    text = open(HEADER).read()
    assert re.search(r"#define DSA_NOALLOC_SCRATCH_BYTES \(72u << 20\)", text)
    worst = 0
    for rows in list(range(1, 600)) + [1024, 4096, 8192]:
        for heads in range(16, 129, 16):
            for k in (2048, 2047, 1000, 256, 33):
                need = dsa.dsa_sparse_attn_workspace_size(_layout(B=rows, max_pages=4, max_len=256),
                                                          _ashape(H=heads, K=k))
                worst = max(worst, need)
    assert 0 < worst <= limit, worst


def test_quantisers_reject_grids_past_31_bits():
    lib = dsa.lib()
    assert lib.dsa_mxfp8_quantize(FAKE, 1 << 40, 32, FAKE, FAKE, None) == 2
    assert lib.dsa_fp8_quantize_heads(FAKE, 1 << 31, 128, FAKE, FAKE, None) == 2
    big = L.Layout(FAKE, FAKE + 256, 1 << 30, 1 << 14, 64, 9, 1 << 20)
    assert lib.dsa_indexer_cache_append(FAKE, ctypes.byref(big), 1 << 10, 4096, FAKE, FAKE, None) == 2
    assert lib.dsa_latent_cache_append_fp8(FAKE, ctypes.byref(big), 1 << 10, FAKE, FAKE, None) == 2


def test_fp8_heads_rejects():
    lib = dsa.lib()
    assert lib.dsa_fp8_quantize_heads(FAKE, 4, 96, FAKE, FAKE, None) == 4
    assert lib.dsa_fp8_quantize_heads(None, 4, 128, FAKE, FAKE, None) == 1
    assert lib.dsa_fp8_quantize_heads(FAKE + 8, 4, 128, FAKE, FAKE, None) == 3
    assert lib.dsa_fp8_quantize_heads(FAKE, -1, 128, FAKE, FAKE, None) == 2
    assert lib.dsa_fp8_quantize_heads(None, 0, 64, None, None, None) == 0


def test_latent_append_rejects():
    lib = dsa.lib()
    assert lib.dsa_latent_cache_append_fp8(None, ctypes.byref(_layout()), 1, FAKE, FAKE, None) == 1
    assert lib.dsa_latent_cache_append_fp8(FAKE, ctypes.byref(_layout()), 1, FAKE, FAKE + 4, None) == 3
    assert lib.dsa_latent_cache_append_fp8(FAKE, ctypes.byref(_layout()), 0, FAKE, FAKE, None) == 2
    assert lib.dsa_latent_cache_append_fp8(FAKE, ctypes.byref(_layout(B=0)), 1, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("kw,status", [
    (dict(kvs=None), 1), (dict(kv=None), 1), (dict(kvs=FAKE + 4), 3), (dict(kv=FAKE + 8), 3),
    (dict(shape=_ashape(H=100)), 4), (dict(shape=_ashape(K=2048), ws=None), 5),
])
def test_attn_fp8kv_rejects(kw, status):
    a = dict(q=FAKE, kv=FAKE, kvs=FAKE, idx=FAKE, shape=_ashape(), out=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    lib = dsa.lib()
    assert lib.dsa_sparse_attn_fp8kv(a["q"], a["kv"], a["kvs"], a["idx"], ctypes.byref(_layout()),
                                     ctypes.byref(a["shape"]), a["out"], None, a["ws"], a["wsb"], None) == status
    assert lib.dsa_last_error().decode() != ""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        L.lib()


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scales=None), 1),
    (dict(dim=48), 4), (dict(dim=0), 4), (dict(rows=-1), 2),
    (dict(x=FAKE + 8), 3), (dict(codes=FAKE + 4), 3),
])
def test_mxfp8_quantize_rejects(kw, status):
    a = dict(x=FAKE, rows=4, dim=128, codes=FAKE, scales=FAKE)
    a.update(kw)
    assert dsa.lib().dsa_mxfp8_quantize(a["x"], a["rows"], a["dim"], a["codes"], a["scales"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), 1), (dict(k_cache=None), 1), (dict(k_scale=None), 1),
    (dict(T=0), 2), (dict(dim=100), 4), (dict(k_new=FAKE + 2), 3),
    (dict(layout=_layout(page=32)), 4), (dict(layout=_layout(max_len=0)), 2),
])
def test_cache_append_rejects(kw, status):
    a = dict(k_new=FAKE, layout=_layout(), T=1, dim=128, k_cache=FAKE, k_scale=FAKE)
    a.update(kw)
    assert dsa.lib().dsa_indexer_cache_append(a["k_new"], ctypes.byref(a["layout"]), a["T"], a["dim"],
                                              a["k_cache"], a["k_scale"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), 1), (dict(k_cache=None), 1), (dict(k_scale=None), 1),
    (dict(T=0), 2), (dict(dim=96), 4), (dict(dim=256), 4), (dict(k_new=FAKE + 2), 3),
    (dict(k_cache=FAKE + 8), 3), (dict(k_scale=FAKE + 2), 3),
    (dict(layout=_layout(page=32)), 4), (dict(layout=_layout(max_len=0)), 2),
    (dict(layout=L.Layout(FAKE, FAKE + 256, 1 << 30, 1 << 14, 64, 9, 1 << 20), T=1 << 10), 2),
])
def test_fp8_cache_append_rejects(kw, status):
    a = dict(k_new=FAKE, layout=_layout(), T=1, dim=128, k_cache=FAKE, k_scale=FAKE)
    a.update(kw)
    assert dsa.lib().dsa_indexer_cache_append_fp8(a["k_new"], ctypes.byref(a["layout"]), a["T"], a["dim"],
                                                  a["k_cache"], a["k_scale"], None) == status

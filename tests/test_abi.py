"""The C ABI without a GPU: the library loads, exports every function the
header declares, and every argument check fires on the host before any HIP
call (so these run on a CPU-only machine)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsaidx.h")
LIB = os.path.join(ROOT, "dsa_lightning_indexer_03_amd", "libdsaidx.so")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, 1, 2, 3, 4, 5
P = 4096  # a fake, 16-byte aligned, non-NULL device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libdsaidx.so not built")
    from dsa_lightning_indexer_03_amd import _lib
    return _lib.load(LIB)


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("indexer_prefill", "indexer_decode_paged", "topk_select", "indexer_kcache_append",
                 "indexer_topk_gather", "indexer_prefill_chunk_paged"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    fns = header_functions()
    assert len(fns) >= 9
    for name in fns:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(fns) <= exported
    from dsa_lightning_indexer_03_amd import _lib
    assert set(fns) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    assert lib.dsaidx_status_string(0) == b"ok"
    for s in range(1, 7):
        assert lib.dsaidx_status_string(s) not in (b"ok", b"unknown status")
    assert lib.dsaidx_version() >= 100


def prefill(lib, q=P, qs=None, k=P, ks=None, dt=1, w=P, B=1, L=64, H=16, D=128, topk=8,
            idx=P, val=None, sc=None, ws=None, nws=0):
    return lib.indexer_prefill(q, qs, k, ks, dt, w, B, L, H, D, topk, idx, val, sc, ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(w=None), NULL), (dict(idx=None), NULL),
    (dict(dt=7), DTYPE), (dict(dt=2), NULL), (dict(dt=2, qs=P), NULL), (dict(qs=P), SHAPE),
    (dict(B=0), SHAPE), (dict(L=0), SHAPE), (dict(H=0), SHAPE), (dict(topk=0), SHAPE),
    (dict(L=131073), UNSUP), (dict(H=6), UNSUP), (dict(H=68), UNSUP), (dict(D=96), UNSUP),
    (dict(topk=2049), UNSUP), (dict(q=P + 4), UNSUP),
    (dict(dt=0, H=4, D=32), WS), (dict(dt=0, H=4, D=32, ws=P, nws=64 * 64 * 4 - 1), WS),
])
def test_prefill_rejects_before_launch(lib, kw, status):
    assert prefill(lib, **kw) == status
    assert lib.dsaidx_last_error()  # a detail message is set


def test_prefill_workspace_query(lib):
    # fused fp8: per-key adjusted scale and operand-scale byte (4 + 1 bytes per key)
    assert lib.indexer_prefill_workspace_bytes(1, 8192, 64, 128, 2048, 2, 0) == 8192 * 5
    # bf16 staged: fp32 adjusted scale + the scaled bf16 key, per 64-padded key
    assert lib.indexer_prefill_workspace_bytes(1, 8192, 64, 128, 2048, 1, 0) == 8192 * 260
    assert lib.indexer_prefill_workspace_bytes(2, 100, 16, 128, 64, 1, 0) == 2 * 128 * 260
    assert lib.indexer_prefill_workspace_bytes(1, 70000, 64, 128, 2048, 1, 0) == 0
    assert lib.indexer_prefill_workspace_bytes(2, 256, 4, 32, 16, 0, 0) == 2 * 256 * 256 * 4
    assert lib.indexer_prefill_workspace_bytes(2, 256, 4, 32, 16, 0, 1) == 0


def decode(lib, q=P, qd=1, w=P, kc=P, ks=P, bt=P, mpp=4, cl=P, mcl=256, B=2, H=64, D=128, ps=64,
           npg=8, topk=16, idx=P, val=None, ws=P, nws=None):
    if nws is None:
        nws = lib.indexer_decode_paged_workspace_bytes(B, mcl, H, D, topk)
    return lib.indexer_decode_paged(q, qd, w, kc, ks, bt, mpp, cl, mcl, B, H, D, ps, npg, topk, idx, val,
                                    ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(w=None), NULL), (dict(kc=None), NULL), (dict(ks=None), NULL),
    (dict(bt=None), NULL), (dict(cl=None), NULL), (dict(idx=None), NULL),
    (dict(qd=9), DTYPE), (dict(qd=0), UNSUP), (dict(qd=2), UNSUP),
    (dict(B=0), SHAPE), (dict(mcl=-1), SHAPE), (dict(mcl=257), SHAPE), (dict(npg=0), SHAPE),
    (dict(H=8), UNSUP), (dict(D=64), UNSUP), (dict(ps=32, mcl=128), UNSUP), (dict(topk=4096), UNSUP),
    (dict(ws=None), WS), (dict(nws=100), WS), (dict(kc=P + 8), UNSUP),
])
def test_decode_rejects_before_launch(lib, kw, status):
    assert decode(lib, **kw) == status


def test_decode_workspace_query(lib):
    n = lib.indexer_decode_paged_workspace_bytes(64, 131072, 64, 128, 2048)
    # candidate scores + positions, per-query counters, page prefix
    assert n == 64 * 131072 * 8 + 64 * 64 * 4 + 65 * 4


@pytest.mark.parametrize("args,status", [
    ((None, 4, 100, 100, None, 8, P, None), NULL),
    ((P, 4, 100, 100, None, 8, None, None), NULL),
    ((P, 0, 100, 100, None, 8, P, None), SHAPE),
    ((P, 4, 100, 99, None, 8, P, None), SHAPE),
    ((P, 4, 100, 100, None, 0, P, None), SHAPE),
    ((P, 4, 100, 100, None, 2049, P, None), UNSUP),
    ((P, 4, 4194305, 4194305, None, 8, P, None), UNSUP),
])
def test_topk_select_rejects_before_launch(lib, args, status):
    assert lib.topk_select(*args, None, 0, None) == status


def kcache(lib, k=P, dt=1, seq=P, pos=P, bt=P, B=2, mpp=4, kc=P, ks=P, npg=8, T=16, D=128, ps=64):
    return lib.indexer_kcache_append(k, dt, seq, pos, bt, B, mpp, kc, ks, npg, T, D, ps, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), NULL), (dict(seq=None), NULL), (dict(pos=None), NULL), (dict(bt=None), NULL),
    (dict(kc=None), NULL), (dict(ks=None), NULL),
    (dict(dt=7), DTYPE), (dict(dt=2), UNSUP),
    (dict(T=-1), SHAPE), (dict(B=0), SHAPE), (dict(mpp=0), SHAPE), (dict(npg=0), SHAPE),
    (dict(D=64), UNSUP), (dict(ps=32), UNSUP), (dict(k=P + 8), UNSUP), (dict(kc=P + 4), UNSUP),
])
def test_kcache_append_rejects_before_launch(lib, kw, status):
    assert kcache(lib, **kw) == status


def test_kcache_append_empty_is_a_no_op(lib):
    # T = 0 returns before any check of the arrays and before any HIP call
    assert kcache(lib, T=0, k=None, seq=None, pos=None) == OK


def gather(lib, lc=P, rb=1024, bt=P, mpp=4, npg=8, ps=64, idx=P, B=2, K=16, out=P):
    return lib.indexer_topk_gather(lc, rb, bt, mpp, npg, ps, idx, B, K, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lc=None), NULL), (dict(bt=None), NULL), (dict(idx=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(K=0), SHAPE), (dict(mpp=0), SHAPE), (dict(npg=0), SHAPE), (dict(rb=0), SHAPE),
    (dict(ps=32), UNSUP), (dict(rb=1000), UNSUP), (dict(rb=65552), UNSUP), (dict(lc=P + 8), UNSUP),
    (dict(out=P + 4), UNSUP),
])
def test_topk_gather_rejects_before_launch(lib, kw, status):
    assert gather(lib, **kw) == status


def chunk(lib, q=P, qs=P, dt=2, w=P, kc=P, ks=P, bt=P, mpp=64, npg=64, B=1, q0=100, Lq=64, H=64, D=128, ps=64,
          topk=2048, idx=P, val=None, ws=P, nws=1 << 20):
    return lib.indexer_prefill_chunk_paged(q, qs, dt, w, kc, ks, bt, mpp, npg, B, q0, Lq, H, D, ps, topk, idx, val,
                                           ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(qs=None), NULL), (dict(w=None), NULL), (dict(kc=None), NULL),
    (dict(ks=None), NULL), (dict(bt=None), NULL), (dict(idx=None), NULL),
    (dict(dt=9), DTYPE), (dict(dt=1), UNSUP), (dict(B=0), SHAPE), (dict(Lq=0), SHAPE), (dict(q0=-1), SHAPE),
    (dict(q0=4033), SHAPE), (dict(H=8), UNSUP), (dict(D=64), UNSUP), (dict(ps=32, mpp=128), UNSUP),
    (dict(topk=4096), UNSUP), (dict(mpp=2048, q0=65500, Lq=64), UNSUP), (dict(ws=None), WS), (dict(nws=100), WS),
    (dict(kc=P + 8), UNSUP),
])
def test_prefill_chunk_rejects_before_launch(lib, kw, status):
    assert chunk(lib, **kw) == status


def test_prefill_chunk_workspace_query(lib):
    # 5 bytes per visible key (64-padded), rounded to 256: q0 + Lq = 4160 keys
    assert lib.indexer_prefill_chunk_paged_workspace_bytes(2, 4096, 64) == (2 * 4160 * 5 + 255) // 256 * 256

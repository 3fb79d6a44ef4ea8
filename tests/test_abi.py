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
                 "indexer_topk_gather", "indexer_prefill_chunk_paged", "indexer_prefill_noalloc",
                 "indexer_topk_gather_layers"):
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


def prefill_noalloc(lib, q=P, qs=None, k=P, ks=None, dt=1, w=P, B=1, L=64, H=16, D=128, topk=8,
                    idx=P, val=None, sc=None):
    return lib.indexer_prefill_noalloc(q, qs, k, ks, dt, w, B, L, H, D, topk, idx, val, sc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(w=None), NULL), (dict(dt=7), DTYPE), (dict(dt=2), NULL), (dict(B=0), SHAPE),
    (dict(L=131073), UNSUP), (dict(H=6), UNSUP), (dict(topk=2049), UNSUP), (dict(q=P + 4), UNSUP),
    # beyond the scratch array: bf16 at 65536 x 2 keys (34 MB), the generic path's L*L matrix
    (dict(B=2, L=65536), UNSUP), (dict(dt=0, H=4, D=32, L=4096), UNSUP),
])
def test_prefill_noalloc_rejects_before_launch(lib, kw, status):
    """Every check of the entry point that allocates nothing -- including the
    scratch limit -- runs on the host before any HIP call."""
    assert prefill_noalloc(lib, **kw) == status
    assert lib.dsaidx_last_error()


def test_prefill_noalloc_scratch_size(lib):
    n = lib.indexer_prefill_noalloc_scratch_bytes()
    assert n == 32 << 20
    # the headline fp8 workload and the bf16 L=8192 workload fit; their workspace sizes are below the array
    assert lib.indexer_prefill_workspace_bytes(1, 32768, 64, 128, 2048, 2, 0) <= n
    assert lib.indexer_prefill_workspace_bytes(1, 8192, 64, 128, 2048, 1, 0) <= n


def test_prefill_workspace_query(lib):
    # fused fp8: per-key adjusted scale and operand-scale byte (4 + 1 bytes per key)
    assert lib.indexer_prefill_workspace_bytes(1, 8192, 64, 128, 2048, 2, 0) == 8192 * 5
    # bf16 staged: fp32 adjusted scale + the scaled bf16 key, per 64-padded key
    assert lib.indexer_prefill_workspace_bytes(1, 8192, 64, 128, 2048, 1, 0) == 8192 * 260
    assert lib.indexer_prefill_workspace_bytes(2, 100, 16, 128, 64, 1, 0) == 2 * 128 * 260
    # beyond 65536 positions the same staged kernel (17-bit candidate encoding)
    assert lib.indexer_prefill_workspace_bytes(1, 70000, 64, 128, 2048, 1, 0) == 70016 * 260
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


def gather_layers(lib, n=3, lc=P, out=P, rb=1024, bt=P, mpp=8, npg=8, ps=64, idx=P, B=2, K=16, caches=None,
                  outs=None):
    cp = (ctypes.c_void_p * max(n, 1))(*([lc] * max(n, 1) if caches is None else caches))
    op = (ctypes.c_void_p * max(n, 1))(*([out] * max(n, 1) if outs is None else outs))
    return lib.indexer_topk_gather_layers(cp, op, n, rb, bt, mpp, npg, ps, idx, B, K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), NULL), (dict(idx=None), NULL), (dict(caches=[P, None, P]), NULL), (dict(outs=[P, P, None]), NULL),
    (dict(n=0), SHAPE), (dict(B=0), SHAPE), (dict(K=0), SHAPE), (dict(rb=0), SHAPE), (dict(mpp=0), SHAPE),
    (dict(n=65), UNSUP), (dict(ps=32), UNSUP), (dict(rb=1000), UNSUP), (dict(caches=[P, P + 8, P]), UNSUP),
    (dict(outs=[P + 4, P, P]), UNSUP),
])
def test_topk_gather_layers_rejects_before_launch(lib, kw, status):
    assert gather_layers(lib, **kw) == status


def test_topk_gather_layers_null_arrays(lib):
    assert lib.indexer_topk_gather_layers(None, (ctypes.c_void_p * 1)(P), 1, 1024, P, 8, 8, 64, P, 2, 16, None) == NULL
    assert lib.indexer_topk_gather_layers((ctypes.c_void_p * 1)(P), None, 1, 1024, P, 8, 8, 64, P, 2, 16, None) == NULL


@pytest.mark.parametrize("args,status", [
    ((0, 4, 8, None), NULL), ((3, 4, 8, P), UNSUP), ((-1, 4, 8, P), UNSUP), ((0, 0, 8, P), SHAPE),
    ((1, 65537, 8, P), SHAPE), ((2, 4, 0, P), SHAPE), ((2, 4, (1 << 20) + 1, P), SHAPE),
])
def test_probe_mfma_rejects_before_launch(lib, args, status):
    assert lib.dsaidx_probe_mfma(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, P, P, 8, 4, P), NULL), ((P, None, P, 8, 4, P), NULL), ((P, P, None, 8, 4, P), NULL),
    ((P, P, P, 8, 4, None), NULL), ((P, P, P, 0, 4, P), SHAPE), ((P, P, P, 8, 0, P), SHAPE),
    ((P + 8, P, P, 8, 4, P), UNSUP),
])
def test_probe_page_read_rejects_before_launch(lib, args, status):
    assert lib.dsaidx_probe_page_read(*args, None) == status


def chunk(lib, q=P, qs=P, dt=2, w=P, cu=P, q0s=P, kc=P, ks=P, bt=P, mpp=64, npg=64, B=1, T=64, mkv=164, H=64, D=128,
          ps=64, topk=2048, idx=P, val=None, ws=P, nws=1 << 20):
    return lib.indexer_prefill_chunk_paged(q, qs, dt, w, cu, q0s, kc, ks, bt, mpp, npg, B, T, mkv, H, D, ps, topk, idx,
                                           val, ws, nws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(qs=None), NULL), (dict(w=None), NULL), (dict(cu=None), NULL), (dict(q0s=None), NULL),
    (dict(kc=None), NULL), (dict(ks=None), NULL), (dict(bt=None), NULL), (dict(idx=None), NULL),
    (dict(dt=9), DTYPE), (dict(dt=0), UNSUP), (dict(dt=1, qs=P), UNSUP), (dict(B=0), SHAPE), (dict(T=0), SHAPE),
    (dict(mkv=0), SHAPE),
    (dict(mkv=4097), SHAPE), (dict(H=8), UNSUP), (dict(D=64), UNSUP), (dict(ps=32, mpp=128), UNSUP),
    (dict(topk=4096), UNSUP), (dict(mpp=4096, mkv=131073), UNSUP), (dict(ws=None), WS), (dict(nws=100), WS),
    (dict(kc=P + 8), UNSUP),
])
def test_prefill_chunk_rejects_before_launch(lib, kw, status):
    assert chunk(lib, **kw) == status


def test_prefill_chunk_workspace_query(lib):
    # fp8 queries: 5 bytes per key up to max_kv_len (64-padded) per sequence,
    # rounded to 256, then one 8-byte plan entry per 8-row block bound (T/8 + B)
    assert lib.indexer_prefill_chunk_paged_workspace_bytes(2, 128, 4160, 2) == \
        (2 * 4160 * 5 + 255) // 256 * 256 + (128 // 8 + 2) * 8
    assert lib.indexer_prefill_chunk_paged_workspace_bytes(64, 64, 131072, 2) == \
        (64 * 131072 * 5 + 255) // 256 * 256 + (64 // 8 + 64) * 8
    # bf16 queries: 4 + 256 bytes per key (adjusted scale, key widened to
    # bf16), then the plan
    assert lib.indexer_prefill_chunk_paged_workspace_bytes(2, 128, 4100, 1) == \
        2 * 4160 * 260 + (128 // 8 + 2) * 8
    assert lib.indexer_prefill_chunk_paged_workspace_bytes(3, 0, 4100, 1) == 0


# ---- the Python binding's own checks (host-side, before any device access) ----

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _wrapper_cases():
    import torch
    i32, i64, f32, f64, u8, bf = torch.int32, torch.int64, torch.float32, torch.float64, torch.uint8, torch.bfloat16
    B, L, H, D, P = 2, 64, 16, 128, 8
    dec = dict(q=_t((B, H, D), bf), w=_t((B, H), f32), k_cache=_t((P, 64, D), u8), k_scale=_t((P, 64), f32),
               block_table=_t((B, 4), i32), context_lens=_t((B,), i32), topk=16)
    pre = dict(q=_t((1, L, H, D), u8), k=_t((1, L, D), u8), w=_t((1, L, H), f32), topk=8,
               q_scale=_t((1, L, H), f32), k_scale=_t((1, L), f32))
    kc = dict(k=_t((5, D), bf), seq_ids=_t((5,), i32), positions=_t((5,), i32), block_table=_t((B, 4), i32),
              k_cache=_t((P, 64, D), u8), k_scale=_t((P, 64), f32))
    ch = dict(q=_t((B, 32, H, D), u8), q_scale=_t((B, 32, H), f32), w=_t((B, 32, H), f32),
              k_cache=_t((P, 64, D), u8), k_scale=_t((P, 64), f32), block_table=_t((B, 4), i32), q0=100, topk=16)
    cv = dict(q=_t((40, H, D), u8), q_scale=_t((40, H), f32), w=_t((40, H), f32), cu_seqlens_q=_t((B + 1,), i32),
              q_start=_t((B,), i32), k_cache=_t((P, 64, D), u8), k_scale=_t((P, 64), f32),
              block_table=_t((B, 4), i32), topk=16, max_kv_len=200)
    ga = dict(latent_cache=_t((P, 64, 512), bf), block_table=_t((B, 4), i32), topk_idx=_t((B, 16), i32))
    cases = []
    for fn, base, bad in (
        ("indexer_decode_paged", dec, [("block_table", i64), ("context_lens", i64), ("w", f64), ("k_scale", f64),
                                       ("k_cache", f32)]),
        ("indexer_prefill", pre, [("w", f64), ("q_scale", f64), ("k_scale", torch.float16)]),
        ("kcache_append", kc, [("seq_ids", i64), ("positions", i64), ("block_table", i64)]),
        ("prefill_chunk_paged", ch, [("block_table", i64), ("q_scale", f64), ("w", f64), ("k_scale", f64),
                                     ("k_cache", i32)]),
        ("topk_gather", ga, [("block_table", i64), ("topk_idx", i64)]),
        ("prefill_chunk_varlen", cv, [("cu_seqlens_q", i64), ("q_start", i64), ("block_table", i64),
                                      ("q_scale", f64), ("w", f64), ("k_scale", f64), ("k_cache", i32)]),
    ):
        for name, dt in bad:
            kw = dict(base)
            kw[name] = kw[name].to(dt)
            cases.append((fn, kw, name))
    return cases


@pytest.mark.parametrize("case", range(len(_wrapper_cases())))
def test_binding_rejects_wrong_element_types(lib, case):
    """An index or table tensor that is not int32, or a weight / scale tensor
    that is not fp32, is refused by the binding with a ValueError naming the
    tensor, before anything reaches the library."""
    import dsa_lightning_indexer_03_amd as dsa
    fn, kw, name = _wrapper_cases()[case]
    with pytest.raises(ValueError, match=name):
        getattr(dsa, fn)(**kw)


def test_binding_rejects_host_tensors(lib):
    """Well-typed tensors on the host are refused (device pointers only)."""
    import dsa_lightning_indexer_03_amd as dsa
    for fn, kw, _ in _wrapper_cases()[:1]:
        kw = dict(kw)
        kw["block_table"] = kw["block_table"].to(__import__("torch").int32)
        kw["context_lens"] = kw["context_lens"].to(__import__("torch").int32)
        kw["w"] = kw["w"].float()
        kw["k_scale"] = kw["k_scale"].float()
        kw["k_cache"] = kw["k_cache"].to(__import__("torch").uint8)
        with pytest.raises(ValueError, match="device tensor"):
            getattr(dsa, fn)(**kw)

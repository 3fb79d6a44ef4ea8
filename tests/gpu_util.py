"""Host <-> device helpers for the GPU parity tests (no arithmetic)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dsa_lightning_indexer_03_amd as dsa


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return None if t is None else t.cpu().numpy()


def run_prefill(inp: dict, K: int, want_scores: bool = False):
    idx, val, sc = dsa.indexer_prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), K,
                                       q_scale=dev(inp.get("q_scale")), k_scale=dev(inp.get("k_scale")),
                                       want_scores=want_scores)
    torch.cuda.synchronize()
    return host(idx), host(val), host(sc)


def run_decode(d: dict, K: int, max_context_len=None):
    idx, val = dsa.indexer_decode_paged(dev(d["q"]), dev(d["w"]), dev(d["k_cache"]), dev(d["k_scale"]),
                                        dev(d["block_table"]), dev(d["context_lens"]), K,
                                        max_context_len=max_context_len)
    torch.cuda.synchronize()
    return host(idx), host(val)

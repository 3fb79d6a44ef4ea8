"""Pins of the top-k gather oracle (oracle/gather.py): a hand-worked case,
the padding rule, and agreement with a vectorised re-indexing."""
import numpy as np

from oracle.gather import topk_gather, topk_gather_layers


def test_hand_worked_gather():
    # 3 pages of 2 slots, rows of 4 bytes: row value = 10*page + slot in every byte
    cache = np.array([[[10 * p + s] * 4 for s in range(2)] for p in range(3)], np.uint8)
    table = np.array([[2, 0], [1, 2]], np.int32)            # seq 0: pages 2, 0; seq 1: pages 1, 2
    idx = np.array([[3, 0, -1], [1, 2, 4]], np.int32)      # position 4 is past 2 pages of 2 slots
    out = topk_gather(cache, table, idx, page_size=2)
    # seq 0: position 3 -> page table[0][1] = 0, slot 1 -> 1; position 0 -> page 2, slot 0 -> 20
    # seq 1: position 1 -> page 1, slot 1 -> 11; position 2 -> page 2, slot 0 -> 20; 4 -> zeros
    assert out[:, :, 0].tolist() == [[1, 20, 0], [11, 20, 0]]
    assert np.all(out[0, 2] == 0) and np.all(out[1, 2] == 0)


def test_matches_vectorised_indexing():
    rng = np.random.default_rng(1)
    cache = rng.integers(0, 256, size=(50, 64, 32), dtype=np.uint8)
    table = rng.permutation(50)[:48].reshape(4, 12).astype(np.int32)
    idx = rng.integers(-1, 12 * 64, size=(4, 100)).astype(np.int32)
    out = topk_gather(cache, table, idx)
    valid = idx >= 0
    b = np.repeat(np.arange(4)[:, None], 100, axis=1)
    pages = table[b, np.where(valid, idx, 0) // 64]
    ref = cache[pages, np.where(valid, idx, 0) % 64] * valid[..., None]
    assert np.array_equal(out, ref)


def test_layers_share_one_selection():
    # three layers whose rows encode (layer, page, slot): each output row
    # names the layer it came from and the page/slot the shared index maps to
    cache = np.array([[[[40 * l + 10 * p + s] * 4 for s in range(2)] for p in range(3)] for l in range(3)],
                     np.uint8)
    table = np.array([[2, 0], [1, 2]], np.int32)
    idx = np.array([[3, 0, -1], [1, 2, 4]], np.int32)
    outs = topk_gather_layers(list(cache), table, idx, page_size=2)
    assert len(outs) == 3
    for l, o in enumerate(outs):
        # the rows of the single-layer hand case, offset by 40 * layer; padding rows stay zero
        assert o[:, :, 0].tolist() == [[1 + 40 * l, 20 + 40 * l, 0], [11 + 40 * l, 20 + 40 * l, 0]]

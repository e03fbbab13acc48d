"""The seeded input generator: determinism, layout, poison placement (CPU only)."""
import hashlib

import numpy as np

from mla_latent_space_amd import workloads as wl


def _digest(w):
    h = hashlib.sha256()
    for a in (w.seqlens, w.q, w.kv, w.block_table) + ((w.kv_scales,) if w.kv_scales is not None else ()):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = wl.make_workload(batch=3, s_q=2, heads=4, seqlens=[65, 1, 130], seed=5)
    b = wl.make_workload(batch=3, s_q=2, heads=4, seqlens=[65, 1, 130], seed=5)
    c = wl.make_workload(batch=3, s_q=2, heads=4, seqlens=[65, 1, 130], seed=6)
    assert _digest(a) == _digest(b) != _digest(c)


def test_block_table_is_a_partial_permutation():
    w = wl.make_workload(batch=4, s_q=1, heads=4, seqlens=[64, 65, 0, 300], seed=1)
    live = w.block_table[w.block_table >= 0]
    assert len(set(live.tolist())) == live.size == 1 + 2 + 0 + 5
    assert w.num_pages == live.size + max(1, live.size // 16)
    for i, t in enumerate(w.seqlens):
        n = (int(t) + 63) // 64
        assert np.all(w.block_table[i, :n] >= 0) and np.all(w.block_table[i, n:] == -1)


def test_poison_only_outside_live_tokens():
    w = wl.make_workload(batch=2, s_q=1, heads=4, seqlens=[70, 128], seed=2)
    nan = (w.kv & 0x7FFF) > 0x7F80
    live = np.zeros(nan.shape[:2], dtype=bool)
    for i, t in enumerate(w.seqlens):
        for u in range(int(t)):
            live[w.block_table[i, u // 64], u % 64] = True
    assert not nan[live].any()
    assert nan[~live].all()


def test_fp8_layout_and_scales():
    w = wl.make_workload(batch=1, s_q=1, heads=4, seqlens=[64], kv_dtype="fp8", seed=3)
    assert w.kv.shape[1:] == (64, 640) and w.kv.dtype == np.uint8
    assert w.kv_scales.shape[1:] == (64, 4)
    page = w.block_table[0, 0]
    codes = w.kv[page, :, :512].reshape(64, 4, 128)
    # every tile's amax maps to the largest finite code magnitude (0x7E = 448)
    assert np.all((codes & 0x7F).max(axis=2) == 0x7E)


def test_named_configs_small_ones_build():
    w = wl.make_config("tiny")
    assert (w.batch, w.s_q, w.heads) == (2, 1, 16) and list(w.seqlens) == [256, 256]
    assert w.q.shape == (2, 1, 16, 576)

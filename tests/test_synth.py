"""Input generator checks (no GPU): determinism, role independence, shapes."""
import hashlib

import numpy as np

import synth


def digest(w):
    h = hashlib.sha256()
    for off, d in w.pool.segments():
        h.update(np.int64(off).tobytes())
        h.update(d.tobytes())
    for a in (w.q, w.seq_lens, w.block_table, w.page_k_off, w.page_v_off, w.page_codec, w.page_scale):
        h.update(np.ascontiguousarray(a).tobytes())
    if w.page_sel is not None:
        h.update(w.page_sel.tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    for cid in (1, 3, 4):
        assert digest(synth.config(cid, small=True)) == digest(synth.config(cid, small=True))


def test_placement_stream_is_independent():
    a = synth.config(3, small=True)
    rng = synth.streams(1003)
    rng["placement"] = np.random.default_rng(1)
    b = synth.build_workload("x", rows=a.rows, hq=32, hkv=8, dim=128, page=16,
                             seq_lens=a.seq_lens, codec_of=lambda r, lp: (3, 4), seed=1003,
                             rng=rng, max_pages=a.max_pages)
    assert np.array_equal(a.q, b.q)
    assert not np.array_equal(a.block_table, b.block_table)


def test_config_shapes_full_geometry():
    w = synth.config(1)
    assert (w.rows, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size) == (1, 14, 2, 64, 1024)
    assert sorted(w.block_table[0].tolist()) == [0, 1, 2, 3]
    w4 = synth.config(4, small=True)
    assert w4.sparse and np.all(w4.page_sel[:, -1] == 4096 // 16 - 1)
    for r in range(w4.rows):
        assert len(set(w4.page_sel[r].tolist())) == w4.page_sel.shape[1]


def test_page_alignment():
    for cid in (2, 3, 5):
        w = synth.config(cid, small=True)
        assert np.all(w.page_k_off % 256 == 0) and np.all(w.page_v_off % 256 == 0)

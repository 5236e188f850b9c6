"""The seeded generators: deterministic, block tables are permutations of the
physical blocks, NaN sentinels sit only in slots no token owns."""
import numpy as np

from rank_compressed_paged_amd import workloads as wl


def _owned_mask(cache):
    nb, H, bs, r_k = cache.k_cache.shape
    owned = np.zeros((nb, bs), dtype=bool)
    for b, L in enumerate(cache.seq_lens):
        for t in range(int(L)):
            owned[cache.block_tables[b, t // bs], t % bs] = True
    return owned


def test_deterministic():
    a = wl.make_config("tiny")
    b = wl.make_config("tiny")
    for x, y in ((a.U, b.U), (a.W, b.W), (a.q, b.q), (a.cache.k_cache, b.cache.k_cache),
                 (a.cache.v_cache, b.cache.v_cache), (a.cache.block_tables, b.cache.block_tables)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_tiny_shapes_and_sentinels():
    c = wl.make_config("tiny", keep_logical=True)
    sh = c.shape
    assert c.U.shape == (sh.H, sh.d, sh.r_k) and c.W.shape == (sh.H * sh.d, sh.r_v)
    assert c.q.shape == (2, sh.H, sh.d)
    bt = c.cache.block_tables
    used = bt[bt >= 0]
    assert len(set(used.tolist())) == used.size          # no block shared
    assert used.max() < c.cache.num_blocks
    owned = _owned_mask(c.cache)
    kc, vc = c.cache.k_cache, c.cache.v_cache
    for blk in range(c.cache.num_blocks):
        for off in range(sh.bs):
            kn = np.isnan(kc[blk, :, off, :])
            vn = np.isnan(vc[blk, :, off])
            if owned[blk, off]:
                assert not kn.any() and not vn.any()
            else:
                assert kn.all() and vn.all()


def test_bases_orthonormal():
    c = wl.make_config("tiny")
    for h in range(c.shape.H):
        g = c.U[h].astype(np.float64).T @ c.U[h].astype(np.float64)
        assert np.max(np.abs(g - np.eye(c.shape.r_k))) < 5e-3
    g = c.W.astype(np.float64).T @ c.W.astype(np.float64)
    assert np.max(np.abs(g - np.eye(c.shape.r_v))) < 5e-3


def test_ragged_uniform_lengths_in_range():
    rng = np.random.default_rng(0)
    L = wl.draw_seq_lens(rng, 1000, ("uniform", 4096, 8192))
    assert L.min() >= 4096 and L.max() <= 8192


def test_prefill_slots_point_at_chunk_positions():
    sh = wl.Shape(H=2, d=8, r_k=4, r_v=8, bs=4)
    c = wl.make_prefill_case(sh, [5, 0], [3, 6], seed=3)
    assert list(c.query_start_loc) == [0, 3, 9]
    assert list(c.seq_lens) == [8, 6]
    # request 0: positions 5, 6, 7 -> logical block 1, offsets 1..3
    bt = c.cache.block_tables
    assert list(c.slot_mapping[:3]) == [bt[0, 1] * 4 + 1, bt[0, 1] * 4 + 2, bt[0, 1] * 4 + 3]
    # the chunk's slots are still NaN before append
    for s in c.slot_mapping:
        assert np.isnan(c.cache.k_cache[s // 4, :, s % 4, :]).all()

"""GPU index checks (starkv_check_indices) against a plain numpy scan of the
same rules, bit-exact: the flag bits and the first offending sequence or
token of each kind.  Block-table entries beyond a sequence's pages, and
negative slots (padding), are not errors.  The arrays are the decode and
prefill workloads' own, then with planted mistakes, then random ones.  Then
what the decode, prefill and append kernels do with such indices: skip them,
against the oracle on the same data with the bad pages removed or the bad
slots made padding."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, decode_tensors, dev, note
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu

NONE = -1  # the uint32 0xFFFFFFFF read as int32


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def reference(bt, sl, max_seq_len, num_blocks, slots):
    """The report the call must write, by a direct loop over the rules."""
    flags, bad_blk, bad_len, bad_slot = 0, NONE, NONE, NONE
    for b, L in enumerate(sl.tolist()):
        if L < 0 or L > max_seq_len:
            flags |= 2
            bad_len = b if bad_len == NONE else bad_len
        pages = (min(max(L, 0), max_seq_len) + 15) // 16
        if any(not (0 <= x < num_blocks) for x in bt[b, :pages].tolist()):
            flags |= 1
            bad_blk = b if bad_blk == NONE else bad_blk
    if slots is not None:
        for n, s in enumerate(slots.tolist()):
            if s >= num_blocks * 16:
                flags |= 4
                bad_slot = n if bad_slot == NONE else bad_slot
    return [flags, bad_blk, bad_len, bad_slot]


def run(sk, bt, sl, max_seq_len, num_blocks, slots=None):
    rep = sk.check_indices(dev(bt), dev(sl), max_seq_len, num_blocks,
                           None if slots is None else dev(slots))
    torch.cuda.synchronize()
    return rep.cpu().tolist()


@pytest.mark.parametrize("name", ["decode_b16", "decode_b64", "prefill_b16", "tiny"])
def test_workload_indices_are_clean(sk, name):
    case = wl.make_config(name)
    c = case.cache
    nb = c.k_cache.shape[0]
    slots = getattr(case, "slot_mapping", None)
    note(f"index check clean {name}")
    got = run(sk, c.block_tables, c.seq_lens, int(c.seq_lens.max()), nb, slots)
    assert got == [0, NONE, NONE, NONE]
    assert got == reference(c.block_tables, c.seq_lens, int(c.seq_lens.max()), nb, slots)


def test_planted_mistakes(sk):
    case = wl.make_decode_case(wl.MAIN, seq_lens=[300, 40, 2048, 17, 1000, 5, 64, 900, 33, 2],
                               seed=91, extra_cols=4)
    c = case.cache
    nb = c.k_cache.shape[0]
    bt, sl = c.block_tables.copy(), c.seq_lens.copy()
    msl = int(bt.shape[1]) * 16
    bt[1, bt.shape[1] - 1] = nb + 7     # past sequence 1's pages: not an error
    bt[4, 62] = nb                      # page 62 of 1000 tokens: an error
    bt[8, 2] = -5                       # the last page of 33 tokens: an error
    sl[6] = msl + 1                     # length beyond the bound
    sl[9] = -3                          # negative length
    slots = np.arange(40, dtype=np.int64) * 3
    slots[[4, 30]] = -1                 # padding
    slots[11] = nb * 16                 # first slot past the cache
    slots[20] = 1 << 40
    note("index check planted mistakes")
    got = run(sk, bt, sl, msl, nb, slots)
    want = reference(bt, sl, msl, nb, slots)
    assert want == [7, 4, 6, 11]
    assert got == want


@pytest.mark.parametrize("seed", range(6))
def test_random_indices(sk, seed):
    """Random tables, lengths and slots with a few mistakes of each kind (or
    none), batch up to 300 with up to 512 table entries per sequence."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 300))
    mb = int(rng.integers(1, 512))
    nb = int(rng.integers(1, 5000))
    msl = mb * 16 - int(rng.integers(0, 16))
    sl = rng.integers(0, msl + 1, size=B).astype(np.int32)
    bt = rng.integers(0, nb, size=(B, mb)).astype(np.int32)
    slots = rng.integers(-1, nb * 16, size=int(rng.integers(0, 3000))).astype(np.int64)
    if seed % 3 != 0:
        for _ in range(int(rng.integers(1, 4))):
            bt[rng.integers(0, B), rng.integers(0, mb)] = int(rng.choice([-1, nb, nb + 100, 1 << 30]))
        if seed % 2:
            sl[rng.integers(0, B)] = msl + int(rng.integers(1, 50))
        if slots.size:
            slots[rng.integers(0, slots.size)] = nb * 16 + int(rng.integers(0, 1000))
    note(f"index check random seed={seed} B={B} max_blocks={mb} slots={slots.size}")
    got = run(sk, bt, sl, msl, nb, slots if slots.size else None)
    assert got == reference(bt, sl, msl, nb, slots if slots.size else None)


# ---------------------------------------------------------------------------
# What the attention and append kernels do with the indices the check
# reports: they skip them.  A page whose block id lies outside the cache
# contributes nothing, which is the oracle's attention over the sequence with
# that page removed (the latents carry no position); a slot past the cache is
# not written, which is the oracle's append with that slot as padding.
# ---------------------------------------------------------------------------


def _drop_pages(bt, sl, drops):
    """Block table and lengths with the (sequence, page) entries removed."""
    bt2, sl2 = bt.copy(), sl.copy()
    for b, pages in drops.items():
        L = int(sl[b])
        keep = [j for j in range((L + 15) // 16) if j not in pages]
        row = [int(bt[b, j]) for j in keep]
        bt2[b, :] = 0
        bt2[b, :len(row)] = row
        sl2[b] = L - sum(min(16, L - 16 * j) for j in pages)
    return bt2, sl2


@pytest.mark.parametrize("shape", ["main", "tiny", "odd"])
def test_decode_skips_out_of_range_block_ids(sk, shape):
    shp = {"main": wl.MAIN, "tiny": wl.TINY, "odd": wl.ODD_H28}[shape]
    case = wl.make_decode_case(shp, seq_lens=[300, 700, 2048], seed=92)
    c = case.cache
    nb = c.k_cache.shape[0]
    bt = c.block_tables.copy()
    bt[0, 18] = nb          # the partial last page (12 of 300 tokens)
    bt[1, 10] = nb + 3      # a full page inside
    bt[2, 127] = -1         # the full last page
    drops = {0: [18], 1: [10], 2: [127]}
    t = decode_tensors(case)
    t["block_tables"] = dev(bt)
    note(f"decode with out-of-range block ids, {shape}")
    rep = sk.check_indices(t["block_tables"], t["seq_lens"], 2048, nb)
    out = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                         t["seq_lens"], 2048, case.scale)
    torch.cuda.synchronize()
    assert rep.cpu().tolist() == [1, 0, NONE, NONE]
    bt2, sl2 = _drop_pages(bt, c.seq_lens, drops)
    ref = oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, bt2, sl2, case.scale)
    assert_parity(out, ref, f"decode skipping bad block ids ({shape})")


def test_prefill_skips_out_of_range_block_ids(sk):
    case = wl.make_prefill_case(wl.MAIN, [64, 300], [40, 65], seed=93)
    c = case.cache
    nb = c.k_cache.shape[0]
    tk, tv = dev(c.k_cache), dev(c.v_cache)
    U, W = dev(case.U), dev(case.W)
    sk.append(dev(case.k_new), dev(case.v_new), U, W, dev(case.slot_mapping), tk, tv)
    bt = c.block_tables.copy()
    bt[1, 5] = nb + 1       # a fully cached page of the second request
    note("prefill with an out-of-range block id")
    chunk = np.diff(case.query_start_loc)
    out = sk.prefill_attn(dev(case.q), dev(case.query_start_loc), int(chunk.max()), tk, tv, U, W,
                          dev(bt), dev(c.seq_lens), int(c.seq_lens.max()), case.scale)
    torch.cuda.synchronize()
    bt2, sl2 = _drop_pages(bt, c.seq_lens, {1: [5]})
    ref = oracle.prefill(case.q, case.query_start_loc, tk.cpu().numpy(), tv.cpu().numpy(), case.U,
                         case.W, bt2, sl2, case.scale)
    assert_parity(out, ref, "prefill skipping a bad block id")


def _ulp_diff(a, b):
    ai = a.view(np.int16).astype(np.int32)
    bi = b.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -32768 - ai, ai)
    bi = np.where(bi < 0, -32768 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("n", [40, 300], ids=["few_tokens", "many_tokens"])
def test_append_skips_slots_past_the_cache(sk, n):
    shape = wl.MAIN
    rng = np.random.default_rng(94 + n)
    U, W = wl.draw_bases(rng, shape)
    nb = (n + 15) // 16 + 2
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    bad = [1, n // 2, n - 1]
    slots[bad] = [nb * 16, nb * 16 + 5, 1 << 40]
    k = rng.standard_normal((n, shape.H, shape.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, shape.H, shape.d), dtype=np.float32).astype(np.float16)
    kc = wl._nan_f16((nb, shape.H, 16, shape.r_k))
    vc = wl._nan_f16((nb, shape.r_v, 16))
    note(f"append with slots past the cache, n={n}")
    tk, tv, ts = dev(kc), dev(vc), dev(slots)
    rep = sk.check_indices(dev(np.zeros((1, 1), np.int32)), dev(np.zeros(1, np.int32)), 16, nb,
                           ts)
    sk.append(dev(k), dev(v), dev(U), dev(W), ts, tk, tv)
    torch.cuda.synchronize()
    assert rep.cpu().tolist() == [4, NONE, NONE, 1]
    pad = slots.copy()
    pad[bad] = -1
    rk, rv = oracle.append(k, v, U, W, pad, kc, vc)
    gk, gv = tk.cpu().numpy(), tv.cpu().numpy()
    for g, r, atol in ((gk, rk, 5e-7), (gv, rv, 5e-6)):
        assert np.array_equal(np.isnan(g), np.isnan(r))
        m = ~np.isnan(r)
        a = np.abs(g[m].astype(np.float64) - r[m].astype(np.float64))
        assert ((_ulp_diff(g[m], r[m]) <= 1) | (a <= atol)).all()

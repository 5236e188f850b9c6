"""GPU parity of decode attention (q projection, split-K latent attention,
merge of the splits with the up-projection) against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, decode_tensors, note, run_decode
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def _oracle(case, rows=None):
    c = case.cache
    return oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                         c.seq_lens, case.scale, batch_indices=rows)


def test_tiny_config(sk):
    case = wl.make_config("tiny")
    note("decode tiny config")
    out = run_decode(sk, case)
    assert_parity(out, _oracle(case), "tiny")


@pytest.mark.parametrize("lens", [[1, 17, 300], [16, 15, 33, 64, 2], [0, 1, 4097, 31]],
                         ids=["short", "page_edges", "long_and_empty"])
def test_main_shape_ragged(sk, lens):
    case = wl.make_decode_case(wl.MAIN, seq_lens=lens, seed=21, extra_cols=3)
    note(f"decode main shape lens={lens}")
    out = run_decode(sk, case)
    ref = _oracle(case)
    assert_parity(out, ref, f"main {lens}")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def test_tiny_shape_ragged(sk):
    case = wl.make_decode_case(wl.TINY, seq_lens=[3, 0, 16, 17, 250], seed=22)
    note("decode tiny shape ragged")
    assert_parity(run_decode(sk, case), _oracle(case), "tiny ragged")


def test_block_table_permutation_is_bit_identical(sk):
    """Same logical latents in shuffled and identity page orders."""
    lens = [40, 513, 7]
    a = wl.make_decode_case(wl.MAIN, seq_lens=lens, seed=23, shuffle=True, keep_logical=True)
    b = wl.make_decode_case(wl.MAIN, seq_lens=lens, seed=23, shuffle=False, keep_logical=True)
    assert not np.array_equal(a.cache.block_tables, b.cache.block_tables)
    note("decode shuffled vs identity block table")
    for x, y in zip(a.cache.logical_ck or [], b.cache.logical_ck or []):
        assert np.array_equal(x, y)
    oa = run_decode(sk, a)
    ob = run_decode(sk, b)
    assert_parity(oa, _oracle(a), "shuffled pages")
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_repeatable(sk):
    case = wl.make_decode_case(wl.MAIN, seq_lens=[100, 1000], seed=24)
    t = decode_tensors(case)
    note("decode repeatability")
    o1 = run_decode(sk, case, t).clone()
    o2 = run_decode(sk, case, t)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def _run_planned(sk, case, **plan):
    t = decode_tensors(case)
    msl = int(case.cache.seq_lens.max())
    out = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                         t["seq_lens"], msl, case.scale, **plan)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("launches", [2, 3])
@pytest.mark.parametrize("pps", [1, 3, 64, 256])
def test_split_plan_invariance(sk, pps, launches):
    """Any split plan (here fixed through the plan-override entry point) gives
    the same attention within the parity bars, with the split pass and the
    merge fused into one kernel (2 launches) or as separate kernels (3)."""
    case = wl.make_decode_case(wl.MAIN, seq_lens=[1500, 700, 33], seed=25)
    ref = _oracle(case)
    note(f"decode split plan pages_per_split={pps} launches={launches}")
    out = _run_planned(sk, case, pages_per_split=pps, launches=launches)
    assert_parity(out, ref, f"plan pps={pps} launches={launches}")


@pytest.mark.parametrize("launches", [2, 3])
@pytest.mark.parametrize("tb", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", ["main", "tiny"])
def test_finish_tiles(sk, tb, shape, launches):
    """The merge of the splits and the up-projection with 1, 2, 4 or 8
    sequences per work group (and so split groups, 16, 8 or 4 splits per
    request round, several rounds where the plan has more splits), on a batch
    that leaves the last sequence group partly empty and holds an empty
    sequence."""
    cfg = wl.MAIN if shape == "main" else wl.TINY
    case = wl.make_decode_case(cfg, seq_lens=[1500, 0, 33, 700, 5], seed=27)
    ref = _oracle(case)
    note(f"decode finish tile tb={tb} shape={shape} launches={launches}")
    out = _run_planned(sk, case, merge_seqs=tb, launches=launches)
    assert_parity(out, ref, f"finish tb={tb} {shape} launches={launches}")
    assert torch.count_nonzero(out[1]).item() == 0


@pytest.mark.parametrize("lens", [[8192], [2048, 2048], [16384, 3, 9000, 600]],
                         ids=["b1_long", "b2", "b4_ragged"])
def test_small_batch_many_splits(sk, lens):
    """Small batches split each sequence into many work groups (up to 256
    splits), which the merge takes in split groups and several rounds."""
    case = wl.make_decode_case(wl.MAIN, seq_lens=lens, seed=28)
    note(f"decode small batch lens={lens}")
    assert_parity(run_decode(sk, case), _oracle(case), f"small batch {lens}")


def test_max_seq_len_bound_larger_than_lengths(sk):
    """The host bound only plans the split; a loose bound gives the same result."""
    case = wl.make_decode_case(wl.MAIN, seq_lens=[90, 31], seed=26, extra_cols=40)
    note("decode loose max_seq_len")
    o1 = run_decode(sk, case)
    o2 = run_decode(sk, case, max_seq_len=(case.cache.block_tables.shape[1]) * 16)
    ref = _oracle(case)
    assert_parity(o1, ref, "tight bound")
    assert_parity(o2, ref, "loose bound")


@pytest.mark.parametrize("name,rows", [("decode_b16", None),
                                       ("decode_b64", [0, 3, 9, 17, 22, 28, 31, 35, 40, 44, 47,
                                                       51, 55, 58, 61, 63]),
                                       ("long_b20", [0, 2, 5, 8, 11, 14, 17, 19])])
def test_full_size_config_sampled(sk, name, rows):
    """Full-size workload in the benchmark's launch configuration; the oracle
    checks all sequences (b16) or a fixed sample of them."""
    case = wl.make_config(name)
    note(f"decode full config {name} rows={rows}")
    out = run_decode(sk, case)
    ref = _oracle(case, rows)
    sel = list(range(case.B)) if rows is None else rows
    assert torch.isfinite(out.float()).all()
    assert_parity(out[sel], ref[sel], f"{name} rows={rows}")


@pytest.mark.parametrize("name,rows", [("decode_b16", None), ("tiny", None),
                                       ("decode_b64", [0, 31, 63]), ("long_b20", [7])])
def test_fused_path_full_size(sk, name, rows):
    """The fused split + merge kernel on full workloads (its grid capped at
    the resident work groups), all or sampled rows."""
    case = wl.make_config(name)
    t = decode_tensors(case)
    msl = int(case.cache.seq_lens.max())
    note(f"decode fused step {name}")
    out = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                         t["seq_lens"], msl, case.scale, launches=2)
    torch.cuda.synchronize()
    sel = list(range(case.B)) if rows is None else rows
    assert_parity(out[sel], _oracle(case, rows)[sel], f"fused {name}")


def test_fused_step_repeats_and_resets(sk):
    """The fused step's counters are cleared by each call's q projection: many
    calls in a row on one workspace, with batches of different sizes, stay
    bit-identical to the first call of each batch."""
    a = wl.make_decode_case(wl.MAIN, seq_lens=[900, 33, 2048, 5], seed=29)
    b = wl.make_decode_case(wl.MAIN, seq_lens=[4000], seed=30)
    ta, tb_ = decode_tensors(a), decode_tensors(b)
    dims = sk.dims_of(ta["k_cache"], ta["v_cache"], ta["U"], ta["W"])
    need = max(sk.decode_workspace_size(dims, 4, 2048, launches=2),
               sk.decode_workspace_size(dims, 1, 4000, launches=2))
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # garbage to start
    note("decode fused step repeated with one workspace")
    outs_a, outs_b = [], []
    for i in range(6):
        for case, t, outs in ((a, ta, outs_a), (b, tb_, outs_b)):
            o = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"],
                               t["block_tables"], t["seq_lens"], int(case.cache.seq_lens.max()),
                               case.scale, workspace=ws, launches=2)
            outs.append(o.clone())
    torch.cuda.synchronize()
    for outs in (outs_a, outs_b):
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert_parity(outs_a[0], _oracle(a), "fused repeat a")
    assert_parity(outs_b[0], _oracle(b), "fused repeat b")


def test_decode_one_million_tokens(sk):
    """One sequence of 2^20 tokens (65536 pages: the planner's largest split,
    256 pages, and 256 splits merged by the wide merge tiles), tiny shape;
    a planted key pair in the middle page keeps the output away from zero."""
    case = wl.make_decode_case(wl.TINY, seq_lens=[1 << 20], seed=33, plant=("mid",), q_mult=4)
    note("decode 2^20 tokens, tiny shape")
    out = run_decode(sk, case)
    assert_parity(out, _oracle(case), "2^20 tokens")


def test_decode_4096_short_sequences(sk):
    """4096 sequences of 0-299 tokens in one call (tiny shape): a grid 4096
    rows tall, empty sequences among them."""
    rng = np.random.default_rng(34)
    lens = rng.integers(0, 300, size=4096).tolist()
    case = wl.make_decode_case(wl.TINY, seq_lens=lens, seed=34)
    note("decode 4096 short sequences, tiny shape")
    out = run_decode(sk, case)
    assert_parity(out, _oracle(case), "4096 sequences")
    empty = [b for b, L in enumerate(lens) if L == 0]
    assert empty and torch.count_nonzero(out[empty]).item() == 0

"""GPU parity of the grouped-query layouts (H query heads on Hkv key/value
heads; U, the key latents and W's rows per key/value head) against the fp64
oracle, through the C ABI: decode, chunked prefill and the append.  The bars
are the multi-head ones: attention within max-abs 2e-3 and rel-L2 1e-3,
append latents within one fp16 ulp (or the fp32 summation allowance near
zero), index work bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, dev, note, run_decode
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def _oracle_decode(case, rows=None):
    c = case.cache
    return oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                         c.seq_lens, case.scale, batch_indices=rows)


def test_decode_tiny_gqa_config(sk):
    case = wl.make_config("tiny_gqa")
    note("gqa decode tiny_gqa config")
    assert_parity(run_decode(sk, case), _oracle_decode(case), "tiny_gqa")


@pytest.mark.parametrize("lens", [[1, 17, 300], [16, 15, 33, 64, 2], [0, 1, 4097, 31]],
                         ids=["short", "page_edges", "long_and_empty"])
def test_decode_gqa8_ragged(sk, lens):
    case = wl.make_decode_case(wl.GQA8, seq_lens=lens, seed=61, extra_cols=3)
    note(f"gqa decode gqa8 lens={lens}")
    out = run_decode(sk, case)
    assert_parity(out, _oracle_decode(case), f"gqa8 {lens}")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def test_decode_tiny_gqa_ragged(sk):
    case = wl.make_decode_case(wl.TINY_GQA, seq_lens=[3, 0, 16, 17, 250], seed=62)
    note("gqa decode tiny ragged")
    assert_parity(run_decode(sk, case), _oracle_decode(case), "tiny_gqa ragged")


def test_decode_gqa8_block_table_permutation_is_bit_identical(sk):
    lens = [40, 513, 7]
    a = wl.make_decode_case(wl.GQA8, seq_lens=lens, seed=63, shuffle=True)
    b = wl.make_decode_case(wl.GQA8, seq_lens=lens, seed=63, shuffle=False)
    assert not np.array_equal(a.cache.block_tables, b.cache.block_tables)
    note("gqa decode gqa8 permutation")
    oa, ob = run_decode(sk, a), run_decode(sk, b)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_decode_gqa_equals_expanded_mha(sk):
    """The grouped-query kernels on Hkv heads against the multi-head kernels
    on the same data expanded to H heads (each key/value head's U, key
    latents and W rows repeated for its query heads): both must match the
    oracle, and each other within the same bar."""
    case = wl.make_decode_case(wl.GQA8, seq_lens=[200, 1031], seed=64)
    G = wl.GQA8.H // wl.GQA8.kv
    c = case.cache
    U_x = np.repeat(case.U, G, axis=0)
    kc_x = np.repeat(c.k_cache, G, axis=1)
    W_x = np.repeat(case.W.reshape(wl.GQA8.kv, wl.GQA8.d, -1), G, axis=0).reshape(
        wl.GQA8.H * wl.GQA8.d, -1)
    note("gqa decode vs expanded mha")
    out_g = run_decode(sk, case)
    out_m = sk.decode_attn(dev(case.q), dev(kc_x), dev(c.v_cache), dev(U_x), dev(W_x),
                           dev(c.block_tables), dev(c.seq_lens), int(c.seq_lens.max()),
                           case.scale)
    torch.cuda.synchronize()
    ref = _oracle_decode(case)
    assert_parity(out_g, ref, "gqa kernels")
    assert_parity(out_m, ref, "expanded mha kernels")
    assert_parity(out_g, out_m.float().cpu().numpy(), "gqa vs expanded mha")


@pytest.mark.parametrize("name,rows", [("gqa8_b16", None), ("gqa8_b64", [0, 31, 63])])
def test_decode_gqa8_full_size(sk, name, rows):
    case = wl.make_config(name)
    note(f"gqa decode full config {name} rows={rows}")
    out = run_decode(sk, case)
    ref = _oracle_decode(case, rows)
    sel = list(range(case.B)) if rows is None else rows
    assert torch.isfinite(out.float()).all()
    assert_parity(out[sel], ref[sel], f"{name} rows={rows}")


def _gpu_prefill(sk, case):
    c = case.cache
    tk, tv = dev(c.k_cache), dev(c.v_cache)
    U, W = dev(case.U), dev(case.W)
    sk.append(dev(case.k_new), dev(case.v_new), U, W, dev(case.slot_mapping), tk, tv)
    chunk = np.diff(case.query_start_loc)
    out = sk.prefill_attn(dev(case.q), dev(case.query_start_loc), int(chunk.max()), tk, tv, U,
                          W, dev(c.block_tables), dev(c.seq_lens), int(c.seq_lens.max()),
                          case.scale)
    torch.cuda.synchronize()
    return out, tk.cpu().numpy(), tv.cpu().numpy()


def _oracle_prefill(case, kc, vc, rows=None):
    return oracle.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                          case.cache.block_tables, case.cache.seq_lens, case.scale,
                          request_indices=rows)


@pytest.mark.parametrize("shape,cached,chunk", [
    (wl.TINY_GQA, [20, 0, 7], [5, 16, 33]),
    (wl.GQA8, [37, 100], [20, 45]),
    (wl.GQA8, [0, 15, 64], [1, 17, 70]),
], ids=["tiny_gqa", "gqa8_ragged", "gqa8_edges"])
def test_prefill_gqa(sk, shape, cached, chunk):
    case = wl.make_prefill_case(shape, cached, chunk, seed=65)
    note(f"gqa prefill {shape} cached={cached} chunk={chunk}")
    out, kc, vc = _gpu_prefill(sk, case)
    assert_parity(out, _oracle_prefill(case, kc, vc), "gqa prefill (gpu caches)")
    okc, ovc = oracle.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                             case.cache.k_cache, case.cache.v_cache)
    assert_parity(out, _oracle_prefill(case, okc, ovc), "gqa prefill (oracle caches)")


def test_prefill_gqa8_full_size_sampled(sk):
    case = wl.make_config("gqa8_prefill_b16")
    note("gqa prefill full config gqa8_prefill_b16")
    out, kc, vc = _gpu_prefill(sk, case)
    rows = [0, 7, 15]
    ref = _oracle_prefill(case, kc, vc, rows=rows)
    sel = np.concatenate([np.arange(case.query_start_loc[r], case.query_start_loc[r + 1])
                          for r in rows])
    assert torch.isfinite(out.float()).all()
    assert_parity(out[torch.from_numpy(sel).cuda()], ref[sel], "gqa8_prefill_b16 sample")


def _ulp_diff(a, b):
    ai = a.view(np.int16).astype(np.int32)
    bi = b.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -32768 - ai, ai)
    bi = np.where(bi < 0, -32768 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("shape,n,seed", [(wl.GQA8, 16, 66), (wl.GQA8, 300, 67),
                                          (wl.TINY_GQA, 40, 68)],
                         ids=["gqa8_decode_step", "gqa8_300", "tiny_gqa_40"])
def test_append_gqa(sk, shape, n, seed):
    """The append runs on the key/value heads: k, v [n, Hkv, d]."""
    rng = np.random.default_rng(seed)
    U, W = wl.draw_bases(rng, shape)
    nb = (n + shape.bs - 1) // shape.bs + 2
    slots = rng.permutation(nb * shape.bs)[:n].astype(np.int64)
    k = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    kc = wl._nan_f16((nb, shape.kv, shape.bs, shape.r_k))
    vc = wl._nan_f16((nb, shape.r_v, shape.bs))
    note(f"gqa append {shape} n={n}")
    tk, tv = dev(kc), dev(vc)
    sk.append(dev(k), dev(v), dev(U), dev(W), dev(slots), tk, tv)
    torch.cuda.synchronize()
    gk, gv = tk.cpu().numpy(), tv.cpu().numpy()
    rk, rv = oracle.append(k, v, U, W, slots, kc, vc)
    assert np.array_equal(np.isnan(gk), np.isnan(rk))
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    # the tuned append's allowances (twice the measured fp32 summation error)
    for g, r, atol, what in ((gk, rk, 5e-7, "k"), (gv, rv, 5e-6, "v")):
        m = ~np.isnan(r)
        u = _ulp_diff(g[m], r[m])
        a = np.abs(g[m].astype(np.float64) - r[m].astype(np.float64))
        print(f"[parity] gqa append {what}: max ulp {u.max(initial=0)} max abs "
              f"{a.max(initial=0):.2e}; beyond 1 ulp: max abs {a[u > 1].max(initial=0):.3e}",
              flush=True)
        assert ((u <= 1) | (a <= atol)).all()

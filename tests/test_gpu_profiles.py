"""GPU parity of a second rank profile of the main shape, (r_k, r_v) =
(32, 256) next to the benchmark's (64, 512): per-layer ranks may differ, so
every entry point has an instance for each.  Bars as for the main profile:
attention within max-abs 2e-3 and rel-L2 1e-3, append latents within one
fp16 ulp (or the fp32 summation allowance near zero)."""
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


@pytest.mark.parametrize("lens", [[1, 17, 300], [0, 16, 4097, 31]], ids=["short", "long_and_empty"])
def test_decode_lowrank_ragged(sk, lens):
    case = wl.make_decode_case(wl.LOWRANK, seq_lens=lens, seed=71, extra_cols=2)
    note(f"lowrank decode lens={lens}")
    out = run_decode(sk, case)
    assert_parity(out, _oracle_decode(case), f"lowrank {lens}")


def test_decode_lowrank_b16(sk):
    case = wl.make_config("lowrank_b16")
    note("lowrank decode lowrank_b16")
    out = run_decode(sk, case)
    assert torch.isfinite(out.float()).all()
    assert_parity(out, _oracle_decode(case), "lowrank_b16")


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


def test_prefill_lowrank(sk):
    case = wl.make_prefill_case(wl.LOWRANK, [0, 15, 64], [1, 17, 70], seed=72)
    note("lowrank prefill edges")
    out, kc, vc = _gpu_prefill(sk, case)
    assert_parity(out, _oracle_prefill(case, kc, vc), "lowrank prefill (gpu caches)")
    okc, ovc = oracle.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                             case.cache.k_cache, case.cache.v_cache)
    assert_parity(out, _oracle_prefill(case, okc, ovc), "lowrank prefill (oracle caches)")


def test_prefill_lowrank_full_size_sampled(sk):
    case = wl.make_config("lowrank_prefill_b16")
    note("lowrank prefill full config")
    out, kc, vc = _gpu_prefill(sk, case)
    rows = [0, 15]
    ref = _oracle_prefill(case, kc, vc, rows=rows)
    sel = np.concatenate([np.arange(case.query_start_loc[r], case.query_start_loc[r + 1])
                          for r in rows])
    assert torch.isfinite(out.float()).all()
    assert_parity(out[torch.from_numpy(sel).cuda()], ref[sel], "lowrank_prefill_b16 sample")


def _ulp_diff(a, b):
    ai = a.view(np.int16).astype(np.int32)
    bi = b.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -32768 - ai, ai)
    bi = np.where(bi < 0, -32768 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("n,seed", [(16, 73), (300, 74)], ids=["decode_step", "chunk_300"])
def test_append_lowrank(sk, n, seed):
    shape = wl.LOWRANK
    rng = np.random.default_rng(seed)
    U, W = wl.draw_bases(rng, shape)
    nb = (n + shape.bs - 1) // shape.bs + 2
    slots = rng.permutation(nb * shape.bs)[:n].astype(np.int64)
    k = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    kc = wl._nan_f16((nb, shape.kv, shape.bs, shape.r_k))
    vc = wl._nan_f16((nb, shape.r_v, shape.bs))
    note(f"lowrank append n={n}")
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
        print(f"[parity] lowrank append {what}: max ulp {u.max(initial=0)} max abs "
              f"{a.max(initial=0):.2e}; beyond 1 ulp: max abs {a[u > 1].max(initial=0):.3e}",
              flush=True)
        assert ((u <= 1) | (a <= atol)).all()

"""GPU parity of chunked-prefill attention (append, q projection, causal
latent attention, up-projection) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, dev, note
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def _gpu_prefill(sk, case, q=None, k_new=None, v_new=None):
    c = case.cache
    tk, tv = dev(c.k_cache), dev(c.v_cache)
    U, W = dev(case.U), dev(case.W)
    kn = case.k_new if k_new is None else k_new
    vn = case.v_new if v_new is None else v_new
    sk.append(dev(kn), dev(vn), U, W, dev(case.slot_mapping), tk, tv)
    chunk = np.diff(case.query_start_loc)
    msl = int(c.seq_lens.max())
    out = sk.prefill_attn(dev(case.q if q is None else q), dev(case.query_start_loc),
                          int(chunk.max()), tk, tv, U, W, dev(c.block_tables), dev(c.seq_lens),
                          msl, case.scale)
    torch.cuda.synchronize()
    return out, tk.cpu().numpy(), tv.cpu().numpy()


def _oracle(case, kc, vc, rows=None, q=None):
    return oracle.prefill(case.q if q is None else q, case.query_start_loc, kc, vc, case.U,
                          case.W, case.cache.block_tables, case.cache.seq_lens, case.scale,
                          request_indices=rows)


@pytest.mark.parametrize("shape,cached,chunk", [
    (wl.TINY, [20, 0, 7], [5, 16, 33]),
    (wl.MAIN, [37, 100], [20, 45]),
    (wl.MAIN, [0, 15, 64], [1, 17, 70]),
], ids=["tiny", "main_ragged", "main_edges"])
def test_prefill_matches_oracle(sk, shape, cached, chunk):
    case = wl.make_prefill_case(shape, cached, chunk, seed=41)
    note(f"prefill {shape} cached={cached} chunk={chunk}")
    out, kc, vc = _gpu_prefill(sk, case)
    # attention-only parity: the oracle reads the caches the GPU appended
    assert_parity(out, _oracle(case, kc, vc), "prefill (gpu caches)")
    # end to end: oracle append + oracle attention
    okc, ovc = oracle.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                             case.cache.k_cache, case.cache.v_cache)
    assert_parity(out, _oracle(case, okc, ovc), "prefill (oracle caches)")


def test_prefill_causal_future_tokens_do_not_leak(sk):
    """Changing the last chunk token's q, k and v leaves every earlier query's
    output bit-identical."""
    case = wl.make_prefill_case(wl.MAIN, [50, 10], [40, 33], seed=42)
    note("prefill causality")
    out1, _, _ = _gpu_prefill(sk, case)
    q2, k2, v2 = case.q.copy(), case.k_new.copy(), case.v_new.copy()
    for b in range(2):
        last = case.query_start_loc[b + 1] - 1
        rng = np.random.default_rng(99 + b)
        for arr in (q2, k2, v2):
            arr[last] = rng.standard_normal(arr[last].shape).astype(np.float16)
    out2, _, _ = _gpu_prefill(sk, case, q=q2, k_new=k2, v_new=v2)
    keep = np.ones(case.q.shape[0], bool)
    keep[case.query_start_loc[1:] - 1] = False
    keep_t = torch.from_numpy(keep).cuda()
    assert torch.equal(out1[keep_t].view(torch.int16), out2[keep_t].view(torch.int16))
    assert not torch.equal(out1[~keep_t].view(torch.int16), out2[~keep_t].view(torch.int16))


def test_prefill_full_size_sampled(sk):
    """prefill_b16 in the benchmark's launch configuration; oracle on a
    fixed sample of requests."""
    case = wl.make_config("prefill_b16")
    note("prefill full config prefill_b16")
    out, kc, vc = _gpu_prefill(sk, case)
    rows = [0, 2, 5, 7, 9, 11, 13, 15]
    ref = _oracle(case, kc, vc, rows=rows)
    sel = np.concatenate([np.arange(case.query_start_loc[r], case.query_start_loc[r + 1])
                          for r in rows])
    assert torch.isfinite(out.float()).all()
    assert_parity(out[torch.from_numpy(sel).cuda()], ref[sel], "prefill_b16 sample")


@pytest.mark.parametrize("shape", [wl.TINY, wl.MAIN], ids=["tiny", "main"])
def test_prefill_long_prefix_and_many_requests(sk, shape):
    """A request with a long cached prefix beside an empty-prefix one and a
    single-token chunk (tiny shape: 131072 cached tokens; main shape: 16384),
    then 64 requests of mixed lengths in one call."""
    long = 131072 if shape is wl.TINY else 16384
    case = wl.make_prefill_case(shape, [long, 0, 5000], [64, 300, 1], seed=44)
    note(f"prefill long prefix {shape}")
    out, kc, vc = _gpu_prefill(sk, case)
    assert_parity(out, _oracle(case, kc, vc), "long prefix (gpu caches)")
    rng = np.random.default_rng(45)
    cached = rng.integers(0, 600, size=64).tolist()
    chunk = rng.integers(1, 90, size=64).tolist()
    case = wl.make_prefill_case(shape, cached, chunk, seed=45)
    note(f"prefill 64 requests {shape}")
    out, kc, vc = _gpu_prefill(sk, case)
    assert_parity(out, _oracle(case, kc, vc), "64 requests (gpu caches)")

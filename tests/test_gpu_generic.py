"""GPU parity of the generic instances, which take any shape within their
limits at run time (d a multiple of 32 up to 256; r_k a multiple of 8 up to
min(d, 256); r_v a multiple of 8 up to min(2048, Hkv d); Hkv dividing H):
odd head counts and head sizes, per-layer rank profiles from r_k 16 to 128 and
r_v 128 to 2048 (the README's learned per-layer ranks and its three profiles),
grouped-query groups of 2 and 8, and FP8 caches on profiles without a tuned FP8
instance.  Same bars as the tuned kernels: max-abs 2e-3 and rel-L2 1e-3
against the fp64 oracle, per (row, head) rel-L2 1e-3, bit-identical output
under a shuffled block table, append latents within one fp16 ulp (or the
fp32 summation allowance near zero) in exactly the listed slots."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, dev, note, run_decode
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu

S = wl.Shape
SHAPES = {
    "odd_h28_d96": S(H=28, d=96, r_k=48, r_v=640),
    "gqa_g2": S(H=32, d=128, r_k=64, r_v=512, Hkv=16),
    "gqa_g8": S(H=32, d=128, r_k=64, r_v=512, Hkv=4),
    "rank_16_128": S(H=32, d=128, r_k=16, r_v=128),
    "rank_48_384": S(H=32, d=128, r_k=48, r_v=384),
    "rank_96_768": S(H=32, d=128, r_k=96, r_v=768),
    "conservative_128_1024": S(H=32, d=128, r_k=128, r_v=1024),
    "d256": S(H=8, d=256, r_k=128, r_v=1024),
    "h3_d32_gqa": S(H=6, d=32, r_k=8, r_v=40, Hkv=3),
    # r_v past 1024: the split kernel's wide instances (16 feature tiles per wave)
    "wide_v_2048": S(H=16, d=128, r_k=32, r_v=2048),
}
# the profiles that also run FP8 caches on the generic kernels
FP8_SHAPES = ["odd_h28_d96", "rank_96_768", "gqa_g2", "wide_v_2048"]


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def per_head(y, ref, what, bar=1e-3):
    y = y.float().cpu().numpy().astype(np.float64)
    e = np.linalg.norm(y - ref, axis=-1)
    n = np.linalg.norm(ref, axis=-1)
    ok = n > 0
    worst = float((e[ok] / n[ok]).max()) if ok.any() else 0.0
    print(f"[per-head] {what}: worst rel_l2 {worst:.3e}", flush=True)
    assert worst <= bar


def _dec_oracle(case):
    c = case.cache
    kc, vc = c.k_cache, c.v_cache
    if kc.dtype == np.uint8:
        kc = oracle.dequantize_cache(kc, case.k_scale)
        vc = oracle.dequantize_cache(vc, case.v_scale)
    return oracle.decode(case.q, kc, vc, case.U, case.W, c.block_tables, c.seq_lens, case.scale)


def _run_dec(sk, case, **kw):
    c = case.cache
    if c.k_cache.dtype == np.uint8:
        out = sk.decode_attn_fp8(dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U),
                                 dev(case.W), dev(c.block_tables), dev(c.seq_lens),
                                 int(max(c.seq_lens.max(), 1)), case.k_scale, case.v_scale,
                                 case.scale)
        torch.cuda.synchronize()
        return out
    if kw:
        out = sk.decode_attn(dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U),
                             dev(case.W), dev(c.block_tables), dev(c.seq_lens),
                             int(max(c.seq_lens.max(), 1)), case.scale, **kw)
        torch.cuda.synchronize()
        return out
    return run_decode(sk, case)


def test_generic_shapes_are_supported(sk):
    for name, sh in SHAPES.items():
        d = sk.make_dims(sh.H, sh.d, sh.r_k, sh.r_v, 4, num_kv_heads=0 if sh.kv == sh.H else sh.kv)
        assert sk.shape_supported(d), name


@pytest.mark.parametrize("name", list(SHAPES))
def test_generic_decode(sk, name):
    sh = SHAPES[name]
    lens = [0, 1, 15, 16, 17, 300, 4097]
    case = wl.make_decode_case(sh, seq_lens=lens, seed=101, extra_cols=2)
    note(f"generic decode {name} lens={lens}")
    out = _run_dec(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"generic decode {name}")
    per_head(out, ref, f"generic decode {name}")
    assert torch.count_nonzero(out[0]).item() == 0


@pytest.mark.parametrize("name", ["odd_h28_d96", "conservative_128_1024", "gqa_g8"])
def test_generic_decode_scaled_queries(sk, name):
    """Sharp rows: queries x16 (scores tens of units apart)."""
    case = wl.make_decode_case(SHAPES[name], seq_lens=[2048, 333], seed=102, q_mult=16)
    note(f"generic decode {name} q x16")
    out = _run_dec(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"generic decode {name} q x16")
    per_head(out, ref, f"generic decode {name} q x16")


@pytest.mark.parametrize("pps", [1, 7, 256])
def test_generic_decode_split_plans(sk, pps):
    """Any split plan (one split, many, one page each) within the bars."""
    case = wl.make_decode_case(SHAPES["odd_h28_d96"], seq_lens=[1500, 40, 2], seed=103)
    note(f"generic decode split plan pps={pps}")
    out = _run_dec(sk, case, pages_per_split=pps)
    assert_parity(out, _dec_oracle(case), f"generic plan pps={pps}")


def test_generic_decode_small_batch_long(sk):
    """Batch 1 over 20000 tokens: the plan spreads one sequence over many
    splits, merged in one pass."""
    case = wl.make_decode_case(SHAPES["rank_96_768"], seq_lens=[20000], seed=104)
    note("generic decode batch 1 x 20000")
    out = _run_dec(sk, case)
    assert_parity(out, _dec_oracle(case), "generic b1 long")


@pytest.mark.parametrize("name,batch", [("odd_h28_d96", 42), ("conservative_128_1024", 9)],
                         ids=["rows_of_4", "rows_of_2"])
def test_generic_decode_merge_row_tiles(sk, name, batch):
    """Batches whose (row, head) pairs reach 1024 (odd_h28 x 42: the merge
    takes four rows per work group, the last block two) or 256
    (conservative x 9: two rows, the last block one), ragged lengths
    including empty rows."""
    rng = np.random.default_rng(120 + batch)
    lens = [int(x) for x in rng.integers(0, 200, size=batch)]
    lens[3] = 0
    case = wl.make_decode_case(SHAPES[name], seq_lens=lens, seed=121)
    note(f"generic decode merge rows {name} B={batch}")
    out = _run_dec(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"generic merge rows {name}")
    per_head(out, ref, f"generic merge rows {name}")
    assert torch.count_nonzero(out[3]).item() == 0


def test_generic_block_table_permutation_is_bit_identical(sk):
    lens = [40, 513, 7]
    sh = SHAPES["gqa_g2"]
    a = wl.make_decode_case(sh, seq_lens=lens, seed=105, shuffle=True)
    b = wl.make_decode_case(sh, seq_lens=lens, seed=105, shuffle=False)
    assert not np.array_equal(a.cache.block_tables, b.cache.block_tables)
    note("generic decode shuffled vs identity block table")
    oa, ob = _run_dec(sk, a), _run_dec(sk, b)
    assert_parity(oa, _dec_oracle(a), "generic shuffled")
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


@pytest.mark.parametrize("name", FP8_SHAPES + ["lowrank"])
def test_generic_decode_fp8(sk, name):
    sh = wl.LOWRANK if name == "lowrank" else SHAPES[name]
    case = wl.make_decode_case(sh, seq_lens=[0, 17, 300, 2049], seed=106, fp8=True)
    note(f"generic decode fp8 {name}")
    out = _run_dec(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"generic decode fp8 {name}")
    per_head(out, ref, f"generic decode fp8 {name}")


def test_generic_decode_noalloc(sk):
    case = wl.make_decode_case(SHAPES["odd_h28_d96"], seq_lens=[700, 5, 0], seed=107)
    c = case.cache
    note("generic decode noalloc")
    ref_out = _run_dec(sk, case)
    out = torch.full_like(ref_out, float("nan"))
    sk.decode_attn_noalloc(dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U), dev(case.W),
                           dev(c.block_tables), dev(c.seq_lens), int(c.seq_lens.max()), out,
                           case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


# ---------------------------------------------------------------- prefill
def _gpu_prefill(sk, case):
    c = case.cache
    fp8 = c.k_cache.dtype == np.uint8
    tk, tv = dev(c.k_cache), dev(c.v_cache)
    U, W = dev(case.U), dev(case.W)
    chunk = np.diff(case.query_start_loc)
    msl = int(c.seq_lens.max())
    if fp8:
        sk.append_fp8(dev(case.k_new), dev(case.v_new), U, W, dev(case.slot_mapping),
                      case.k_scale, case.v_scale, tk, tv)
        out = sk.prefill_attn_fp8(dev(case.q), dev(case.query_start_loc), int(chunk.max()), tk,
                                  tv, U, W, dev(c.block_tables), dev(c.seq_lens), msl,
                                  case.k_scale, case.v_scale, case.scale)
    else:
        sk.append(dev(case.k_new), dev(case.v_new), U, W, dev(case.slot_mapping), tk, tv)
        out = sk.prefill_attn(dev(case.q), dev(case.query_start_loc), int(chunk.max()), tk, tv,
                              U, W, dev(c.block_tables), dev(c.seq_lens), msl, case.scale)
    torch.cuda.synchronize()
    return out, tk.cpu().numpy(), tv.cpu().numpy()


def _pre_oracle(case, kc, vc):
    if kc.dtype == np.uint8:
        kc = oracle.dequantize_cache(kc, case.k_scale)
        vc = oracle.dequantize_cache(vc, case.v_scale)
    return oracle.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                          case.cache.block_tables, case.cache.seq_lens, case.scale)


@pytest.mark.parametrize("name", list(SHAPES))
def test_generic_prefill(sk, name):
    case = wl.make_prefill_case(SHAPES[name], [0, 15, 130], [1, 17, 40], seed=111)
    note(f"generic prefill {name}")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"generic prefill {name} (gpu caches)")
    per_head(out, ref, f"generic prefill {name}")
    okc, ovc = oracle.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                             case.cache.k_cache, case.cache.v_cache)
    assert_parity(out, _pre_oracle(case, okc, ovc), f"generic prefill {name} (oracle caches)")


def test_generic_prefill_many_chunk_tokens(sk):
    """290 chunk tokens: the q projection takes 64 tokens per work group."""
    case = wl.make_prefill_case(SHAPES["odd_h28_d96"], [30, 7], [200, 90], seed=123)
    note("generic prefill 290 chunk tokens")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, "generic prefill 290 tokens")
    per_head(out, ref, "generic prefill 290 tokens")


def test_generic_prefill_long_prefix_reads_table(sk):
    """9000 cached tokens (more than 512 pages): the tiled prefill kernel
    stages all of a request's block ids in LDS, up to 8192 pages."""
    case = wl.make_prefill_case(SHAPES["h3_d32_gqa"], [9000, 40], [20, 9], seed=122)
    assert case.cache.block_tables.shape[1] > 512
    note("generic prefill over 9000 cached tokens")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, "generic prefill long prefix")
    per_head(out, ref, "generic prefill long prefix")


def test_generic_prefill_table_past_lds_ids(sk):
    """A table row longer than 8192 pages (132000 cached tokens) does not fit
    the tiled kernel's staged block ids: the call runs on the row kernel,
    which reads the block ids from the table page by page."""
    case = wl.make_prefill_case(SHAPES["h3_d32_gqa"], [132000, 40], [20, 9], seed=124)
    assert case.cache.block_tables.shape[1] > 8192
    note("generic prefill over 132000 cached tokens")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, "generic prefill table past 8192 pages")
    per_head(out, ref, "generic prefill table past 8192 pages")


@pytest.mark.parametrize("name", ["odd_h28_d96", "gqa_g8"])
def test_generic_prefill_sharp_rows(sk, name):
    """Queries x16, and key latents ramped along the request."""
    case = wl.make_prefill_case(SHAPES[name], [300, 64], [40, 33], seed=112, q_mult=16)
    note(f"generic prefill {name} q x16")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"generic prefill {name} q x16")
    per_head(out, ref, f"generic prefill {name} q x16")
    case = wl.make_prefill_case(SHAPES[name], [500, 90], [64, 70], seed=113, q_mult=2, ramp=30.0)
    note(f"generic prefill {name} rising")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"generic prefill {name} rising")
    per_head(out, ref, f"generic prefill {name} rising")


@pytest.mark.parametrize("name", FP8_SHAPES + ["lowrank"])
def test_generic_prefill_fp8(sk, name):
    sh = wl.LOWRANK if name == "lowrank" else SHAPES[name]
    case = wl.make_prefill_case(sh, [64, 7], [33, 20], seed=114, fp8=True)
    note(f"generic prefill fp8 {name}")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"generic prefill fp8 {name}")
    per_head(out, ref, f"generic prefill fp8 {name}")


def test_generic_prefill_causal_future_tokens_do_not_leak(sk):
    case = wl.make_prefill_case(SHAPES["odd_h28_d96"], [50, 10], [40, 33], seed=115)
    note("generic prefill causality")
    out1, _, _ = _gpu_prefill(sk, case)
    last = case.query_start_loc[1:] - 1
    for arr in (case.q, case.k_new, case.v_new):
        for i, n in enumerate(last):
            arr[n] = np.random.default_rng(7 + i).standard_normal(arr[n].shape).astype(np.float16)
    out2, _, _ = _gpu_prefill(sk, case)
    keep = np.ones(case.q.shape[0], bool)
    keep[last] = False
    keep_t = torch.from_numpy(keep).cuda()
    assert torch.equal(out1[keep_t].view(torch.int16), out2[keep_t].view(torch.int16))
    assert not torch.equal(out1[~keep_t].view(torch.int16), out2[~keep_t].view(torch.int16))


# ---------------------------------------------------------------- append
def _ulp_diff(a, b):
    ai = a.view(np.int16).astype(np.int32)
    bi = b.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -32768 - ai, ai)
    bi = np.where(bi < 0, -32768 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("n", [16, 300])
@pytest.mark.parametrize("name", ["odd_h28_d96", "gqa_g2", "conservative_128_1024", "h3_d32_gqa"])
def test_generic_append(sk, name, n):
    """The tiled append on the key/value heads of a generic shape: exactly the
    listed slots written (NaN sentinels elsewhere), latents within one fp16
    ulp of the oracle's or within the fp32 summation allowance near zero
    (K = d for keys, Hkv d for values)."""
    sh = SHAPES[name]
    rng = np.random.default_rng(121)
    U, W = wl.draw_bases(rng, sh)
    nb = (n + 15) // 16 + 3
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[::7] = -1
    k = rng.standard_normal((n, sh.kv, sh.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, sh.kv, sh.d), dtype=np.float32).astype(np.float16)
    kc = wl._nan_f16((nb, sh.kv, 16, sh.r_k))
    vc = wl._nan_f16((nb, sh.r_v, 16))
    note(f"generic append {name} n={n}")
    tk, tv = dev(kc), dev(vc)
    sk.append(dev(k), dev(v), dev(U), dev(W), dev(slots), tk, tv)
    torch.cuda.synchronize()
    gk, gv = tk.cpu().numpy(), tv.cpu().numpy()
    rk, rv = oracle.append(k, v, U, W, slots, kc, vc)
    assert np.array_equal(np.isnan(gk), np.isnan(rk))
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    for g, r, K, what in ((gk, rk, sh.d, "k"), (gv, rv, sh.kv * sh.d, "v")):
        m = ~np.isnan(r)
        u = _ulp_diff(g[m], r[m])
        a = np.abs(g[m].astype(np.float64) - r[m].astype(np.float64))
        atol = 5e-7 if what == "k" else 5e-6   # as the tuned append's allowances
        print(f"[parity] generic append {name} n={n} {what}: max ulp {u.max(initial=0)} "
              f"max abs {a.max(initial=0):.2e}; beyond 1 ulp: max abs "
              f"{a[u > 1].max(initial=0):.3e} (K {K})", flush=True)
        assert ((u <= 1) | (a <= atol)).all()

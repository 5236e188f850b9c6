"""GPU parity of the FP8 latent variant (OCP E4M3 codes with one scale per
tensor) against the fp64 oracle, through the C ABI.

Tolerance model: the variant is lossy only in the quantisation of the
latents.  Attention over given FP8 caches is compared with the oracle's
attention over the same caches dequantised (scale * value(code)), at the
multi-head bars (max-abs 2e-3, rel-L2 1e-3): the quantisation error is not
in that comparison.  The append's codes must equal the oracle's or be a
neighbouring code: the GPU divides an fp32 sum by the scale in fp32, the
oracle an fp64 one, so a value within rounding of the midpoint between two
codes may go either way.  The loss itself (FP8 against fp16 latents of the
same projections) is reported, bounded loosely by the format's half-step
relative error 2^-4."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, dev, errors, note
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def _run_fp8(sk, case, max_seq_len=None):
    c = case.cache
    msl = int(max(c.seq_lens.max(initial=0), 1)) if max_seq_len is None else max_seq_len
    out = sk.decode_attn_fp8(dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U),
                             dev(case.W), dev(c.block_tables), dev(c.seq_lens), msl,
                             case.k_scale, case.v_scale, case.scale)
    torch.cuda.synchronize()
    return out


def _oracle_fp8(case, kc8=None, vc8=None, rows=None):
    c = case.cache
    kc8 = c.k_cache if kc8 is None else kc8
    vc8 = c.v_cache if vc8 is None else vc8
    return oracle.decode(case.q, oracle.dequantize_cache(kc8, case.k_scale),
                         oracle.dequantize_cache(vc8, case.v_scale), case.U, case.W,
                         c.block_tables, c.seq_lens, case.scale, batch_indices=rows)


@pytest.mark.parametrize("shape,lens", [
    (wl.MAIN, [1, 17, 300]), (wl.MAIN, [0, 16, 4097, 31]), (wl.TINY, [3, 0, 16, 17, 250]),
    (wl.GQA8, [2, 64, 1031]),
], ids=["main_short", "main_long_and_empty", "tiny", "gqa8"])
def test_decode_fp8(sk, shape, lens):
    case = wl.make_decode_case(shape, seq_lens=lens, seed=81, extra_cols=2, fp8=True)
    note(f"fp8 decode {shape} lens={lens}")
    out = _run_fp8(sk, case)
    assert_parity(out, _oracle_fp8(case), f"fp8 {lens}")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


@pytest.mark.parametrize("name,rows", [("decode_b16_fp8", None), ("decode_b64_fp8", [0, 40, 63])])
def test_decode_fp8_full_size(sk, name, rows):
    case = wl.make_config(name)
    note(f"fp8 decode full config {name}")
    out = _run_fp8(sk, case)
    ref = _oracle_fp8(case, rows=rows)
    sel = list(range(case.B)) if rows is None else rows
    assert torch.isfinite(out.float()).all()
    assert_parity(out[sel], ref[sel], f"{name} rows={rows}")


def _code_rank(c):
    """Position of a code on the number line (monotone in value)."""
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


@pytest.mark.parametrize("shape,n,seed", [(wl.MAIN, 16, 82), (wl.MAIN, 300, 83),
                                          (wl.MAIN, 2000, 86), (wl.MAIN, 3000, 87),
                                          (wl.TINY, 40, 84), (wl.GQA8, 100, 85)],
                         ids=["main_16", "main_300_split4", "main_2000_split2",
                              "main_3000_unsplit", "tiny_40", "gqa8_100"])
def test_append_fp8(sk, shape, n, seed):
    """FP8 codes from every append form: one launch (16 tokens), the tiled
    kernel with its value contraction split four ways (300), two ways (2000)
    or not at all (3000), and the smaller shapes."""
    rng = np.random.default_rng(seed)
    U, W = wl.draw_bases(rng, shape)
    nb = (n + shape.bs - 1) // shape.bs + 2
    slots = rng.permutation(nb * shape.bs)[:n].astype(np.int64)
    slots[::7] = -1
    k = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    kc = np.full((nb, shape.kv, shape.bs, shape.r_k), wl.E4M3_NAN_CODE, np.uint8)
    vc = np.full((nb, shape.r_v, shape.bs), wl.E4M3_NAN_CODE, np.uint8)
    ks, vs = 0.25, 0.125
    note(f"fp8 append {shape} n={n}")
    tk, tv = dev(kc), dev(vc)
    sk.append_fp8(dev(k), dev(v), dev(U), dev(W), dev(slots), ks, vs, tk, tv)
    torch.cuda.synchronize()
    gk, gv = tk.cpu().numpy(), tv.cpu().numpy()
    rk, rv = oracle.append_fp8(k, v, U, W, slots, ks, vs, kc, vc)
    for g, r, what in ((gk, rk, "k"), (gv, rv, "v")):
        # exactly the listed slots were written
        assert np.array_equal(g == wl.E4M3_NAN_CODE, r == wl.E4M3_NAN_CODE), what
        m = r != wl.E4M3_NAN_CODE
        d = np.abs(_code_rank(g[m]) - _code_rank(r[m]))
        print(f"[parity] fp8 append {what}: {np.count_nonzero(d)} of {d.size} codes off by "
              f"one, max {d.max(initial=0)}", flush=True)
        assert d.max(initial=0) <= 1 and np.count_nonzero(d) <= max(4, d.size // 1000)


def test_fp8_end_to_end_and_loss(sk):
    """Append with FP8 then decode with FP8, against the oracle doing the
    same; and the quantisation loss against the fp16 path on the same
    tokens."""
    shape = wl.MAIN
    rng = np.random.default_rng(86)
    U, W = wl.draw_bases(rng, shape)
    lens = [300, 77]
    case16 = wl.make_decode_case(shape, seq_lens=lens, seed=87, bases=(U, W))
    n = sum(lens)
    k = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((n, shape.kv, shape.d), dtype=np.float32).astype(np.float16)
    bt = case16.cache.block_tables
    slots = np.concatenate([bt[b, np.arange(L) // 16].astype(np.int64) * 16 + np.arange(L) % 16
                            for b, L in enumerate(lens)])
    nb = case16.cache.k_cache.shape[0]
    ks, vs = 1.0 / 16, 1.0 / 16   # projections of N(0,1) inputs stay well inside +-448 * scale
    kc8 = np.full((nb, shape.kv, 16, shape.r_k), wl.E4M3_NAN_CODE, np.uint8)
    vc8 = np.full((nb, shape.r_v, 16), wl.E4M3_NAN_CODE, np.uint8)
    tk8, tv8 = dev(kc8), dev(vc8)
    tk16, tv16 = dev(case16.cache.k_cache), dev(case16.cache.v_cache)
    note("fp8 end to end")
    sk.append_fp8(dev(k), dev(v), dev(U), dev(W), dev(slots), ks, vs, tk8, tv8)
    sk.append(dev(k), dev(v), dev(U), dev(W), dev(slots), tk16, tv16)
    msl = max(lens)
    q, btd, sld = dev(case16.q), dev(bt), dev(case16.cache.seq_lens)
    out8 = sk.decode_attn_fp8(q, tk8, tv8, dev(U), dev(W), btd, sld, msl, ks, vs, case16.scale)
    out16 = sk.decode_attn(q, tk16, tv16, dev(U), dev(W), btd, sld, msl, case16.scale)
    torch.cuda.synchronize()
    g8 = tk8.cpu().numpy(), tv8.cpu().numpy()
    ref8 = oracle.decode(case16.q, oracle.dequantize_cache(g8[0], ks),
                         oracle.dequantize_cache(g8[1], vs), U, W, bt, case16.cache.seq_lens,
                         case16.scale)
    assert_parity(out8, ref8, "fp8 append + decode (oracle on the GPU's codes)")
    ma, rl = errors(out8.float().cpu().numpy(), out16.float().cpu().numpy())
    print(f"[loss] fp8 vs fp16 latents: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert rl < 2.0 ** -4


def _gpu_prefill_fp8(sk, case):
    c = case.cache
    tk, tv = dev(c.k_cache), dev(c.v_cache)
    U, W = dev(case.U), dev(case.W)
    sk.append_fp8(dev(case.k_new), dev(case.v_new), U, W, dev(case.slot_mapping), case.k_scale,
                  case.v_scale, tk, tv)
    chunk = np.diff(case.query_start_loc)
    out = sk.prefill_attn_fp8(dev(case.q), dev(case.query_start_loc), int(chunk.max()), tk, tv,
                              U, W, dev(c.block_tables), dev(c.seq_lens), int(c.seq_lens.max()),
                              case.k_scale, case.v_scale, case.scale)
    torch.cuda.synchronize()
    return out, tk.cpu().numpy(), tv.cpu().numpy()


def _oracle_prefill_fp8(case, kc8, vc8, rows=None):
    return oracle.prefill(case.q, case.query_start_loc, oracle.dequantize_cache(kc8, case.k_scale),
                          oracle.dequantize_cache(vc8, case.v_scale), case.U, case.W,
                          case.cache.block_tables, case.cache.seq_lens, case.scale,
                          request_indices=rows)


@pytest.mark.parametrize("shape,cached,chunk", [
    (wl.TINY, [20, 0, 7], [5, 16, 33]),
    (wl.MAIN, [0, 15, 64], [1, 17, 70]),
    (wl.GQA8, [37, 100], [20, 45]),
], ids=["tiny", "main_edges", "gqa8"])
def test_prefill_fp8(sk, shape, cached, chunk):
    case = wl.make_prefill_case(shape, cached, chunk, seed=88, fp8=True)
    note(f"fp8 prefill {shape} cached={cached} chunk={chunk}")
    out, kc8, vc8 = _gpu_prefill_fp8(sk, case)
    # attention over the GPU's caches, and end to end with the oracle's append
    assert_parity(out, _oracle_prefill_fp8(case, kc8, vc8), "fp8 prefill (gpu caches)")
    okc, ovc = oracle.append_fp8(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                                 case.k_scale, case.v_scale, case.cache.k_cache,
                                 case.cache.v_cache)
    assert_parity(out, _oracle_prefill_fp8(case, okc, ovc), "fp8 prefill (oracle caches)")


def test_prefill_fp8_full_size_sampled(sk):
    case = wl.make_config("prefill_b16_fp8")
    note("fp8 prefill full config prefill_b16_fp8")
    out, kc8, vc8 = _gpu_prefill_fp8(sk, case)
    rows = [0, 15]
    ref = _oracle_prefill_fp8(case, kc8, vc8, rows=rows)
    sel = np.concatenate([np.arange(case.query_start_loc[r], case.query_start_loc[r + 1])
                          for r in rows])
    assert torch.isfinite(out.float()).all()
    assert_parity(out[torch.from_numpy(sel).cuda()], ref[sel], "prefill_b16_fp8 sample")

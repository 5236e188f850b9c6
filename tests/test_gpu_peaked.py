"""GPU parity on sharp softmax rows, the method's hardest numerical case.

Scores of N(0,1) inputs spread by about 0.7 nats; trained models put tens of
nats between a row's largest scores.  These cases sharpen the rows with the
same draws (queries scaled by powers of two, a planted +/- key pair on the
first, middle or last page, key latents ramped along the sequence) and hold
the unchanged bars: max-abs 2e-3 and rel-L2 1e-3 over the output, and also
rel-L2 1e-3 per (row, head).

The prefill kernel raises a row's reference maximum lazily, only when a step's
maximum exceeds it by more than 8 (log2 units).  The ramped prefill cases are
built so that such raises happen after a row's first step; a CPU emulation of
that rule on the exact scores counts them and the test requires some.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, dev, errors, note, run_decode
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu

KRAISE = 8.0          # the prefill kernel's lazy-rescale threshold (log2 units)
STEP_TOKENS = 32      # tokens per prefill step (two 16-token pages)
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def per_head_check(y, ref, what, bar=1e-3):
    """rel-L2 of every (row, head) slice of [rows, H, d] outputs."""
    y = y.float().cpu().numpy().astype(np.float64) if isinstance(y, torch.Tensor) else y
    e = np.linalg.norm(y - ref, axis=-1)
    n = np.linalg.norm(ref, axis=-1)
    ok = n > 0
    worst = float((e[ok] / n[ok]).max()) if ok.any() else 0.0
    print(f"[per-head] {what}: worst rel_l2 {worst:.3e}", flush=True)
    assert worst <= bar, f"{what}: per-head rel_l2 {worst:.3e}"


def _dec_oracle(case):
    c = case.cache
    if case.k_scale != 1.0 or c.k_cache.dtype == np.uint8:
        kc = oracle.dequantize_cache(c.k_cache, case.k_scale)
        vc = oracle.dequantize_cache(c.v_cache, case.v_scale)
    else:
        kc, vc = c.k_cache, c.v_cache
    return oracle.decode(case.q, kc, vc, case.U, case.W, c.block_tables, c.seq_lens, case.scale)


def _run_decode(sk, case):
    if case.cache.k_cache.dtype == np.uint8:
        c = case.cache
        out = sk.decode_attn_fp8(dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U),
                                 dev(case.W), dev(c.block_tables), dev(c.seq_lens),
                                 int(c.seq_lens.max()), case.k_scale, case.v_scale, case.scale)
        torch.cuda.synchronize()
        return out
    return run_decode(sk, case)


DECODE_SHAPES = {"main": wl.MAIN, "tiny": wl.TINY, "gqa8": wl.GQA8, "lowrank": wl.LOWRANK,
                 "tiny_gqa": wl.TINY_GQA}


@pytest.mark.parametrize("mult", [4, 16, 32])
@pytest.mark.parametrize("shape", ["main", "tiny", "gqa8", "lowrank", "tiny_gqa"])
def test_decode_scaled_queries(sk, shape, mult):
    lens = [2048, 777, 4097, 33] if shape in ("main", "gqa8", "lowrank") else [256, 3, 100]
    case = wl.make_decode_case(DECODE_SHAPES[shape], seq_lens=lens, seed=61, q_mult=mult)
    note(f"peaked decode {shape} q x{mult} lens={lens}")
    out = _run_decode(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"decode {shape} q x{mult}")
    per_head_check(out, ref, f"decode {shape} q x{mult}")


@pytest.mark.parametrize("mult", [16, 32])
def test_decode_fp8_scaled_queries(sk, mult):
    case = wl.make_decode_case(wl.MAIN, seq_lens=[2048, 300, 17], seed=62, q_mult=mult, fp8=True)
    note(f"peaked decode fp8 q x{mult}")
    out = _run_decode(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"decode fp8 q x{mult}")
    per_head_check(out, ref, f"decode fp8 q x{mult}")


@pytest.mark.parametrize("where", ["first", "mid", "last"])
@pytest.mark.parametrize("shape", ["main", "gqa8", "tiny"])
def test_decode_planted_dominant_key(sk, shape, where):
    lens = [2048, 1000, 47] if shape != "tiny" else [256, 47]
    case = wl.make_decode_case(DECODE_SHAPES[shape], seq_lens=lens, seed=63, plant=(where,),
                               plant_factor=12.0, q_mult=2)
    note(f"peaked decode {shape} planted pair on the {where} page")
    out = _run_decode(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, f"decode {shape} planted {where}")
    per_head_check(out, ref, f"decode {shape} planted {where}")


def test_decode_rising_scores(sk):
    case = wl.make_decode_case(wl.MAIN, seq_lens=[3000, 513], seed=64, ramp=30.0, q_mult=2)
    note("peaked decode rising scores")
    out = _run_decode(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, "decode rising")
    per_head_check(out, ref, "decode rising")


def test_decode_full_b16_scaled(sk):
    """decode_b16's shape and launch configuration with queries scaled x16."""
    cfg = wl.CONFIGS["decode_b16"]
    case = wl.make_decode_case(wl.MAIN, B=16, seq=cfg["seq"], seed=65, q_mult=16)
    note("peaked decode b16 q x16")
    out = _run_decode(sk, case)
    ref = _dec_oracle(case)
    assert_parity(out, ref, "decode b16 q x16")
    per_head_check(out, ref, "decode b16 q x16")


# ---------------------------------------------------------------- prefill
def lazy_raises(case, kc):
    """Emulate the prefill kernel's lazy reference maximum on exact scores:
    per (query, head), steps of 32 keys in the kernel's order; count the
    steps after a row's first whose maximum exceeds the reference by more
    than KRAISE (log2 units), which then rescale the accumulators."""
    U = case.U.astype(np.float64)
    H, Hkv = case.shape.H, case.shape.kv
    qs = case.query_start_loc
    total = 0
    rows = 0
    for b in range(len(qs) - 1):
        L = int(case.cache.seq_lens[b])
        C = int(qs[b + 1] - qs[b])
        ck, _ = oracle.gather_sequence_latents(kc, np.zeros((kc.shape[0], 1, 16)),
                                               case.cache.block_tables[b], L)
        for h in range(H):
            g = h // (H // Hkv)
            qt = case.q[qs[b]:qs[b + 1], h].astype(np.float64) @ U[g]   # [C, r_k]
            s = qt @ ck[:, g].T * case.scale * LOG2E                     # [C, L]
            P0 = L - C
            for j in range(C):
                vis = s[j, :P0 + j + 1]
                m = -np.inf
                raised = 0
                for st in range(0, vis.shape[0], STEP_TOKENS):
                    pm = vis[st:st + STEP_TOKENS].max()
                    if pm > m + KRAISE:
                        if st > 0:
                            raised += 1
                        m = pm
                total += raised
                rows += raised > 0
    return total, rows


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


def _pre_oracle(case, kc, vc, rows=None):
    if kc.dtype == np.uint8:
        kc = oracle.dequantize_cache(kc, case.k_scale)
        vc = oracle.dequantize_cache(vc, case.v_scale)
    return oracle.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                          case.cache.block_tables, case.cache.seq_lens, case.scale,
                          request_indices=rows)


PREFILL_SHAPES = {"main": wl.MAIN, "tiny": wl.TINY, "gqa8": wl.GQA8, "lowrank": wl.LOWRANK}


@pytest.mark.parametrize("mult", [4, 16, 32])
@pytest.mark.parametrize("shape", ["main", "tiny", "gqa8", "lowrank"])
def test_prefill_scaled_queries(sk, shape, mult):
    cached, chunk = ([0, 15, 300], [1, 17, 70]) if shape != "tiny" else ([20, 7], [5, 33])
    case = wl.make_prefill_case(PREFILL_SHAPES[shape], cached, chunk, seed=71, q_mult=mult)
    note(f"peaked prefill {shape} q x{mult}")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"prefill {shape} q x{mult}")
    per_head_check(out, ref, f"prefill {shape} q x{mult}")


@pytest.mark.parametrize("mult", [16, 32])
def test_prefill_fp8_scaled_queries(sk, mult):
    case = wl.make_prefill_case(wl.MAIN, [64, 300], [40, 65], seed=72, q_mult=mult, fp8=True)
    note(f"peaked prefill fp8 q x{mult}")
    out, kc, vc = _gpu_prefill(sk, case)
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"prefill fp8 q x{mult}")
    per_head_check(out, ref, f"prefill fp8 q x{mult}")


@pytest.mark.parametrize("shape", ["main", "gqa8", "tiny"])
def test_prefill_rising_scores_raise_mid_chunk(sk, shape):
    """Key latents ramped by position: each row's maximum keeps rising, so
    the kernel's reference maximum moves (by more than 8 log2 units) after
    the first step, also inside the chunk."""
    cached, chunk = ([700, 90], [64, 130]) if shape != "tiny" else ([200, 40], [30, 60])
    case = wl.make_prefill_case(PREFILL_SHAPES[shape], cached, chunk, seed=73, q_mult=2,
                                ramp=30.0)
    note(f"peaked prefill {shape} rising scores")
    out, kc, vc = _gpu_prefill(sk, case)
    raises, rows = lazy_raises(case, kc)
    print(f"[raise] prefill {shape} rising: {raises} raises after a row's first step "
          f"in {rows} of {out.shape[0] * out.shape[1]} (query, head) rows", flush=True)
    assert raises > 0 and rows > 0
    ref = _pre_oracle(case, kc, vc)
    assert_parity(out, ref, f"prefill {shape} rising")
    per_head_check(out, ref, f"prefill {shape} rising")


def test_prefill_full_b16_scaled_sampled(sk):
    """prefill_b16's shape and launch configuration with queries scaled x16;
    the oracle checks a fixed sample of requests."""
    case = wl.make_prefill_case(wl.MAIN, [4096] * 16, [256] * 16, seed=74, q_mult=16)
    note("peaked prefill b16 q x16")
    out, kc, vc = _gpu_prefill(sk, case)
    rows = [0, 5, 11, 15]
    ref = _pre_oracle(case, kc, vc, rows=rows)
    sel = np.concatenate([np.arange(case.query_start_loc[r], case.query_start_loc[r + 1])
                          for r in rows])
    y = out[torch.from_numpy(sel).cuda()]
    assert_parity(y, ref[sel], "prefill b16 q x16 sample")
    per_head_check(y, ref[sel], "prefill b16 q x16 sample")

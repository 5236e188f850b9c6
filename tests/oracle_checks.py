"""Checks that pin the CPU oracle to facts other than itself.

Every check takes the oracle module as ``orc`` so that the same checks can be
run against deliberately broken copies of the oracle (see
``test_oracle_mutants.py``): each planted mistake must make at least one of
them fail.  The checks rely on

* torch's ``scaled_dot_product_attention`` in fp64 on the CPU, for the full
  rank special case where the compressed cache holds K and V exactly;
* closed forms (one token, zero query, identical latents, empty sequence);
* the algebraic identity between the rebuild-then-attend definition and the
  latent shortcut (scores on U_h^T q, values summed before W_h);
* brute-force scalar loops on logical-order latents, which never touch the
  block tables;
* invariants: softmax rows sum to one, prefill equals one decode per query,
  append with identity bases copies bit-exactly into exactly its slots.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from rank_compressed_paged_amd.workloads import (
    Shape, make_decode_case, make_prefill_case, fill_cache, _nan_f16)

TIGHT = 1e-12


def _max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def signed_permutation(rng, n):
    """An orthonormal matrix that is exact in fp16: a permutation with signs."""
    m = np.zeros((n, n))
    perm = rng.permutation(n)
    m[np.arange(n), perm] = rng.choice([-1.0, 1.0], size=n)
    return m


def _sdpa(q, K, V, scale, mask=None):
    """q [Q, H, d], K/V [L, H, d] -> [Q, H, d] via torch fp64 CPU."""
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(q, (1, 0, 2)))).double()[None]
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)))).double()[None]
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)))).double()[None]
    mt = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return np.transpose(o[0].numpy(), (1, 0, 2))


def _sdpa_gqa(q, K, V, scale, mask=None):
    """q [Q, H, d], K/V [L, Hkv, d] -> [Q, H, d] via torch's grouped-query
    mode (its own head mapping), fp64 CPU."""
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(q, (1, 0, 2)))).double()[None]
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)))).double()[None]
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)))).double()[None]
    mt = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale,
                                                         enable_gqa=True)
    return np.transpose(o[0].numpy(), (1, 0, 2))


def _dense_from_latents(ck, cv, U, W):
    """Test-side rebuild for exact bases only (signed permutations)."""
    U = U.astype(np.float64)
    W = W.astype(np.float64)
    H, d, _ = U.shape
    L = ck.shape[0]
    K = np.einsum("hdr,thr->thd", U, ck.astype(np.float64))
    V = np.einsum("jr,tr->tj", W, cv.astype(np.float64)).reshape(L, H, d)
    return K, V


# --------------------------------------------------------------------------
def check_full_rank_decode_matches_sdpa(orc):
    """U_h, W square signed permutations: the cache holds K and V exactly, so
    the oracle must equal uncompressed attention."""
    rng = np.random.default_rng(11)
    sh = Shape(H=3, d=8, r_k=8, r_v=24, bs=4)
    U = np.stack([signed_permutation(rng, 8) for _ in range(3)])
    W = signed_permutation(rng, 24)
    case = make_decode_case(sh, seq_lens=[1, 7, 13, 16], seed=5, keep_logical=True,
                            bases=(U, W))
    out = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                     case.cache.block_tables, case.cache.seq_lens, case.scale)
    for b, L in enumerate(case.cache.seq_lens):
        K, V = _dense_from_latents(case.cache.logical_ck[b], case.cache.logical_cv[b], case.U, case.W)
        ref = _sdpa(case.q[b:b + 1].astype(np.float64), K, V, case.scale)[0]
        assert _max_rel(out[b], ref) < TIGHT, (b, _max_rel(out[b], ref))


def check_full_rank_prefill_matches_sdpa(orc):
    """Same exact bases, chunked prefill with the causal offset mask."""
    rng = np.random.default_rng(12)
    sh = Shape(H=2, d=8, r_k=8, r_v=16, bs=4)
    U = np.stack([signed_permutation(rng, 8) for _ in range(2)])
    W = signed_permutation(rng, 16)
    cached = [5, 0, 9]
    chunk = [3, 4, 1]
    case = make_prefill_case(sh, cached, chunk, seed=6, keep_logical=True, bases=(U, W))
    kc, vc = orc.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                        case.cache.k_cache, case.cache.v_cache)
    out = orc.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                      case.cache.block_tables, case.seq_lens, case.scale)
    for b in range(3):
        P0, C = cached[b], chunk[b]
        q0, q1 = case.query_start_loc[b], case.query_start_loc[b + 1]
        ck_old = case.cache.logical_ck[b].astype(np.float64)
        cv_old = case.cache.logical_cv[b].astype(np.float64)
        K_old, V_old = _dense_from_latents(ck_old, cv_old, case.U, case.W)
        # exact bases: the new tokens' dense K/V are the inputs themselves
        K = np.concatenate([K_old, case.k_new[q0:q1].astype(np.float64)])
        V = np.concatenate([V_old, case.v_new[q0:q1].astype(np.float64)])
        mask = np.arange(P0 + C)[None, :] <= (P0 + np.arange(C))[:, None]
        ref = _sdpa(case.q[q0:q1].astype(np.float64), K, V, case.scale,
                    mask=np.broadcast_to(mask, (sh.H, C, P0 + C)).copy())
        assert _max_rel(out[q0:q1], ref) < TIGHT, b


def check_gqa_decode_matches_sdpa(orc):
    """Grouped-query layout (6 query heads on 2 key/value heads) with exact
    bases: the oracle must equal torch's grouped-query attention on the
    uncompressed K and V."""
    rng = np.random.default_rng(21)
    sh = Shape(H=6, d=8, r_k=8, r_v=16, bs=4, Hkv=2)
    U = np.stack([signed_permutation(rng, 8) for _ in range(2)])
    W = signed_permutation(rng, 16)
    case = make_decode_case(sh, seq_lens=[1, 9, 16, 5], seed=7, keep_logical=True,
                            bases=(U, W))
    out = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                     case.cache.block_tables, case.cache.seq_lens, case.scale)
    for b, L in enumerate(case.cache.seq_lens):
        K, V = _dense_from_latents(case.cache.logical_ck[b], case.cache.logical_cv[b], case.U, case.W)
        ref = _sdpa_gqa(case.q[b:b + 1].astype(np.float64), K, V, case.scale)[0]
        assert _max_rel(out[b], ref) < TIGHT, (b, _max_rel(out[b], ref))


def check_gqa_prefill_matches_sdpa(orc):
    """Grouped-query chunked prefill (4 query heads on 2) with exact bases and
    the causal offset mask, against torch's grouped-query attention."""
    rng = np.random.default_rng(22)
    sh = Shape(H=4, d=8, r_k=8, r_v=16, bs=4, Hkv=2)
    U = np.stack([signed_permutation(rng, 8) for _ in range(2)])
    W = signed_permutation(rng, 16)
    cached = [6, 0, 3]
    chunk = [2, 5, 4]
    case = make_prefill_case(sh, cached, chunk, seed=8, keep_logical=True, bases=(U, W))
    kc, vc = orc.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                        case.cache.k_cache, case.cache.v_cache)
    out = orc.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                      case.cache.block_tables, case.seq_lens, case.scale)
    for b in range(3):
        P0, C = cached[b], chunk[b]
        q0, q1 = case.query_start_loc[b], case.query_start_loc[b + 1]
        K_old, V_old = _dense_from_latents(case.cache.logical_ck[b].astype(np.float64),
                                           case.cache.logical_cv[b].astype(np.float64),
                                           case.U, case.W)
        K = np.concatenate([K_old, case.k_new[q0:q1].astype(np.float64)])
        V = np.concatenate([V_old, case.v_new[q0:q1].astype(np.float64)])
        mask = np.arange(P0 + C)[None, :] <= (P0 + np.arange(C))[:, None]
        ref = _sdpa_gqa(case.q[q0:q1].astype(np.float64), K, V, case.scale,
                        mask=np.broadcast_to(mask, (sh.H, C, P0 + C)).copy())
        assert _max_rel(out[q0:q1], ref) < TIGHT, b


def check_subspace_lossless(orc):
    """r_k < d and r_v < H*d with exact bases; k and v inside the spans.
    Appending then attending must equal dense attention on k and v, with the
    1/sqrt(d) scale (not 1/sqrt(r_k))."""
    rng = np.random.default_rng(13)
    sh = Shape(H=2, d=8, r_k=3, r_v=5, bs=4)
    U = np.stack([signed_permutation(rng, 8)[:, :3] for _ in range(2)])
    W = signed_permutation(rng, 16)[:, :5]
    N = 11
    a = rng.standard_normal((N, 2, 3)).astype(np.float16).astype(np.float64)
    bvec = rng.standard_normal((N, 5)).astype(np.float16).astype(np.float64)
    k = np.einsum("hdr,nhr->nhd", U, a).astype(np.float16)
    v = (bvec @ W.T).reshape(N, 2, 8).astype(np.float16)
    case = make_decode_case(sh, seq_lens=[N], seed=7, bases=(U, W))
    bt = case.cache.block_tables
    slots = np.array([bt[0, t // 4] * 4 + t % 4 for t in range(N)], dtype=np.int64)
    kc = _nan_f16(case.cache.k_cache.shape)
    vc = _nan_f16(case.cache.v_cache.shape)
    kc, vc = orc.append(k, v, case.U, case.W, slots, kc, vc)
    out = orc.decode(case.q, kc, vc, case.U, case.W, bt, case.cache.seq_lens, 1.0 / math.sqrt(8))
    ref = _sdpa(case.q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                1.0 / math.sqrt(8))
    assert _max_rel(out, ref) < TIGHT, _max_rel(out, ref)


def check_random_orthonormal_roundtrip(orc):
    """Square random orthonormal bases (fp16): append then attend is dense
    attention up to the fp16 rounding of bases and latents."""
    rng = np.random.default_rng(14)
    sh = Shape(H=2, d=16, r_k=16, r_v=32, bs=4)
    from rank_compressed_paged_amd.workloads import orthonormal_fp16
    U = np.stack([orthonormal_fp16(rng, 16, 16) for _ in range(2)])
    W = orthonormal_fp16(rng, 32, 32)
    N = 21
    k = rng.standard_normal((N, 2, 16)).astype(np.float16)
    v = rng.standard_normal((N, 2, 16)).astype(np.float16)
    case = make_decode_case(sh, seq_lens=[N], seed=8, bases=(U, W))
    bt = case.cache.block_tables
    slots = np.array([bt[0, t // 4] * 4 + t % 4 for t in range(N)], dtype=np.int64)
    kc, vc = orc.append(k, v, U, W, slots, _nan_f16(case.cache.k_cache.shape),
                        _nan_f16(case.cache.v_cache.shape))
    out = orc.decode(case.q, kc, vc, U, W, bt, case.cache.seq_lens, case.scale)
    ref = _sdpa(case.q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), case.scale)
    err = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err < 5e-3, err


def check_latent_identity(orc):
    """Arbitrary (non-orthonormal) bases: the oracle's rebuild path equals the
    latent shortcut q~ = U_h^T q, s = q~.c_k*scale, z = sum p c_v, W_h z."""
    rng = np.random.default_rng(15)
    sh = Shape(H=3, d=6, r_k=4, r_v=7, bs=4)
    U = rng.standard_normal((3, 6, 4)).astype(np.float16)
    W = rng.standard_normal((18, 7)).astype(np.float16)
    case = make_decode_case(sh, seq_lens=[9, 4, 1], seed=9, keep_logical=True, bases=(U, W))
    out = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, U, W,
                     case.cache.block_tables, case.cache.seq_lens, case.scale)
    from scipy.special import softmax
    Uf, Wf = U.astype(np.float64), W.astype(np.float64)
    for b in range(3):
        ck = case.cache.logical_ck[b].astype(np.float64)
        cv = case.cache.logical_cv[b].astype(np.float64)
        for h in range(3):
            qt = Uf[h].T @ case.q[b, h].astype(np.float64)
            p = softmax((ck[:, h, :] @ qt) * case.scale)
            z = p @ cv
            ref = Wf[h * 6:(h + 1) * 6] @ z
            assert _max_rel(out[b, h], ref) < 1e-11, (b, h)


def check_softmax_invariants(orc):
    case = make_decode_case(Shape(H=2, d=8, r_k=4, r_v=8, bs=4), seq_lens=[13, 3],
                            seed=10)
    _, probs = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                          case.cache.block_tables, case.cache.seq_lens, case.scale,
                          return_probs=True)
    for b, L in enumerate(case.cache.seq_lens):
        p = probs[b]
        assert p.shape == (2, L)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < TIGHT


def check_closed_forms(orc):
    """L = 1: out_h = W_h c_v[0].  q = 0: out_h = W_h mean_t c_v[t].
    Identical latents: out_h = W_h c_v whatever q.  L = 0: zeros."""
    sh = Shape(H=3, d=4, r_k=2, r_v=6, bs=4)
    case = make_decode_case(sh, seq_lens=[1, 10, 0], seed=11, keep_logical=True)
    Wf = case.W.astype(np.float64)
    out = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                     case.cache.block_tables, case.cache.seq_lens, case.scale)
    cv0 = case.cache.logical_cv[0][0].astype(np.float64)
    for h in range(3):
        assert _max_rel(out[0, h], Wf[h * 4:(h + 1) * 4] @ cv0) < TIGHT
    assert np.all(out[2] == 0.0)
    q0 = np.zeros_like(case.q)
    out0 = orc.decode(q0, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                      case.cache.block_tables, case.cache.seq_lens, case.scale)
    mean_cv = case.cache.logical_cv[1].astype(np.float64).mean(axis=0)
    for h in range(3):
        assert _max_rel(out0[1, h], Wf[h * 4:(h + 1) * 4] @ mean_cv) < TIGHT
    # identical latents in every slot of sequence 1
    kc = case.cache.k_cache.copy()
    vc = case.cache.v_cache.copy()
    blocks = case.cache.block_tables[1, :3]
    kc[blocks] = kc[blocks][0:1, :, 0:1, :]
    vc[blocks] = vc[blocks][0:1, :, 0:1]
    outi = orc.decode(case.q, kc, vc, case.U, case.W, case.cache.block_tables,
                      case.cache.seq_lens, case.scale)
    cvi = vc[blocks[0], :, 0].astype(np.float64)
    for h in range(3):
        assert _max_rel(outi[1, h], Wf[h * 4:(h + 1) * 4] @ cvi) < TIGHT


def brute_force_decode(q, U, W, logical_ck, logical_cv, scale):
    """Scalar loops over the latent formulas on logical-order tokens."""
    B, H, d = q.shape
    r_k = U.shape[2]
    r_v = W.shape[1]
    out = np.zeros((B, H, d))
    for b in range(B):
        ck, cv = logical_ck[b], logical_cv[b]
        L = ck.shape[0]
        for h in range(H):
            qt = [sum(float(U[h, i, r]) * float(q[b, h, i]) for i in range(d)) for r in range(r_k)]
            s = [scale * sum(qt[r] * float(ck[t, h, r]) for r in range(r_k)) for t in range(L)]
            if L == 0:
                continue
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            z = [sum(e[t] / tot * float(cv[t, j]) for t in range(L)) for j in range(r_v)]
            for i in range(d):
                out[b, h, i] = sum(float(W[h * d + i, j]) * z[j] for j in range(r_v))
    return out


def check_brute_force_tiny_ragged(orc):
    sh = Shape(H=2, d=4, r_k=2, r_v=4, bs=4)
    case = make_decode_case(sh, seq_lens=[1, 5, 17, 0, 8], seed=12, keep_logical=True,
                            extra_cols=2)
    out = orc.decode(case.q, case.cache.k_cache, case.cache.v_cache, case.U, case.W,
                     case.cache.block_tables, case.cache.seq_lens, case.scale)
    ref = brute_force_decode(case.q, case.U, case.W, case.cache.logical_ck,
                             case.cache.logical_cv, case.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def check_prefill_is_sequence_of_decodes(orc):
    """Chunk query j equals a decode over the first P0 + j + 1 tokens."""
    sh = Shape(H=2, d=8, r_k=4, r_v=8, bs=4)
    case = make_prefill_case(sh, [6, 3], [5, 2], seed=13)
    kc, vc = orc.append(case.k_new, case.v_new, case.U, case.W, case.slot_mapping,
                        case.cache.k_cache, case.cache.v_cache)
    out = orc.prefill(case.q, case.query_start_loc, kc, vc, case.U, case.W,
                      case.cache.block_tables, case.seq_lens, case.scale)
    for b in range(2):
        P0 = int(case.cached_lens[b])
        q0, q1 = case.query_start_loc[b], case.query_start_loc[b + 1]
        for j in range(q1 - q0):
            od = orc.decode(case.q[q0 + j][None], kc, vc, case.U, case.W,
                            case.cache.block_tables[b:b + 1], np.array([P0 + j + 1]), case.scale)
            assert _max_rel(out[q0 + j], od[0]) < TIGHT, (b, j)


def check_append_identity_copy(orc):
    """U = I, W = I: append copies k and v bit-exactly into exactly the
    listed slots (hand-computed), skips negative slots, touches nothing else."""
    sh = Shape(H=2, d=3, r_k=3, r_v=6, bs=4)
    U = np.stack([np.eye(3), np.eye(3)]).astype(np.float16)
    W = np.eye(6, dtype=np.float16)
    rng = np.random.default_rng(14)
    k = rng.standard_normal((4, 2, 3)).astype(np.float16)
    v = rng.standard_normal((4, 2, 3)).astype(np.float16)
    kc = _nan_f16((3, 2, 4, 3))
    vc = _nan_f16((3, 6, 4))
    # slots: block 2 offset 1, skipped, block 0 offset 3, block 1 offset 0
    slots = np.array([9, -1, 3, 4], dtype=np.int64)
    kc2, vc2 = orc.append(k, v, U, W, slots, kc, vc)
    written = {(2, 1): 0, (0, 3): 2, (1, 0): 3}
    for blk in range(3):
        for off in range(4):
            if (blk, off) in written:
                n = written[(blk, off)]
                assert np.array_equal(kc2[blk, :, off, :].view(np.uint16), k[n].view(np.uint16))
                assert np.array_equal(vc2[blk, :, off].view(np.uint16), v[n].reshape(-1).view(np.uint16))
            else:
                assert np.all(np.isnan(kc2[blk, :, off, :])) and np.all(np.isnan(vc2[blk, :, off]))
    assert np.all(np.isnan(kc)) and np.all(np.isnan(vc)), "inputs must not be modified"


def check_append_rounds_to_nearest(orc):
    """Each stored latent is an fp16 value nearest to the exact projection."""
    sh = Shape(H=2, d=8, r_k=4, r_v=6, bs=4)
    rng = np.random.default_rng(15)
    from rank_compressed_paged_amd.workloads import draw_bases
    U, W = draw_bases(rng, sh)
    k = rng.standard_normal((3, 2, 8)).astype(np.float16)
    v = rng.standard_normal((3, 2, 8)).astype(np.float16)
    slots = np.array([0, 5, 2], dtype=np.int64)
    kc, vc = orc.append(k, v, U, W, slots, _nan_f16((2, 2, 4, 4)), _nan_f16((2, 6, 4)))
    Uf, Wf = U.astype(np.float64), W.astype(np.float64)
    for n, s in enumerate(slots):
        blk, off = divmod(int(s), 4)
        exact_k = np.stack([Uf[h].T @ k[n, h].astype(np.float64) for h in range(2)])
        exact_v = Wf.T @ v[n].astype(np.float64).reshape(-1)
        for got, ex in ((kc[blk, :, off, :].ravel(), exact_k.ravel()),
                        (vc[blk, :, off].ravel(), exact_v.ravel())):
            g64 = got.astype(np.float64)
            up = np.nextafter(got, np.float16(np.inf)).astype(np.float64)
            dn = np.nextafter(got, np.float16(-np.inf)).astype(np.float64)
            assert np.all(np.abs(g64 - ex) <= np.abs(up - ex))
            assert np.all(np.abs(g64 - ex) <= np.abs(dn - ex))


def check_paging_fixture(orc, fixture):
    """Hand-worked block-table example: the oracle gathers token t of
    sequence b from the (block, offset) written in the fixture."""
    bs = fixture["block_size"]
    bt = np.array(fixture["block_tables"], dtype=np.int32)
    lens = np.array(fixture["seq_lens"], dtype=np.int32)
    nb = fixture["num_blocks"]
    H, r_k, r_v = 1, 1, 1
    kc = _nan_f16((nb, H, bs, r_k))
    vc = _nan_f16((nb, r_v, bs))
    for b, row in enumerate(fixture["token_slots"]):
        for t, (blk, off) in enumerate(row):
            kc[blk, 0, off, 0] = np.float16(100 * b + t)
            vc[blk, 0, off] = np.float16(-(100 * b + t))
    for b, L in enumerate(lens):
        ck, cv = orc.gather_sequence_latents(kc, vc, bt[b], L)
        assert np.array_equal(ck[:, 0, 0], 100 * b + np.arange(L))
        assert np.array_equal(cv[:, 0], -(100 * b + np.arange(L)))


# ---------------------------------------------------------------------------
# Bases from samples (fit_bases): planted subspaces with exact small-integer
# data, optimality against independent candidate bases, agreement with an
# SVD of the sample matrix, and invariances.
# ---------------------------------------------------------------------------
def _planted(rng, N, H, d, rk, rv, mean_dir=False):
    """Integer samples exact in fp16: keys of head h in span(A_h) (plus,
    with mean_dir, a constant offset along a direction outside it), values
    vec(v[n]) (head-major) in span(B)."""
    A = rng.integers(-2, 3, size=(H, d, rk)).astype(np.float64)
    B = rng.integers(-2, 3, size=(H * d, rv)).astype(np.float64)
    zk = rng.integers(-3, 4, size=(N, H, rk)).astype(np.float64)
    zv = rng.integers(-3, 4, size=(N, rv)).astype(np.float64)
    k = np.einsum("hdr,nhr->nhd", A, zk)
    v = (zv @ B.T).reshape(N, H, d)
    return k, v, A, B


def _residual(X, B):
    """Sum of squared reconstruction errors of the rows of X through the
    orthonormal columns of B."""
    R = X - (X @ B) @ B.T
    return float(np.sum(R * R))


def check_fit_planted_subspace(orc):
    rng = np.random.default_rng(40)
    N, H, d, rk, rv = 48, 3, 8, 3, 5
    k, v, A, B = _planted(rng, N, H, d, rk, rv)
    assert np.array_equal(k.astype(np.float16).astype(np.float64), k)  # exact in fp16
    U, W, ek, ev = orc.fit_bases(k.astype(np.float16), v.astype(np.float16), rk, rv)
    for h in range(H):
        assert np.abs(orc.projector(U[h]) - orc.projector(A[h])).max() < 1e-9
        assert ek[h][rk] < 1e-9 * ek[h][0]  # nothing outside the planted span
    assert np.abs(orc.projector(W) - orc.projector(B)).max() < 1e-9
    assert ev[rv] < 1e-9 * ev[0]


def check_fit_uncentred(orc):
    """Samples with a constant offset outside span(A): the uncentred
    second moment keeps the offset's direction, so rank(A)+1 columns
    reconstruct every sample exactly (a mean-centred fit would not)."""
    rng = np.random.default_rng(41)
    N, d, r = 40, 8, 2
    A = rng.integers(-2, 3, size=(d, r)).astype(np.float64)
    mu = None
    for i in range(d):  # an integer offset 4 e_i outside span(A)
        e = np.zeros(d)
        e[i] = 1.0
        if np.linalg.matrix_rank(np.column_stack([A, e])) == r + 1:
            mu = 4.0 * e
            break
    assert mu is not None
    z = rng.integers(-3, 4, size=(N, r)).astype(np.float64)
    k = (mu[None, :] + z @ A.T)[:, None, :]
    v = k.copy()
    U, W, _, _ = orc.fit_bases(k.astype(np.float16), v.astype(np.float16), r + 1, r + 1)
    X = k[:, 0, :]
    assert _residual(X, U[0]) < 1e-18 * np.sum(X * X) + 1e-20
    assert _residual(X, W) < 1e-18 * np.sum(X * X) + 1e-20


def check_fit_optimal_against_candidates(orc):
    """Eckart-Young: no other orthonormal rank-r basis reconstructs the
    samples better (random bases, and bases of r of the samples)."""
    rng = np.random.default_rng(42)
    N, H, d, rk, rv = 64, 2, 12, 4, 6
    scale = np.linspace(3.0, 0.2, d)
    k = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    v = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    U, W, _, _ = orc.fit_bases(k, v, rk, rv)
    kf, vf = k.astype(np.float64), v.astype(np.float64).reshape(N, H * d)
    for h in range(H):
        best = _residual(kf[:, h, :], U[h])
        for _ in range(20):
            Q = np.linalg.qr(rng.standard_normal((d, rk)))[0]
            assert best <= _residual(kf[:, h, :], Q) * (1 + 1e-12)
        Q = np.linalg.qr(kf[rng.choice(N, rk, replace=False), h, :].T)[0]
        assert best <= _residual(kf[:, h, :], Q) * (1 + 1e-12)
    best = _residual(vf, W)
    for _ in range(20):
        Q = np.linalg.qr(rng.standard_normal((H * d, rv)))[0]
        assert best <= _residual(vf, Q) * (1 + 1e-12)


def check_fit_matches_svd_of_samples(orc):
    """The top right singular vectors of the sample matrix (a different
    LAPACK path) span the same subspaces; the bases are orthonormal."""
    rng = np.random.default_rng(43)
    N, H, d, rk, rv = 80, 2, 10, 3, 7
    scale = np.geomspace(4.0, 0.1, d)
    k = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    v = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    U, W, _, _ = orc.fit_bases(k, v, rk, rv)
    for h in range(H):
        Vt = np.linalg.svd(k[:, h, :].astype(np.float64), full_matrices=False)[2]
        assert np.abs(orc.projector(U[h]) - orc.projector(Vt[:rk].T)).max() < 1e-9
        assert np.abs(U[h].T @ U[h] - np.eye(rk)).max() < 1e-12
    Vt = np.linalg.svd(v.astype(np.float64).reshape(N, H * d), full_matrices=False)[2]
    assert np.abs(orc.projector(W) - orc.projector(Vt[:rv].T)).max() < 1e-9
    assert np.abs(W.T @ W - np.eye(rv)).max() < 1e-12


def check_fit_invariances(orc):
    """Sample order and a common power-of-two scale leave the subspaces."""
    rng = np.random.default_rng(44)
    N, H, d, rk, rv = 50, 2, 8, 3, 4
    scale = np.linspace(2.0, 0.3, d)
    k = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    v = (rng.standard_normal((N, H, d)) * scale).astype(np.float16)
    U, W, _, _ = orc.fit_bases(k, v, rk, rv)
    perm = rng.permutation(N)
    U2, W2, _, _ = orc.fit_bases(k[perm] * np.float16(2), v[perm] * np.float16(2), rk, rv)
    for h in range(H):
        assert np.abs(orc.projector(U[h]) - orc.projector(U2[h])).max() < 1e-9
    assert np.abs(orc.projector(W) - orc.projector(W2)).max() < 1e-9


# --------------------------------------------------------------------------
# FP8 latents
def check_e4m3_table_matches_torch(orc):
    """The 256 E4M3 code values equal torch's float8_e4m3fn conversion."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = orc.e4m3_values()
    assert np.array_equal(np.isnan(v), np.isnan(ref))
    assert np.array_equal(v[~np.isnan(v)], ref[~np.isnan(ref)])


def check_e4m3_rounding_matches_torch(orc):
    """Rounding to nearest, ties to even, on fp32 inputs inside +-448 (where
    torch's conversion and the clamped one agree): random values over eight
    decades, every exact midpoint between neighbouring codes, subnormals."""
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 1e-2, 0.1, 1, 10, 100)])
    vals = np.sort(np.unique(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
                             .to(torch.float64).numpy()))
    vals = vals[np.isfinite(vals)]
    mids = (vals[1:] + vals[:-1]) / 2            # exact in fp32 for this grid
    x = np.clip(np.concatenate([x, mids, -mids, vals]), -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.quantize_e4m3(x)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def check_e4m3_saturates(orc):
    """Magnitudes at or beyond the largest finite value clamp to +-448."""
    x = np.array([448.0, 449.0, 479.0, 480.0, 1e6, -500.0, -1e30])
    v = orc.e4m3_values()[orc.quantize_e4m3(x)]
    assert np.array_equal(v, np.array([448, 448, 448, 448, 448, -448, -448], dtype=float))


def check_fp8_append_exact_roundtrip(orc):
    """Signed-permutation bases and inputs that are scale times E4M3 values:
    the FP8 append stores exactly those values, so dequantising gives back
    the projections (closed form), with the scales on both sides."""
    rng = np.random.default_rng(32)
    sh = Shape(H=2, d=8, r_k=8, r_v=16, bs=4)
    U = np.stack([signed_permutation(rng, 8) for _ in range(2)])
    W = signed_permutation(rng, 16)
    grid = orc.e4m3_values()[:0x70]              # positive finite values up to 1.875 * 2^6
    ks, vs = 0.5, 4.0
    n = 6
    k = (rng.choice(grid, size=(n, 2, 8)) * rng.choice([-1, 1], size=(n, 2, 8)) * ks)
    v = (rng.choice(grid, size=(n, 2, 8)) * rng.choice([-1, 1], size=(n, 2, 8)) * vs)
    k, v = k.astype(np.float16), v.astype(np.float16)
    slots = np.array([3, 9, -1, 0, 15, 6])
    kc = np.zeros((4, 2, 4, 8), np.uint8)
    vc = np.zeros((4, 16, 4), np.uint8)
    kc, vc = orc.append_fp8(k, v, U, W, slots, ks, vs, kc, vc)
    kd, vd = orc.dequantize_cache(kc, ks), orc.dequantize_cache(vc, vs)
    for i, s_ in enumerate(slots):
        if s_ < 0:
            continue
        blk, off = divmod(int(s_), 4)
        for h in range(2):
            assert np.array_equal(kd[blk, h, off], U[h].T @ k[i, h].astype(np.float64))
        assert np.array_equal(vd[blk, :, off], W.T @ v[i].astype(np.float64).reshape(-1))


ALL_CHECKS = [
    check_e4m3_table_matches_torch,
    check_e4m3_rounding_matches_torch,
    check_e4m3_saturates,
    check_fp8_append_exact_roundtrip,
    check_fit_planted_subspace,
    check_fit_uncentred,
    check_fit_optimal_against_candidates,
    check_fit_matches_svd_of_samples,
    check_fit_invariances,
    check_full_rank_decode_matches_sdpa,
    check_full_rank_prefill_matches_sdpa,
    check_gqa_decode_matches_sdpa,
    check_gqa_prefill_matches_sdpa,
    check_subspace_lossless,
    check_random_orthonormal_roundtrip,
    check_latent_identity,
    check_softmax_invariants,
    check_closed_forms,
    check_brute_force_tiny_ragged,
    check_prefill_is_sequence_of_decodes,
    check_append_identity_copy,
    check_append_rounds_to_nearest,
]

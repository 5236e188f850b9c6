"""Decode, serving and prefill steps captured in HIP graphs: the calls launch kernels
only (no allocation, no memset, no host synchronisation), so a caller can
capture one step on its stream and replay it.  The test replays the graph
several times, with eager work and synchronisations between the replays and
new inputs written in place before each, and checks every replay against an
eager call on the same inputs (bit-identical: the same kernels on the same
data) and against the oracle."""
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


@pytest.mark.parametrize("lens", [[2048], [700, 3000, 1, 16]], ids=["b1", "b4"])
def test_decode_graph_replays(sk, lens):
    case = wl.make_decode_case(wl.MAIN, seq_lens=lens, seed=91)
    c = case.cache
    q, kc, vc, U, W = dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U), dev(case.W)
    bt, sl = dev(c.block_tables), dev(c.seq_lens)
    B, msl = len(lens), int(max(lens))
    dims = sk.dims_of(kc, vc, U, W)
    ws = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl), "cuda")
    out = torch.empty((B, 32, 128), dtype=torch.float16, device="cuda")
    note(f"graph capture of decode lens={lens}")

    def step(o):
        sk.decode_attn(q, kc, vc, U, W, bt, sl, msl, case.scale, out=o, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(out)                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    rng = np.random.default_rng(92)
    for rep in range(4):
        qn = rng.standard_normal(case.q.shape, dtype=np.float32).astype(np.float16)
        q.copy_(torch.from_numpy(qn))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(out)
        step(eager)                    # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        ref = oracle.decode(qn, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                            c.seq_lens, case.scale)
        assert_parity(got, ref, f"graph replay {rep}")


@pytest.mark.parametrize("chunk", [16, 300], ids=["few_token_append", "tiled_append"])
def test_serving_step_graph_replays(sk, chunk):
    """A whole serving step captured as one graph: the append of the step's
    new tokens (the few-token form, whose arrival counters must return to
    zero, or the tiled form with its split contraction) and then decode over
    the grown sequences.  Each replay gets new q, k, v written in place;
    every replay must equal the eager step bit for bit and the oracle's
    append-then-decode within the bars."""
    shape = wl.MAIN
    B = 4 if chunk == 16 else 1
    per = chunk // B
    lens0 = [600, 33, 1500, 0][:B] if B > 1 else [900]
    case = wl.make_decode_case(shape, seq_lens=[L + per for L in lens0], seed=93)
    c = case.cache
    # the step's tokens: the last `per` positions of every sequence
    slots = np.concatenate([c.block_tables[b, (lens0[b] + j) // 16] * 16 + (lens0[b] + j) % 16
                            for b in range(B) for j in [np.arange(per)]]).astype(np.int64)
    kc0, vc0 = c.k_cache.copy(), c.v_cache.copy()
    q, U, W = dev(case.q), dev(case.U), dev(case.W)
    kc, vc = dev(kc0), dev(vc0)
    bt, sl = dev(c.block_tables), dev(c.seq_lens)
    ts = dev(slots)
    msl = int(c.seq_lens.max())
    rng = np.random.default_rng(94)
    kn = torch.zeros((chunk, shape.kv, shape.d), dtype=torch.float16, device="cuda")
    vn = torch.zeros_like(kn)
    dims = sk.dims_of(kc, vc, U, W)
    ws_a = sk.alloc_workspace(sk.append_workspace_size(dims, chunk), "cuda")
    ws_d = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl), "cuda")
    out = torch.empty((B, shape.H, shape.d), dtype=torch.float16, device="cuda")
    note(f"graph capture of append ({chunk} tokens) + decode")

    def step(o):
        sk.append(kn, vn, U, W, ts, kc, vc, workspace=ws_a)
        sk.decode_attn(q, kc, vc, U, W, bt, sl, msl, case.scale, out=o, workspace=ws_d)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    for rep in range(4):
        qn = rng.standard_normal(case.q.shape, dtype=np.float32).astype(np.float16)
        knn = rng.standard_normal(tuple(kn.shape), dtype=np.float32).astype(np.float16)
        vnn = rng.standard_normal(tuple(vn.shape), dtype=np.float32).astype(np.float16)
        q.copy_(torch.from_numpy(qn))
        kn.copy_(torch.from_numpy(knn))
        vn.copy_(torch.from_numpy(vnn))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        assert int(torch.count_nonzero(ws_a[:256]).item()) == 0
        eager = torch.empty_like(out)
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        okc, ovc = oracle.append(knn, vnn, case.U, case.W, slots, kc0, vc0)
        ref = oracle.decode(qn, okc, ovc, case.U, case.W, c.block_tables, c.seq_lens, case.scale)
        assert_parity(got, ref, f"step graph replay {rep}")


@pytest.mark.parametrize("shape", [wl.MAIN, wl.LOWRANK], ids=["main_fused_upprojection", "lowrank_upprojection_kernel"])
def test_prefill_step_graph_replays(sk, shape):
    """A chunked-prefill step (append of the chunks, then attention; the main
    shape applies W_h in the attention epilogue, the lower rank profile in a
    launch of its own) captured as one graph and replayed with new chunk
    tokens: each replay bit-identical to the eager step and within the bars."""
    case = wl.make_prefill_case(shape, [100, 700], [40, 90], seed=95)
    c = case.cache
    kc0, vc0 = c.k_cache.copy(), c.v_cache.copy()
    U, W = dev(case.U), dev(case.W)
    kc, vc = dev(kc0), dev(vc0)
    bt, sl, qsl = dev(c.block_tables), dev(c.seq_lens), dev(case.query_start_loc)
    ts = dev(case.slot_mapping)
    T = int(case.query_start_loc[-1])
    mq = int(np.diff(case.query_start_loc).max())
    msl = int(c.seq_lens.max())
    q = torch.zeros(tuple(case.q.shape), dtype=torch.float16, device="cuda")
    kn = torch.zeros(tuple(case.k_new.shape), dtype=torch.float16, device="cuda")
    vn = torch.zeros_like(kn)
    dims = sk.dims_of(kc, vc, U, W, num_heads=shape.H)
    ws_a = sk.alloc_workspace(sk.append_workspace_size(dims, T), "cuda")
    ws_p = sk.alloc_workspace(sk.prefill_workspace_size(dims, len(case.query_start_loc) - 1, T,
                                                        msl), "cuda")
    out = torch.empty((T, shape.H, shape.d), dtype=torch.float16, device="cuda")
    note(f"graph capture of append + prefill {shape}")

    def step(o):
        sk.append(kn, vn, U, W, ts, kc, vc, workspace=ws_a)
        sk.prefill_attn(q, qsl, mq, kc, vc, U, W, bt, sl, msl, case.scale, out=o, workspace=ws_p)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    rng = np.random.default_rng(96)
    for rep in range(3):
        qn = rng.standard_normal(tuple(q.shape), dtype=np.float32).astype(np.float16)
        knn = rng.standard_normal(tuple(kn.shape), dtype=np.float32).astype(np.float16)
        vnn = rng.standard_normal(tuple(vn.shape), dtype=np.float32).astype(np.float16)
        q.copy_(torch.from_numpy(qn))
        kn.copy_(torch.from_numpy(knn))
        vn.copy_(torch.from_numpy(vnn))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(out)
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        okc, ovc = oracle.append(knn, vnn, case.U, case.W, case.slot_mapping, kc0, vc0)
        ref = oracle.prefill(qn, case.query_start_loc, okc, ovc, case.U, case.W, c.block_tables,
                             c.seq_lens, case.scale)
        assert_parity(got, ref, f"prefill step graph replay {rep}")

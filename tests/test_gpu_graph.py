"""Low-batch decode captured in a HIP graph: the decode call launches kernels
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

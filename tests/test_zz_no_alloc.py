"""The decode entry point that allocates nothing (its scratch is a device
array of the library) against starkv_decode_attn with a caller workspace, on
the same inputs: bit-identical outputs (same kernels, same plan), and both
within the oracle's bars; two calls in a row, the second smaller, so the
second reads a scratch that still holds the first call's contents."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, decode_tensors, note
from rank_compressed_paged_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sk():
    from rank_compressed_paged_amd import starkv
    return starkv


def _both(sk, case):
    t = decode_tensors(case)
    msl = int(case.cache.seq_lens.max())
    ref_out = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"],
                             t["block_tables"], t["seq_lens"], msl, case.scale)
    out = torch.full_like(ref_out, float("nan"))
    sk.decode_attn_noalloc(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                           t["seq_lens"], msl, out, case.scale)
    torch.cuda.synchronize()
    return out, ref_out


def _oracle(case):
    c = case.cache
    return oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                         c.seq_lens, case.scale)


def test_noalloc_matches_workspace_entry_point(sk):
    big = wl.make_config("decode_b16")
    small = wl.make_decode_case(wl.MAIN, seq_lens=[300, 0, 17, 4097], seed=81)
    for what, case in (("decode_b16", big), ("smaller ragged batch", small)):
        note(f"noalloc decode {what}")
        out, ref_out = _both(sk, case)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), what
        assert_parity(out, _oracle(case), f"noalloc {what}")


def test_noalloc_tiny_shape(sk):
    case = wl.make_config("tiny")
    note("noalloc decode tiny")
    out, ref_out = _both(sk, case)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert_parity(out, _oracle(case), "noalloc tiny")


def test_noalloc_rejects_plans_beyond_its_scratch(sk):
    """256 sequences of 4096 tokens need 34 MiB of partials, more than the
    library's 32 MiB: refused on the host, nothing launched, out untouched."""
    d = sk.make_dims(32, 128, 64, 512, 8)
    assert sk.decode_workspace_size(d, 256, 4096) > sk.NOALLOC_SCRATCH_BYTES
    B, L = 256, 4096
    q = torch.zeros((B, 32, 128), dtype=torch.float16, device="cuda")
    kc = torch.zeros((8, 32, 16, 64), dtype=torch.float16, device="cuda")
    vc = torch.zeros((8, 512, 16), dtype=torch.float16, device="cuda")
    U = torch.zeros((32, 128, 64), dtype=torch.float16, device="cuda")
    W = torch.zeros((32 * 128, 512), dtype=torch.float16, device="cuda")
    bt = torch.zeros((B, L // 16), dtype=torch.int32, device="cuda")
    sl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, 32, 128), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(sk.StarKVError) as ei:
        sk.decode_attn_noalloc(q, kc, vc, U, W, bt, sl, L, out)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

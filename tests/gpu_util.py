"""Helpers shared by the GPU parity tests: move a seeded case to the GPU,
call the HIP library through the binding, and compare with the oracle."""
import sys

import numpy as np
import torch

PARITY_MAX_ABS = 2e-3
PARITY_REL_L2 = 1e-3


def note(msg):
    """Name the case before each GPU step, flushed, so a crash can be traced."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def decode_tensors(case):
    c = case.cache
    return dict(q=dev(case.q), k_cache=dev(c.k_cache), v_cache=dev(c.v_cache), U=dev(case.U),
                W=dev(case.W), block_tables=dev(c.block_tables), seq_lens=dev(c.seq_lens))


def run_decode(sk, case, t=None, max_seq_len=None):
    t = t or decode_tensors(case)
    msl = int(max(case.cache.seq_lens.max(initial=0), 1)) if max_seq_len is None else max_seq_len
    msl = min(msl, t["block_tables"].shape[1] * case.shape.bs)
    out = sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                         t["seq_lens"], msl, case.scale)
    torch.cuda.synchronize()
    return out


def errors(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    e = y - ref
    ma = float(np.max(np.abs(e))) if e.size else 0.0
    den = float(np.linalg.norm(ref))
    rl = float(np.linalg.norm(e) / den) if den > 0 else float(np.linalg.norm(e))
    return ma, rl


def assert_parity(gpu, ref, what, max_abs=PARITY_MAX_ABS, rel_l2=PARITY_REL_L2):
    y = gpu.float().cpu().numpy() if isinstance(gpu, torch.Tensor) else gpu
    assert np.all(np.isfinite(y)), f"{what}: non-finite GPU output"
    ma, rl = errors(y, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl

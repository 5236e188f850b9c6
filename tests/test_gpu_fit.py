"""Bases from samples on the GPU against the oracle (fp64 eigendecomposition
of the sample second moments).

Bases are compared as subspaces: sin of the largest principal angle between
the GPU basis and the oracle's, which is zero for two bases of one subspace
whatever their rotation inside it.  Tolerance: the GPU result is fp16, so it
sits about as far from the exact subspace as the exact basis rounded to fp16
does (d16, computed per case); the fp32 Gram matrices and products add a
few 1e-5 on these well-separated spectra.  Bound: 2 * d16 + 2e-4.  Columns
must be orthonormal to fp16 rounding: |B^T B - I| <= 2 * 2^-11 + 1e-5 per
entry (each entry of an fp16 column carries at most 2^-11 relative error).
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import starkv_oracle as oracle  # noqa: E402
from rank_compressed_paged_amd import workloads as wl  # noqa: E402
from tests.gpu_util import dev, note  # noqa: E402

pytestmark = pytest.mark.gpu

ORTHO_TOL = 2 * 2.0 ** -11 + 1e-5


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_compressed_paged_amd import starkv
    return starkv


def sin_theta(B, ref):
    """sin of the largest principal angle between span(B) and span(ref)."""
    qb = np.linalg.qr(np.asarray(B, np.float64))[0]
    qr = np.linalg.qr(np.asarray(ref, np.float64))[0]
    return float(np.linalg.norm(qb - qr @ (qr.T @ qb), 2))


def check_basis(B16, ref, what):
    B = np.asarray(B16, np.float64)
    assert np.all(np.isfinite(B)), f"{what}: non-finite"
    d16 = sin_theta(ref.astype(np.float16), ref)
    st = sin_theta(B, ref)
    orth = float(np.max(np.abs(B.T @ B - np.eye(B.shape[1]))))
    print(f"[parity] {what}: sin_theta={st:.3e} (fp16 rounding of the exact basis "
          f"{d16:.3e}) max|B^T B - I|={orth:.3e}", flush=True)
    assert st <= 2 * d16 + 2e-4, f"{what}: sin_theta={st:.3e}"
    assert orth <= ORTHO_TOL, f"{what}: orthonormality {orth:.3e}"


def run_fit(sk, case, iters):
    info = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sh = case.shape
    U, W = sk.fit_bases(dev(case.k), dev(case.v), sh.r_k, sh.r_v, dev(case.u0), dev(case.w0),
                        iters, info=info)
    torch.cuda.synchronize()
    return U.float().cpu().numpy(), W.float().cpu().numpy(), int(info.item())


def compare(case, U, W):
    Uo, Wo, _, _ = oracle.fit_bases(case.k, case.v, case.shape.r_k, case.shape.r_v)
    for h in range(case.shape.H):
        check_basis(U[h], Uo[h], f"{case.name} U[{h}]")
    check_basis(W, Wo, f"{case.name} W")


@pytest.mark.parametrize("N", [1000, 4096])
def test_fit_tiny(sk, N):
    # N = 1000 ends in a partial 32-sample chunk
    case = wl.make_fit_case(wl.TINY, N, seed=11, name=f"tiny N={N}")
    note(f"fit tiny N={N} seed=11")
    U, W, info = run_fit(sk, case, iters=6)
    assert info == 0
    compare(case, U, W)


def test_fit_main(sk):
    case = wl.make_fit_case(wl.MAIN, 1500, seed=12, name="main N=1500")
    note("fit main N=1500 seed=12")
    U, W, info = run_fit(sk, case, iters=6)
    assert info == 0
    compare(case, U, W)


def test_fit_odd_shape(sk):
    # d = 192 (three 64-tiles, so 64-wide Gram tiles), ranks that are not
    # multiples of 64 (ragged Cholesky panels and solve blocks), 3 heads
    shape = wl.Shape(H=3, d=192, r_k=40, r_v=100)
    case = wl.make_fit_case(shape, 777, seed=13, name="H3 d192 r40/100 N=777")
    note("fit odd shape seed=13")
    U, W, info = run_fit(sk, case, iters=6)
    assert info == 0
    compare(case, U, W)


def test_fit_min_samples(sk):
    # exactly r_v samples: G_v has rank r_v, its top r_v eigenspace is the
    # row space of the samples
    case = wl.make_fit_case(wl.TINY, wl.TINY.r_v, seed=14, name="tiny N=r_v")
    note("fit tiny N=r_v seed=14")
    U, W, info = run_fit(sk, case, iters=4)
    assert info == 0
    compare(case, U, W)


def test_fit_rank_deficient_reported(sk):
    # all-zero samples: every pivot is zero; the call reports it in info and
    # leaves finite output
    case = wl.make_fit_case(wl.TINY, 128, seed=15, name="tiny zeros")
    case.k[:] = 0
    case.v[:] = 0
    note("fit zero samples seed=15")
    U, W, info = run_fit(sk, case, iters=2)
    assert info > 0
    assert np.all(np.isfinite(U)) and np.all(np.isfinite(W))


def test_fit_full_size(sk):
    # the workload the benchmark times: 16384 samples, main shape, 8 iterations
    case = wl.make_config("fit_n16384")
    note("fit fit_n16384 (16384 samples, main shape)")
    U, W, info = run_fit(sk, case, iters=8)
    assert info == 0
    compare(case, U, W)

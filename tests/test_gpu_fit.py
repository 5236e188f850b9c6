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


def run_fit(sk, case, iters, with_residual=False):
    info = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    res = torch.full((2,), -1.0, dtype=torch.float32, device="cuda") if with_residual else None
    sh = case.shape
    U, W = sk.fit_bases(dev(case.k), dev(case.v), sh.r_k, sh.r_v, dev(case.u0), dev(case.w0),
                        iters, info=info, residual=res)
    torch.cuda.synchronize()
    out = (U.float().cpu().numpy(), W.float().cpu().numpy(), int(info.item()))
    return out + (res.cpu().numpy(),) if with_residual else out


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


def dk_bound(res, ev, r, n_samples):
    """Davis-Kahan: sin of the largest angle between a basis B and the top-r
    eigenspace of G is at most ||G B - B (B^T G B)||_F / (lambda_r -
    lambda_{r+1}).  The GPU reports that residual relative to ||G B||_F
    (sqrt of the sum of the top r eigenvalues squared for a converged basis)
    against its own fp32 Gram matrix, which differs from the exact one by
    about 2^-24 sqrt(N) ||G||_F (fp32 sums of N products); that perturbation
    enters the same bound."""
    ev = np.asarray(ev, np.float64)
    gap = ev[r - 1] - ev[r]
    resid = float(res) * float(np.sqrt(np.sum(ev[:r] ** 2)))
    gram = 2.0 ** -24 * np.sqrt(n_samples) * float(np.sqrt(np.sum(ev ** 2)))
    return (resid + gram) / gap


DECAY_SHAPES = [wl.Shape(H=4, d=64, r_k=16, r_v=32), wl.Shape(H=3, d=128, r_k=24, r_v=48)]


@pytest.mark.parametrize("spectrum", ["power", "exp"])
@pytest.mark.parametrize("shape", DECAY_SHAPES, ids=["h4_d64", "h3_d128"])
def test_fit_decaying_spectrum(sk, shape, spectrum):
    """Spectra with no planted gap (sample eigenvalue ratio at the rank
    0.80-0.97 with these shapes and 16384 samples): 600 iterations; the
    reported residual must be small, and the GPU basis must lie within the
    Davis-Kahan bound that residual implies (plus the fp16 rounding of the
    exact basis) of the oracle's eigenspace."""
    iters = 600
    case = wl.make_fit_case(shape, 16384, seed=16, spectrum=spectrum,
                            name=f"{spectrum} H{shape.H} d{shape.d}")
    note(f"fit {spectrum} spectrum H{shape.H} d{shape.d} iters={iters}")
    U, W, info, res = run_fit(sk, case, iters, with_residual=True)
    assert info == 0
    Uo, Wo, ek, ev = oracle.fit_bases(case.k, case.v, shape.r_k, shape.r_v)
    ratio_k = max(ek[h][shape.r_k] / ek[h][shape.r_k - 1] for h in range(shape.H))
    ratio_v = ev[shape.r_v] / ev[shape.r_v - 1]
    print(f"[fit] {spectrum} H{shape.H} d{shape.d}: {iters} iterations, residual keys "
          f"{res[0]:.3e} values {res[1]:.3e}; eigenvalue ratio at the rank keys {ratio_k:.3f} "
          f"values {ratio_v:.3f}", flush=True)
    assert 0.0 <= res[0] < 1e-3 and 0.0 <= res[1] < 1e-3
    for h in range(shape.H):
        b = dk_bound(res[0], ek[h], shape.r_k, 16384)
        d16 = sin_theta(Uo[h].astype(np.float16), Uo[h])
        st = sin_theta(U[h], Uo[h])
        print(f"[parity] {case.name} U[{h}]: sin_theta={st:.3e} bound {b + 2 * d16 + 2e-4:.3e}",
              flush=True)
        assert st <= b + 2 * d16 + 2e-4
    b = dk_bound(res[1], ev, shape.r_v, 16384)
    d16 = sin_theta(Wo.astype(np.float16), Wo)
    st = sin_theta(W, Wo)
    print(f"[parity] {case.name} W: sin_theta={st:.3e} bound {b + 2 * d16 + 2e-4:.3e}", flush=True)
    assert st <= b + 2 * d16 + 2e-4


def test_fit_residual_falls_with_iterations(sk):
    """The residual is a convergence measure: on a decaying spectrum it falls
    as the iterations grow, and it is near zero on the planted one."""
    case = wl.make_fit_case(DECAY_SHAPES[0], 16384, seed=17, spectrum="exp", name="exp h4")
    note("fit residual vs iterations")
    rs = [run_fit(sk, case, it, with_residual=True)[3] for it in (2, 20, 200)]
    print(f"[fit] residual after 2 / 20 / 200 iterations: keys "
          f"{[f'{r[0]:.2e}' for r in rs]} values {[f'{r[1]:.2e}' for r in rs]}", flush=True)
    for side in (0, 1):
        assert rs[0][side] > rs[1][side] > rs[2][side]
    planted = wl.make_fit_case(wl.TINY, 4096, seed=18, name="planted tiny")
    r = run_fit(sk, planted, 8, with_residual=True)[3]
    print(f"[fit] planted spectrum, 8 iterations: residual {r[0]:.2e} {r[1]:.2e}", flush=True)
    assert r[0] < 1e-3 and r[1] < 1e-3

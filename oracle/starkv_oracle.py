"""Plain fp64 CPU oracle for attention over a paged, low-rank-compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path and imports nothing from the package.

What it computes (Proxima README, introduction: STAR-KV keeps a per-layer
low-rank projection of the KV cache, head-wise for K and joint across heads
for V, stored in a compressed paged format with 16-token blocks -- "KV-cache
capacity" table):

* key latents    c_k[t, h] = U_h^T k[t, h],   U_h in R^{d x r_k}, one per head
* value latents  c_v[t]    = W^T vec(v[t]),   W in R^{(H*d) x r_v}, shared
                 by all heads; vec() flattens [H, d] head-major (row h*d + i)
* grouped-query layouts: H query heads share Hkv key/value heads, query head
  h reading key/value head h // (H / Hkv) (consecutive groups); U, the key
  latents and W's rows are per key/value head.  Hkv = H is multi-head
  attention.
* attention reads the latents through block tables.  The oracle takes the
  plain definition: rebuild K^[t,h] = U_h c_k[t,h] and V^[t] = W c_v[t]
  explicitly, then run textbook two-pass softmax attention in fp64 with the
  caller's scale (1/sqrt(d) in every caller).  The latent shortcut the GPU
  takes (q~ = U_h^T q, softmax(q~ . c_k), W_h sum p c_v) equals this up to
  rounding order, for any U and W.

Readings taken where the pages are silent (each listed in the design notes):
* layouts: k_cache [NB, Hkv, bs, r_k], v_cache [NB, r_v, bs], fp16;
* the write kernel's "normalization" (README, "Kernel profiling breakdown")
  is read as none: the stored latent is exactly fp16(U_h^T k), fp16(W^T v);
* a decode query attends to all seq_lens[b] cached tokens (append first);
* a prefill chunk query j of request b sits at position P0 + j with
  P0 = seq_lens[b] - C_b and sees keys 0 .. P0 + j (causal, diagonal kept);
* slot_mapping < 0 means "skip"; seq_len 0 gives a zero output.

Every floating-point input is fp16 in the ABI and is widened exactly to fp64
here; outputs are fp64 and never rounded.  Integer inputs are used as given.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gather_sequence_latents",
    "reconstruct_sequence",
    "append",
    "softmax_rows",
    "decode",
    "prefill",
    "fit_bases",
    "projector",
    "e4m3_values",
    "quantize_e4m3",
    "append_fp8",
    "dequantize_cache",
]


def _f64(x):
    return np.asarray(x).astype(np.float64)


# ---------------------------------------------------------------------------
# Paged addressing (README, "KV-cache capacity": block size 16; the compressed
# paged format of the introduction).  Logical token t of sequence b lives in
# physical block block_tables[b, t // bs] at offset t % bs.
# ---------------------------------------------------------------------------
def gather_sequence_latents(k_cache, v_cache, block_table_row, seq_len):
    """Return the logical-order latents of one sequence.

    k_cache [NB, H, bs, r_k], v_cache [NB, r_v, bs]; block_table_row [>= ceil(L/bs)].
    Returns (ck [L, H, r_k] fp64, cv [L, r_v] fp64); H here (and in the
    rebuild and the append) counts the key/value heads.
    """
    NB, H, bs, r_k = k_cache.shape
    r_v = v_cache.shape[1]
    L = int(seq_len)
    ck = np.empty((L, H, r_k), dtype=np.float64)
    cv = np.empty((L, r_v), dtype=np.float64)
    for t in range(L):
        blk = int(block_table_row[t // bs])
        off = t % bs
        if not (0 <= blk < NB):
            raise IndexError(f"block id {blk} out of range for token {t}")
        ck[t] = k_cache[blk, :, off, :]
        cv[t] = v_cache[blk, :, off]
    return ck, cv


def reconstruct_sequence(ck, cv, U, W):
    """K^[t,h,:] = U_h c_k[t,h,:];  V^[t,h,:] = rows h*d..h*d+d-1 of W c_v[t].

    ck [L, H, r_k], cv [L, r_v], U [H, d, r_k], W [H*d, r_v]  ->  K^, V^ [L, H, d].
    """
    U = _f64(U)
    W = _f64(W)
    H, d, _ = U.shape
    L = ck.shape[0]
    # one library matmul per head for K, one for the joint V
    K = np.empty((L, H, d), dtype=np.float64)
    for h in range(H):
        K[:, h, :] = ck[:, h, :] @ U[h].T
    V = (cv @ W.T).reshape(L, H, d)
    return K, V


def append(k, v, U, W, slot_mapping, k_cache, v_cache):
    """Project new tokens to latents and write them to their paged slots.

    k, v [N, H, d] fp16; U [H, d, r_k]; W [H*d, r_v]; slot_mapping [N] ints
    (slot = block * bs + offset, negative = skip).  Returns new fp16 caches
    (copies); the inputs are not modified.  Latents are rounded to fp16 by
    numpy's round-to-nearest-even cast.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    NB, H, bs, r_k = kc.shape
    Uf = _f64(U)
    Wf = _f64(W)
    kf = _f64(k)
    vf = _f64(v)
    N = kf.shape[0]
    for n in range(N):
        slot = int(slot_mapping[n])
        if slot < 0:
            continue
        blk, off = divmod(slot, bs)
        if blk >= NB:
            raise IndexError(f"slot {slot} beyond cache")
        for h in range(H):
            kc[blk, h, off, :] = (Uf[h].T @ kf[n, h]).astype(np.float16)
        vc[blk, :, off] = (Wf.T @ vf[n].reshape(-1)).astype(np.float16)
    return kc, vc


# ---------------------------------------------------------------------------
# FP8 latents (the quantised-latent variant the adjacent pages measure for
# KV caches).  Format: OCP FP8 E4M3 -- one sign bit, four exponent bits with
# bias 7, three mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6;
# S.1111.111 is NaN and there are no infinities, so the largest finite value
# is 1.75 * 2^8 = 448.  A latent is stored as the code of c / scale with one
# scale per tensor (keys, values), rounded to nearest with ties to the even
# mantissa after clamping to +-448 (saturation); it reads back as
# scale * value(code).
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_values():
    """Value of each of the 256 E4M3 byte codes (NaN for the two NaN codes)."""
    vals = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def quantize_e4m3(x):
    """E4M3 codes (uint8) of x: clamp to +-448, then round to the nearest
    representable value with ties to the even mantissa.  The grid step in
    the binade [2^e, 2^(e+1)) is 2^(e-3); below the smallest normal 2^-6
    the step is the subnormal one, 2^-9."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    q = np.round(a / step) * step          # numpy rounds half to even
    codes = np.zeros(a.shape, dtype=np.int64)
    nz = q > 0
    eq = np.floor(np.log2(np.where(nz, q, 1.0)))   # binade of the rounded value
    sub = nz & (eq < -6)
    nrm = nz & ~sub
    codes[sub] = np.round(q[sub] / 2.0 ** -9).astype(np.int64)
    codes[nrm] = (((eq[nrm] + 7).astype(np.int64) << 3)
                  | np.round((q[nrm] / 2.0 ** eq[nrm] - 1.0) * 8.0).astype(np.int64))
    codes |= np.where(np.signbit(x), 0x80, 0)
    return codes.astype(np.uint8)


def dequantize_cache(codes, scale):
    """fp64 latents scale * value(code) of an FP8 cache."""
    return e4m3_values()[np.asarray(codes, dtype=np.uint8)] * float(scale)


def append_fp8(k, v, U, W, slot_mapping, k_scale, v_scale, k_cache8, v_cache8):
    """append() into FP8 caches (uint8 codes, same layouts): the exact fp64
    projections divided by the tensor's scale and quantised by
    quantize_e4m3.  Returns new caches (copies)."""
    kc = np.array(k_cache8, dtype=np.uint8, copy=True)
    vc = np.array(v_cache8, dtype=np.uint8, copy=True)
    NB, H, bs, r_k = kc.shape
    Uf = _f64(U)
    Wf = _f64(W)
    kf = _f64(k)
    vf = _f64(v)
    for n, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot >= 0:                  # negative slots are skipped
            blk, off = int(slot) // bs, int(slot) % bs
            if blk >= NB:
                raise IndexError(f"slot {slot} beyond cache")
            for h in range(H):
                kc[blk, h, off, :] = quantize_e4m3((Uf[h].T @ kf[n, h]) / k_scale)
            vc[blk, :, off] = quantize_e4m3((Wf.T @ vf[n].reshape(-1)) / v_scale)
    return kc, vc


def _group_size(H, U):
    """Query heads per key/value head: H over the heads of U."""
    Hkv = U.shape[0]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return H // Hkv


def softmax_rows(s):
    """Textbook two-pass softmax along the last axis (max-subtracted)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _attend(qh, Kh, Vh, scale, visible=None):
    """One head: qh [Q, d], Kh [L, d], Vh [L, d] -> (out [Q, d], p [Q, L])."""
    s = (qh @ Kh.T) * scale
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    p = softmax_rows(s)
    return p @ Vh, p


def decode(q, k_cache, v_cache, U, W, block_tables, seq_lens, scale,
           return_probs=False, batch_indices=None):
    """Decode attention: one query per sequence over all its cached tokens.

    q [B, H, d].  Returns out [B, H, d] fp64 (and, if asked, a list with the
    [H, L_b] probabilities of each sequence).  batch_indices restricts the
    work to a subset of sequences (the other rows of out stay NaN).
    """
    qf = _f64(q)
    B, H, d = qf.shape
    G = _group_size(H, U)
    out = np.full((B, H, d), np.nan)
    probs = [None] * B
    rows = range(B) if batch_indices is None else batch_indices
    for b in rows:
        L = int(seq_lens[b])
        if L == 0:
            out[b] = 0.0
            probs[b] = np.zeros((H, 0))
            continue
        ck, cv = gather_sequence_latents(k_cache, v_cache, block_tables[b], L)
        K, V = reconstruct_sequence(ck, cv, U, W)
        ph = np.empty((H, L))
        for h in range(H):
            g = h // G
            o, p = _attend(qf[b, h][None, :], K[:, g, :], V[:, g, :], scale)
            out[b, h] = o[0]
            ph[h] = p[0]
        probs[b] = ph
    if return_probs:
        return out, probs
    return out


def prefill(q, query_start_loc, k_cache, v_cache, U, W, block_tables,
            seq_lens, scale, request_indices=None):
    """Chunked-prefill attention (README, "Per-prefill-chunk attention").

    q [total_q, H, d]; request b owns query rows qsl[b] .. qsl[b+1]-1, the
    last C_b of its seq_lens[b] cached tokens (already appended).  Query j
    of the chunk sees keys 0 .. P0 + j with P0 = seq_lens[b] - C_b.
    Returns out [total_q, H, d] fp64 (rows of skipped requests stay NaN).
    """
    qf = _f64(q)
    T, H, d = qf.shape
    G = _group_size(H, U)
    out = np.full((T, H, d), np.nan)
    B = len(seq_lens)
    rows = range(B) if request_indices is None else request_indices
    for b in rows:
        q0, q1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        C = q1 - q0
        if C == 0:
            continue
        L = int(seq_lens[b])
        P0 = L - C
        if P0 < 0:
            raise ValueError("chunk longer than the sequence")
        ck, cv = gather_sequence_latents(k_cache, v_cache, block_tables[b], L)
        K, V = reconstruct_sequence(ck, cv, U, W)
        key_pos = np.arange(L)[None, :]
        qry_pos = P0 + np.arange(C)[:, None]
        visible = key_pos <= qry_pos
        for h in range(H):
            g = h // G
            o, _ = _attend(qf[q0:q1, h], K[:, g, :], V[:, g, :], scale, visible)
            out[q0:q1, h] = o
    return out


# ---------------------------------------------------------------------------
# Bases from samples.  The pages calibrate U_h and W offline by short
# knowledge distillation (README, introduction), which needs a trained model
# and stays out of scope.  The unlearned stand-in: the rank-r linear
# compression c = B^T x, x^ = B c with orthonormal B that loses the least
# squared error over the samples (Eckart-Young), i.e. B spans the top-r
# eigenspace of the uncentred second moment X^T X (X = samples as rows; no
# mean is subtracted because the reconstruction B c has no offset term).
# Keys: one basis per head from that head's keys; values: one joint basis
# from vec(v[n]) flattened head-major (row h*d + i), as in append().
# ---------------------------------------------------------------------------
def _top_eigvecs(G, r):
    """Orthonormal eigenvectors of the symmetric G for its r largest
    eigenvalues (columns, largest first), and all eigenvalues descending."""
    w, Q = np.linalg.eigh(G)  # ascending
    order = np.argsort(w)[::-1]
    return Q[:, order[:r]], w[order]


def fit_bases(k, v, r_k, r_v):
    """Least-squares bases of the samples k, v [N, H, d] (fp16).

    Returns U [H, d, r_k] and W [H*d, r_v] fp64 with orthonormal columns
    spanning the top eigenspaces of K_h^T K_h (per head) and V^T V, plus
    their descending eigenvalues (lists: per head for keys, one for values).
    The subspaces are unique when the r-th and (r+1)-th eigenvalues differ;
    the bases themselves only up to a rotation inside them.
    """
    kf = _f64(k)
    vf = _f64(v)
    N, H, d = kf.shape
    U = np.empty((H, d, r_k))
    ev_k = []
    for h in range(H):
        Kh = kf[:, h, :]
        U[h], w = _top_eigvecs(Kh.T @ Kh, r_k)
        ev_k.append(w)
    Vm = vf.reshape(N, H * d)
    W, ev_v = _top_eigvecs(Vm.T @ Vm, r_v)
    return U, W, ev_k, ev_v


def projector(B):
    """Orthogonal projector B (B^T B)^-1 B^T onto the column space of B: the
    rotation-free quantity two bases of one subspace share."""
    Bf = _f64(B)
    return Bf @ np.linalg.solve(Bf.T @ Bf, Bf.T)

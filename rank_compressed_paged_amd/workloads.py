"""Seeded synthetic inputs for paged low-rank-compressed attention.

This module only draws random numbers and lays them out in the library's
paged cache format; it holds none of the attention arithmetic, so both the
HIP path and the CPU checker can be fed from it.

Workload shapes follow the Proxima README: 32-head MHA with head size 128
and rank 64 ("Per-decode-step attention"), 16-token KV blocks ("KV-cache
capacity"), and chunked prefill of N new tokens per request
("Per-prefill-chunk attention").  Rank 64 is read as r_k = 64 per head for K
and a joint r_v = 512 for V.  Grouped-query shapes (the next step the
pages' multi-model support points to) keep H query heads and Hkv key/value
heads: U, the key latents and W's rows are per key/value head.

Draw order for one case (numpy PCG64, ``default_rng(seed)``):
  1. U_h for h = 0..Hkv-1: reduced QR of N(0,1)^{d x r_k}, column signs fixed so
     diag(R) > 0, cast to fp16;
  2. W: the same from N(0,1)^{(Hkv*d) x r_v};
  3. sequence lengths, when the config draws them (inclusive uniform);
  4. the physical block permutation ``rng.permutation(NB)``, handed out to
     (sequence, logical block) in sequence-major order;
  5. latents in logical (sequence, token) order, per sequence: c_k ~ N(0,1)
     of shape [L, Hkv, r_k] then c_v ~ N(0,1) of shape [L, r_v], drawn as
     float32 and cast to fp16 (round to nearest even);
  6. prefill only: new k, then v ([sum C, Hkv, d]), then q ~ N(0,1)
     [sum C, H, d] fp16;
     decode: q ~ N(0,1) [B, H, d] fp16.
Cache slots that hold no token (ragged tails, the spare block) are fp16 NaN
(0x7E00) so that any read of them shows up in the output.

Cache layouts: k_cache [NB, Hkv, bs, r_k] fp16, v_cache [NB, r_v, bs] fp16
(Hkv = H for multi-head attention).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

FP16_NAN_BITS = 0x7E00
E4M3_NAN_CODE = 0x7F   # OCP FP8 E4M3: S.1111.111


def draw_e4m3_codes(rng, shape):
    """Random FP8 E4M3 codes drawn as bit fields (no rounding involved):
    exponent field 1..9 (magnitudes 2^-6 .. 15), any mantissa, either sign."""
    exp = rng.integers(1, 10, size=shape)
    man = rng.integers(0, 8, size=shape)
    sign = rng.integers(0, 2, size=shape)
    return ((sign << 7) | (exp << 3) | man).astype(np.uint8)


@dataclass(frozen=True)
class Shape:
    H: int          # query heads
    d: int
    r_k: int
    r_v: int
    bs: int = 16
    Hkv: int = 0    # key/value heads (grouped-query attention); 0 means H

    @property
    def kv(self):
        """Key/value heads: the heads of U, of the key latents and of W's rows."""
        return self.Hkv or self.H


MAIN = Shape(H=32, d=128, r_k=64, r_v=512, bs=16)
TINY = Shape(H=4, d=64, r_k=16, r_v=64, bs=16)
# grouped-query layouts: 8 key/value heads for 32 query heads (groups of 4),
# and a tiny one with groups of 2
GQA8 = Shape(H=32, d=128, r_k=64, r_v=512, bs=16, Hkv=8)
# a lower rank profile of the main shape (per-layer ranks may differ)
LOWRANK = Shape(H=32, d=128, r_k=32, r_v=256, bs=16)
TINY_GQA = Shape(H=4, d=64, r_k=16, r_v=64, bs=16, Hkv=2)
# shapes without a tuned instance (the generic kernels): a conservative rank
# profile of the main shape, and an odd head count and head size
CONSERVATIVE = Shape(H=32, d=128, r_k=128, r_v=1024, bs=16)
ODD_H28 = Shape(H=28, d=96, r_k=48, r_v=640, bs=16)

# Named workloads.  "seq" is ("fixed", L) or ("uniform", lo, hi) inclusive.
CONFIGS = {
    "tiny": dict(kind="decode", shape=TINY, B=2, seq=("fixed", 256), seed=0),
    "decode_b16": dict(kind="decode", shape=MAIN, B=16, seq=("fixed", 2048), seed=1),
    "decode_b64": dict(kind="decode", shape=MAIN, B=64, seq=("uniform", 4096, 8192), seed=2),
    "long_b20": dict(kind="decode", shape=MAIN, B=20, seq=("fixed", 32768), seed=3),
    "prefill_b16": dict(kind="prefill", shape=MAIN, B=16, cached=4096, chunk=256, seed=4),
    "fit_n16384": dict(kind="fit", shape=MAIN, N=16384, seed=5),
    "gqa8_b16": dict(kind="decode", shape=GQA8, B=16, seq=("fixed", 2048), seed=6),
    "gqa8_b64": dict(kind="decode", shape=GQA8, B=64, seq=("uniform", 4096, 8192), seed=7),
    "gqa8_prefill_b16": dict(kind="prefill", shape=GQA8, B=16, cached=4096, chunk=256, seed=8),
    "tiny_gqa": dict(kind="decode", shape=TINY_GQA, B=2, seq=("fixed", 256), seed=9),
    "decode_b16_fp8": dict(kind="decode", shape=MAIN, B=16, seq=("fixed", 2048), seed=12, fp8=True),
    "decode_b64_fp8": dict(kind="decode", shape=MAIN, B=64, seq=("uniform", 4096, 8192), seed=13,
                           fp8=True),
    "prefill_b16_fp8": dict(kind="prefill", shape=MAIN, B=16, cached=4096, chunk=256, seed=14,
                            fp8=True),
    "lowrank_b16": dict(kind="decode", shape=LOWRANK, B=16, seq=("fixed", 2048), seed=10),
    "lowrank_prefill_b16": dict(kind="prefill", shape=LOWRANK, B=16, cached=4096, chunk=256,
                                seed=11),
    "conservative_b16": dict(kind="decode", shape=CONSERVATIVE, B=16, seq=("fixed", 2048),
                             seed=15),
    "odd_h28_b16": dict(kind="decode", shape=ODD_H28, B=16, seq=("fixed", 2048), seed=16),
    "conservative_prefill_b16": dict(kind="prefill", shape=CONSERVATIVE, B=16, cached=4096,
                                     chunk=256, seed=17),
}


def _nan_f16(shape):
    return np.full(shape, FP16_NAN_BITS, dtype=np.uint16).view(np.float16)


def orthonormal_fp16(rng, rows, cols):
    """Reduced QR of an N(0,1) matrix, sign-fixed, cast to fp16."""
    a = rng.standard_normal((rows, cols))
    qm, rm = np.linalg.qr(a)
    sgn = np.sign(np.diag(rm))
    sgn[sgn == 0] = 1.0
    return (qm * sgn[None, :]).astype(np.float16)


def draw_bases(rng, shape: Shape):
    U = np.stack([orthonormal_fp16(rng, shape.d, shape.r_k) for _ in range(shape.kv)])
    W = orthonormal_fp16(rng, shape.kv * shape.d, shape.r_v)
    return U, W


@dataclass
class PagedCache:
    """Block tables plus fp16 caches in the library layout."""
    shape: Shape
    seq_lens: np.ndarray          # [B] int32, tokens in the cache
    block_tables: np.ndarray      # [B, max_blocks] int32, -1 = unused
    k_cache: np.ndarray           # [NB, Hkv, bs, r_k] fp16
    v_cache: np.ndarray           # [NB, r_v, bs] fp16
    logical_ck: Optional[List[np.ndarray]] = None  # per sequence [L, H, r_k]
    logical_cv: Optional[List[np.ndarray]] = None  # per sequence [L, r_v]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]


def build_block_tables(rng, blocks_per_seq: Sequence[int], spare_blocks=1,
                       shuffle=True, extra_cols=0):
    nb = int(sum(blocks_per_seq)) + int(spare_blocks)
    perm = rng.permutation(nb)          # drawn either way: the later draws stay the same
    if not shuffle:
        perm = np.arange(nb)
    max_blocks = max([int(x) for x in blocks_per_seq] + [1]) + int(extra_cols)
    bt = np.full((len(blocks_per_seq), max_blocks), -1, dtype=np.int32)
    i = 0
    for b, n in enumerate(blocks_per_seq):
        bt[b, :n] = perm[i:i + n]
        i += n
    return bt, nb


def scatter_tokens(k_cache, v_cache, table_row, t0, ck, cv, bs):
    """Place logical tokens t0..t0+len-1 (ck [n,H,r_k], cv [n,r_v]) in their pages."""
    n = ck.shape[0]
    t = t0 + np.arange(n)
    blk = table_row[t // bs]
    off = t % bs
    k_cache[blk, :, off, :] = ck
    v_cache[blk, :, off] = cv


def fill_cache(rng, shape: Shape, seq_lens, cache_lens=None, spare_blocks=1,
               shuffle=True, keep_logical=False, extra_cols=0, fp8=False):
    """Block tables for seq_lens tokens, latents drawn for the first cache_lens
    (fp16 N(0,1); or, with fp8, FP8 E4M3 codes from draw_e4m3_codes, unused
    slots holding the NaN code)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    cache_lens = seq_lens if cache_lens is None else np.asarray(cache_lens, dtype=np.int32)
    bs = shape.bs
    nblk = [(int(L) + bs - 1) // bs for L in seq_lens]
    bt, nb = build_block_tables(rng, nblk, spare_blocks, shuffle, extra_cols)
    if fp8:
        kc = np.full((nb, shape.kv, bs, shape.r_k), E4M3_NAN_CODE, dtype=np.uint8)
        vc = np.full((nb, shape.r_v, bs), E4M3_NAN_CODE, dtype=np.uint8)
    else:
        kc = _nan_f16((nb, shape.kv, bs, shape.r_k))
        vc = _nan_f16((nb, shape.r_v, bs))
    lck, lcv = [], []
    for b, L in enumerate(cache_lens):
        L = int(L)
        if fp8:
            ck = draw_e4m3_codes(rng, (L, shape.kv, shape.r_k))
            cv = draw_e4m3_codes(rng, (L, shape.r_v))
        else:
            ck = rng.standard_normal((L, shape.kv, shape.r_k), dtype=np.float32).astype(np.float16)
            cv = rng.standard_normal((L, shape.r_v), dtype=np.float32).astype(np.float16)
        if L:
            scatter_tokens(kc, vc, bt[b], 0, ck, cv, bs)
        if keep_logical:
            lck.append(ck)
            lcv.append(cv)
    return PagedCache(shape, seq_lens, bt, kc, vc,
                      lck if keep_logical else None, lcv if keep_logical else None)


@dataclass
class DecodeCase:
    shape: Shape
    U: np.ndarray          # [Hkv, d, r_k] fp16
    W: np.ndarray          # [Hkv*d, r_v] fp16
    cache: PagedCache
    q: np.ndarray          # [B, H, d] fp16
    scale: float
    seed: int = 0
    name: str = ""
    k_scale: float = 1.0   # FP8 caches: per-tensor scales of the codes
    v_scale: float = 1.0

    @property
    def B(self):
        return self.q.shape[0]


@dataclass
class PrefillCase:
    shape: Shape
    U: np.ndarray
    W: np.ndarray
    cache: PagedCache               # caches hold the first cached_lens tokens
    cached_lens: np.ndarray         # [B] tokens already in the cache
    k_new: np.ndarray               # [T, Hkv, d] fp16, T = sum of chunk lengths
    v_new: np.ndarray               # [T, Hkv, d] fp16
    q: np.ndarray                   # [T, H, d] fp16
    slot_mapping: np.ndarray        # [T] int64 slot of each new token
    query_start_loc: np.ndarray     # [B+1] int32
    scale: float
    seed: int = 0
    name: str = ""
    k_scale: float = 1.0            # FP8 caches: per-tensor scales of the codes
    v_scale: float = 1.0

    @property
    def seq_lens(self):
        return self.cache.seq_lens


def draw_seq_lens(rng, B, seq):
    if seq[0] == "fixed":
        return np.full(B, int(seq[1]), dtype=np.int32)
    if seq[0] == "uniform":
        return rng.integers(int(seq[1]), int(seq[2]), size=B, endpoint=True).astype(np.int32)
    raise ValueError(seq)


def _pow2(mult):
    m = float(mult)
    if m <= 0 or 2.0 ** round(np.log2(m)) != m:
        raise ValueError("q_mult must be a power of two (exact in fp16)")
    return m


def plant_key_pairs(cache: PagedCache, where, factor):
    """Sharpen the scores without touching the draws' order: in each sequence
    and each chosen page ("first", "mid", "last"), the key latents of page
    offsets 3 and 9 become +factor and -factor times offset 3's draw (fp16),
    so one of the pair scores far above the rest in every head whatever the
    query's sign.  Pages shorter than 10 tokens are skipped."""
    bs = cache.shape.bs
    for b, L in enumerate(cache.seq_lens):
        n_pages = (int(L) + bs - 1) // bs
        for w in where:
            p = {"first": 0, "mid": n_pages // 2, "last": n_pages - 1}[w]
            if p < 0 or (p + 1) * bs > int(L) and int(L) - p * bs < 10:
                continue
            blk = int(cache.block_tables[b, p])
            base = cache.k_cache[blk, :, 3, :].astype(np.float32)
            cache.k_cache[blk, :, 3, :] = (base * factor).astype(np.float16)
            cache.k_cache[blk, :, 9, :] = (-base * factor).astype(np.float16)


def ramp_keys(cache: PagedCache, ramp, lens=None):
    """Key latents of token t scaled by 1 + ramp * t / L (fp16), so scores and
    their running maximum rise along each sequence (L = lens[b], default the
    sequence length; only the first L tokens are touched)."""
    bs = cache.shape.bs
    lens = cache.seq_lens if lens is None else lens
    for b, L in enumerate(lens):
        L = int(L)
        for t in range(L):
            blk = int(cache.block_tables[b, t // bs])
            f = 1.0 + ramp * t / max(int(cache.seq_lens[b]), 1)
            cache.k_cache[blk, :, t % bs, :] = (
                cache.k_cache[blk, :, t % bs, :].astype(np.float32) * f).astype(np.float16)


def make_decode_case(shape: Shape, seq_lens=None, B=None, seq=None, seed=0,
                     spare_blocks=1, shuffle=True, keep_logical=False,
                     bases=None, extra_cols=0, name="", fp8=False, q_mult=1,
                     plant=(), plant_factor=12.0, ramp=0.0):
    """One decode step: B sequences of seq_lens tokens, one query each.  With
    fp8 the caches hold FP8 E4M3 codes read with k_scale 1/4, v_scale 1/8
    (latent magnitudes up to about 4 and 2).  Sharper softmax rows, with the
    same draws: q_mult (a power of two) scales q; plant puts a dominant +/-
    key pair on the first / middle / last page (fp16 only); ramp makes the
    scores rise along each sequence (fp16 only)."""
    rng = np.random.default_rng(seed)
    if bases is None:
        U, W = draw_bases(rng, shape)
    else:
        U, W = (np.asarray(x, dtype=np.float16) for x in bases)
    if seq_lens is None:
        seq_lens = draw_seq_lens(rng, B, seq)
    cache = fill_cache(rng, shape, seq_lens, spare_blocks=spare_blocks,
                       shuffle=shuffle, keep_logical=keep_logical, extra_cols=extra_cols,
                       fp8=fp8)
    q = rng.standard_normal((len(cache.seq_lens), shape.H, shape.d),
                            dtype=np.float32).astype(np.float16)
    if q_mult != 1:
        q = (q.astype(np.float32) * _pow2(q_mult)).astype(np.float16)
    if (plant or ramp) and fp8:
        raise ValueError("planted and ramped keys are fp16-cache options")
    if plant:
        plant_key_pairs(cache, plant, plant_factor)
    if ramp:
        ramp_keys(cache, ramp)
    if fp8:
        return DecodeCase(shape, U, W, cache, q, 1.0 / np.sqrt(shape.d), seed, name, 0.25, 0.125)
    return DecodeCase(shape, U, W, cache, q, 1.0 / np.sqrt(shape.d), seed, name)


def make_prefill_case(shape: Shape, cached_lens, chunk_lens, seed=0,
                      spare_blocks=1, shuffle=True, keep_logical=False,
                      bases=None, name="", fp8=False, q_mult=1, ramp=0.0):
    """One chunked-prefill step: request b has cached_lens[b] latent tokens and
    appends chunk_lens[b] new full-precision tokens, then attends causally.
    With fp8 the cached latents are FP8 E4M3 codes (k_scale 1/16, v_scale
    1/16, so that the chunk's own projections also fit the format).  Sharper
    rows with the same draws: q_mult (a power of two) scales q; ramp scales
    cached key latents and the chunk's new keys by 1 + ramp * t / L at
    absolute position t (fp16 only), so the scores' maximum rises along the
    request, also inside the chunk."""
    rng = np.random.default_rng(seed)
    if bases is None:
        U, W = draw_bases(rng, shape)
    else:
        U, W = (np.asarray(x, dtype=np.float16) for x in bases)
    cached_lens = np.asarray(cached_lens, dtype=np.int32)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int32)
    total = cached_lens + chunk_lens
    cache = fill_cache(rng, shape, total, cache_lens=cached_lens,
                       spare_blocks=spare_blocks, shuffle=shuffle,
                       keep_logical=keep_logical, fp8=fp8)
    T = int(chunk_lens.sum())
    dims = (T, shape.H, shape.d)
    kv_dims = (T, shape.kv, shape.d)
    k_new = rng.standard_normal(kv_dims, dtype=np.float32).astype(np.float16)
    v_new = rng.standard_normal(kv_dims, dtype=np.float32).astype(np.float16)
    q = rng.standard_normal(dims, dtype=np.float32).astype(np.float16)
    qsl = np.zeros(len(chunk_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(chunk_lens)
    if q_mult != 1:
        q = (q.astype(np.float32) * _pow2(q_mult)).astype(np.float16)
    if ramp:
        if fp8:
            raise ValueError("ramped keys are an fp16-cache option")
        ramp_keys(cache, ramp, lens=cached_lens)
        for b in range(len(chunk_lens)):
            L = int(total[b])
            for j in range(int(chunk_lens[b])):
                t = int(cached_lens[b]) + j
                n = qsl[b] + j
                k_new[n] = (k_new[n].astype(np.float32) * (1.0 + ramp * t / L)).astype(np.float16)
    slots = np.empty(T, dtype=np.int64)
    bs = shape.bs
    for b in range(len(chunk_lens)):
        pos = cached_lens[b] + np.arange(chunk_lens[b])
        slots[qsl[b]:qsl[b + 1]] = (cache.block_tables[b, pos // bs].astype(np.int64) * bs
                                    + pos % bs)
    if fp8:
        return PrefillCase(shape, U, W, cache, cached_lens, k_new, v_new, q, slots, qsl,
                           1.0 / np.sqrt(shape.d), seed, name, 1.0 / 16, 1.0 / 16)
    return PrefillCase(shape, U, W, cache, cached_lens, k_new, v_new, q, slots, qsl,
                       1.0 / np.sqrt(shape.d), seed, name)


@dataclass
class FitCase:
    """K/V samples for fitting the bases, plus the starting matrices."""
    shape: Shape
    k: np.ndarray      # [N, H, d] fp16
    v: np.ndarray      # [N, H, d] fp16
    u0: np.ndarray     # [H, d, r_k] fp32
    w0: np.ndarray     # [H*d, r_v] fp32
    seed: int
    name: str = ""


def make_fit_case(shape: Shape, N, seed=0, noise=0.05, name="", spectrum="planted"):
    """K/V samples for the bases fit, with one of three spectra.

    spectrum "power" or "exp" (decaying spectra with no gap at the rank, as
    real K/V are): per head an orthonormal d x d frame A_h (reduced QR of
    N(0,1), sign-fixed), then one (H*d) x (H*d) frame B; coefficients z_k ~
    N(0,1) [N, H, d] and z_v ~ N(0,1) [N, H*d]; then u0, w0 as below.
    k[n, h] = A_h (s_k * z_k[n, h]) and vec(v[n]) = B (s_v * z_v[n]) with
    s^2 (the second moment's spectrum up to sampling) falling as (i + 1)^-2
    ("power") or exp(-4 i / r) ("exp", r the side's rank), scaled to a largest
    s of 4.  The eigenvalue ratio at the rank is then about (r / (r+1))^2 or
    exp(-4 / r): subspace iteration needs hundreds of steps.

    spectrum "planted" (the default):

    Draw order (numpy PCG64, ``default_rng(seed)``):
      1. per head h: an orthonormal d x r_k frame A_h (reduced QR of N(0,1),
         sign-fixed, fp64); then the value frame B, (H*d) x r_v, the same way;
      2. key coefficients z_k ~ N(0,1) [N, H, r_k], key noise e_k ~ N(0,1)
         [N, H, d]; value coefficients z_v ~ N(0,1) [N, r_v], value noise
         e_v ~ N(0,1) [N, H*d];
      3. u0 ~ N(0,1) [H, d, r_k], w0 ~ N(0,1) [H*d, r_v] (fp32).
    k[n, h] = A_h (s_k * z_k[n, h]) + noise * e_k[n, h] and
    vec(v[n]) = B (s_v * z_v[n]) + noise * e_v[n], with per-direction scales
    s falling linearly from 3 to 1, cast to fp16.  The r-th eigenvalue of the
    second moment then sits near N (1 + noise^2) and the (r+1)-th near
    N noise^2, a wide gap.
    """
    rng = np.random.default_rng(seed)

    def frame(rows, cols):
        a = rng.standard_normal((rows, cols))
        qm, rm = np.linalg.qr(a)
        sgn = np.sign(np.diag(rm))
        sgn[sgn == 0] = 1.0
        return qm * sgn[None, :]

    H, d, rk, rv = shape.H, shape.d, shape.r_k, shape.r_v
    if spectrum in ("power", "exp"):
        def scales(m, r):
            i = np.arange(m, dtype=np.float64)
            s2 = (i + 1.0) ** -2.0 if spectrum == "power" else np.exp(-4.0 * i / r)
            return 4.0 * np.sqrt(s2 / s2[0])
        A = np.stack([frame(d, d) for _ in range(H)])        # [H, d, d]
        B = frame(H * d, H * d)
        zk = rng.standard_normal((N, H, d))
        zv = rng.standard_normal((N, H * d))
        k = np.einsum("hde,nhe->nhd", A, zk * scales(d, rk))
        v = (zv * scales(H * d, rv)) @ B.T
        u0 = rng.standard_normal((H, d, rk), dtype=np.float32)
        w0 = rng.standard_normal((H * d, rv), dtype=np.float32)
        return FitCase(shape, k.astype(np.float16), v.reshape(N, H, d).astype(np.float16),
                       u0, w0, seed, name)
    if spectrum != "planted":
        raise ValueError(spectrum)
    A = np.stack([frame(d, rk) for _ in range(H)])          # [H, d, rk]
    B = frame(H * d, rv)                                     # [H*d, rv]
    zk = rng.standard_normal((N, H, rk))
    ek = rng.standard_normal((N, H, d))
    zv = rng.standard_normal((N, rv))
    ev = rng.standard_normal((N, H * d))
    sk = np.linspace(3.0, 1.0, rk)
    sv = np.linspace(3.0, 1.0, rv)
    k = np.einsum("hdr,nhr->nhd", A, zk * sk) + noise * ek
    v = (zv * sv) @ B.T + noise * ev
    u0 = rng.standard_normal((H, d, rk), dtype=np.float32)
    w0 = rng.standard_normal((H * d, rv), dtype=np.float32)
    return FitCase(shape, k.astype(np.float16), v.reshape(N, H, d).astype(np.float16),
                   u0, w0, seed, name)


def make_config(name: str, keep_logical=False):
    """Build a named workload with its own seed."""
    cfg = CONFIGS[name]
    shape = cfg["shape"]
    if cfg["kind"] == "fit":
        return make_fit_case(shape, cfg["N"], seed=cfg["seed"], name=name)
    if cfg["kind"] == "decode":
        return make_decode_case(shape, B=cfg["B"], seq=cfg["seq"], seed=cfg["seed"],
                                keep_logical=keep_logical, name=name, fp8=cfg.get("fp8", False))
    B = cfg["B"]
    return make_prefill_case(shape, [cfg["cached"]] * B, [cfg["chunk"]] * B,
                             seed=cfg["seed"], keep_logical=keep_logical, name=name,
                             fp8=cfg.get("fp8", False))

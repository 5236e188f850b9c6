"""Work and byte accounting for the roofline figures.

Latent bytes per cached token (fp16): H*r_k for the head-wise key latents
plus r_v for the joint value latent, times two bytes.  Dense bytes per token
(one layer, K and V): 2*H*d*2.  The Proxima README's capacity tables ("KV-cache
capacity", "Long-context capacity") are consistent with these at H = 32,
d = 128, r_k = 64, r_v = 512 (checked in the tests against the printed
numbers).
"""
from __future__ import annotations

import numpy as np

FP16_BYTES = 2


def latent_bytes_per_token(H, r_k, r_v, elt=FP16_BYTES):
    return (H * r_k + r_v) * elt


def dense_bytes_per_token(H, d, elt=FP16_BYTES):
    return 2 * H * d * elt


def basis_bytes(H, d, r_k, r_v, elt=FP16_BYTES):
    """U (H*d*r_k) plus W (H*d*r_v) per layer."""
    return (H * d * r_k + H * d * r_v) * elt


def decode_latent_bytes(seq_lens, H, r_k, r_v):
    """Algorithmic bytes of one decode step: every cached latent read once."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * latent_bytes_per_token(H, r_k, r_v)


def decode_flops(seq_lens, H, r_k, r_v):
    """Scores (2*r_k per head) plus P.c_v (2*r_v per head) per (sequence, token)."""
    tokens = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    return tokens * H * (2 * r_k + 2 * r_v)


def prefill_pairs(cached_lens, chunk_lens):
    """(query, key) pairs under the causal rule: C*P0 + C*(C+1)/2 per request."""
    c = np.asarray(chunk_lens, dtype=np.int64)
    p0 = np.asarray(cached_lens, dtype=np.int64)
    return int(np.sum(c * p0 + c * (c + 1) // 2))


def prefill_flops(cached_lens, chunk_lens, H, d, r_k, r_v):
    """q projection + scores + P.c_v + up-projection, 2 flops per MAC."""
    c = int(np.sum(np.asarray(chunk_lens, dtype=np.int64)))
    pairs = prefill_pairs(cached_lens, chunk_lens)
    return 2 * H * (c * d * r_k + pairs * r_k + pairs * r_v + c * r_v * d)


def append_flops(n_tokens, H, d, r_k, r_v):
    return 2 * n_tokens * (H * d * r_k + H * d * r_v)


def gram_flops(n_samples, H, d):
    """The bases fit's second moments: the n(n+1)/2 distinct entries of
    V^T V (n = H*d) and of each K_h^T K_h (n = d), one MAC per sample each,
    2 flops per MAC."""
    nv = H * d
    return int(n_samples) * (nv * (nv + 1) + H * d * (d + 1))


def fit_iteration_flops(H, d, r_k, r_v):
    """One subspace-iteration step of the bases fit, 2 flops per MAC: Y = G Q
    (n^2 r), S = Y^T Y (n r(r+1)/2 distinct), Q = Y L^-T (n r(r+1)/2), for the
    value problem (n = H*d) and the H key problems (n = d); the r^3/3 of the
    Cholesky factorisation is left out."""
    def one(n, r):
        return 2 * (n * n * r + n * r * (r + 1))
    return one(H * d, r_v) + H * one(d, r_k)

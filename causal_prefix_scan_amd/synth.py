"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the attention arithmetic, so the CPU oracle and the HIP
path can both be fed from it without sharing any of the method.

Recipe (the pages use no dataset; every workload is synthetic):
  * numpy.random.default_rng(seed) (PCG64); draws in the order q, k, v, then
    the per-head decay, each as float32 standard normals of the full shape;
  * q, k, v are scaled by 1/sqrt(d) (v by 1/sqrt(dv));
  * optional per-token L2 normalisation of k, in float32, before rounding;
  * rounding to bf16 is round-to-nearest-even on the float32 bit pattern;
  * per-head decay gamma_h = 1 - exp(U[ln 1e-3, ln 1e-1]) in float32, the
    same for every batch element;
  * decode steps draw from default_rng([seed, 1 + step]) so any step can be
    regenerated on its own;
  * an upstream gradient dO for the backward is float32 standard normal of
    the output's shape, from default_rng([seed, 0]).
"""

import math

import numpy as np

__all__ = ["bf16_round", "FwdInputs", "make_fwd_inputs", "make_decode_prefix",
           "make_decode_step", "make_upstream_grad", "FWD_WORKLOADS", "DECODE_WORKLOAD"]


def bf16_round(x):
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns (values as float32, raw bf16 bit patterns as uint16).  Inputs are
    finite here, so no NaN special case is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    hi = rounded.astype(np.uint16)
    vals = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, hi


class FwdInputs:
    """Inputs of one forward workload.

    q, k: float32 [B, H, T, d]; v: float32 [B, H, T, dv] -- the exact values
    the GPU receives (already bf16-representable when dtype == "bf16").
    q_bits/k_bits/v_bits: uint16 bf16 patterns (dtype "bf16") or None.
    gamma: float32 [H] or None (no decay).
    """

    def __init__(self, q, k, v, gamma, dtype, bits=None):
        self.q, self.k, self.v = q, k, v
        self.gamma = gamma
        self.dtype = dtype
        self.q_bits, self.k_bits, self.v_bits = bits if bits is not None else (None, None, None)

    @property
    def shape(self):
        B, H, T, d = self.q.shape
        return B, H, T, d, self.v.shape[3]

    def units(self):
        """Views flattened over units u = b*H + h: ([U,T,d], [U,T,d], [U,T,dv], gamma [U] or None)."""
        B, H, T, d, dv = self.shape
        g = None if self.gamma is None else np.tile(self.gamma, B)
        return (self.q.reshape(B * H, T, d), self.k.reshape(B * H, T, d),
                self.v.reshape(B * H, T, dv), g)


def _draw_decay(rng, H):
    lo, hi = math.log(1e-3), math.log(1e-1)
    one_minus = np.exp(rng.uniform(lo, hi, size=H)).astype(np.float32)
    return (np.float32(1.0) - one_minus).astype(np.float32)


def make_fwd_inputs(B, H, T, d, dv, dtype="bf16", seed=0, k_l2norm=False, decay=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    k = rng.standard_normal((B, H, T, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32) * np.float32(1.0 / math.sqrt(dv))
    if k_l2norm:
        nrm = np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32))
        k = (k / np.maximum(nrm, np.float32(1e-30))).astype(np.float32)
    gamma = _draw_decay(rng, H) if decay else None
    if dtype == "bf16":
        (q, qb), (k, kb), (v, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
        return FwdInputs(q, k, v, gamma, dtype, (qb, kb, vb))
    if dtype == "f32":
        return FwdInputs(q, k, v, gamma, dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_upstream_grad(B, H, T, dv, seed):
    """Upstream gradient dL/do, float32 [B, H, T, dv], standard normal."""
    rng = np.random.default_rng([seed, 0])
    return rng.standard_normal((B, H, T, dv), dtype=np.float32)


def make_decode_prefix(n_seq, H, d, dv, prefix_len, seed, n_unique=None):
    """Prefix tokens for the decode workload, bf16-rounded, [U, prefix_len, .]
    with U = n_unique (default n_seq*H) distinct prefixes."""
    U = n_seq * H if n_unique is None else n_unique
    inp = make_fwd_inputs(1, U, prefix_len, d, dv, "bf16", seed)
    return inp


def make_decode_step(n_seq, H, d, dv, seed, step):
    """The new token of every (sequence, head) at one decode step, bf16.
    Returns (q, k, v float32 values [N*H, d|dv], (q_bits, k_bits, v_bits))."""
    rng = np.random.default_rng([seed, 1 + step])
    U = n_seq * H
    q = rng.standard_normal((U, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    k = rng.standard_normal((U, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    v = rng.standard_normal((U, dv), dtype=np.float32) * np.float32(1.0 / math.sqrt(dv))
    (q, qb), (k, kb), (v, vb) = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v, (qb, kb, vb)


# The forward workloads, named by what they are.  `chunk` is the number of
# tokens per materialised segment summary; `credit_chunk` is the chunk length
# at which the algorithmic flops per token are counted (the 64-token tile when
# the segments are longer than that).
FWD_WORKLOADS = {
    "fwd_f32_b1h1t256d16": dict(B=1, H=1, T=256, d=16, dv=16, dtype="f32", seed=0,
                                chunk=32, credit_chunk=32, normalize=False, eps=0.0,
                                k_l2norm=False, decay=False, tol=1e-4),
    "fwd_norm_bf16_b2h8t4096d64": dict(B=2, H=8, T=4096, d=64, dv=64, dtype="bf16", seed=1,
                                       chunk=64, credit_chunk=64, normalize=True, eps=1e-6,
                                       k_l2norm=True, decay=False, tol=2e-2),
    "fwd_decay_bf16_b4h16t16384d128": dict(B=4, H=16, T=16384, d=128, dv=128, dtype="bf16",
                                           seed=2, chunk=4096, credit_chunk=64, normalize=False,
                                           eps=0.0, k_l2norm=False, decay=True, tol=2e-2),
    "fwd_bf16_b1h32t65536d64": dict(B=1, H=32, T=65536, d=64, dv=64, dtype="bf16", seed=3,
                                    chunk=128, credit_chunk=128, normalize=False, eps=0.0,
                                    k_l2norm=False, decay=False, tol=2e-2),
}

DECODE_WORKLOAD = ("decode_bf16_n64h32d128",
                   dict(n_seq=64, H=32, d=128, dv=128, prefix_len=2048, steps=1024, seed=4,
                        normalize=True, eps=1e-6, tol=2e-2))

"""GPU parity of the backward pass (gradients of the unnormalised masked forward).

Calls go through the C ABI (hla_bwd, via the ctypes binding).  Small cases
are compared element by element with the oracle's float64 autograd of the
masked matrix form (ragged tiles, one or many segments, d != dv, decay, both
input dtypes); the full-size decayed B4 H16 T16384 d128 workload runs in the
launch configuration the benchmark times and is compared on sampled
(batch, head) units with the oracle's serial forward/reverse state form
(pinned to autograd and to finite differences in the CPU tests).

Tolerance (max|got - want| / max|want|), from the precision the kernels
contract in, which follows the forward: fp32 inputs stay fp32 end to end
(fp32 MFMA), so 1e-4 covers fp32 rounding over sums of a few thousand terms;
bf16 inputs contract in bf16 with fp32 accumulation, and the fp32
intermediates p, dp and the upstream gradient are rounded to bf16 (relative
error 2^-9 per operand) before their products, so the bound is the forward's
2e-2.
"""

import numpy as np
import pytest

from causal_prefix_scan_amd import hla, synth
from oracle import hla_backward_oracle as BO

from gpu_util import host, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()          # raises if the HIP library is missing: no silent fallback
    return torch


# (B, H, T, d, dv, chunk, dtype, decay)
SMALL = [
    (1, 2, 128, 16, 32, 64, "bf16", True),        # d below one bf16 MFMA step (zero padding)
    (1, 2, 256, 16, 16, 64, "f32", False),
    (1, 1, 200, 32, 32, 100, "bf16", True),       # 3 tiles + ragged 4 per segment
    (2, 1, 320, 64, 32, 64, "bf16", True),        # n = 5, d > dv
    (1, 2, 256, 128, 128, 256, "bf16", False),    # n = 1 (no segment scan)
    (1, 1, 384, 128, 64, 96, "bf16", True),       # n = 4
    (1, 2, 192, 64, 128, 64, "bf16", True),       # d < dv
    (1, 1, 96, 64, 64, 32, "f32", True),          # n = 3
    (1, 1, 600, 32, 64, 200, "bf16", False),      # ragged 8-token last tile
    (1, 2, 144, 64, 64, 48, "f32", True),         # fp32, n = 3, a 32-token tile + a ragged 16 per segment
]


def case_id(c):
    B, H, T, d, dv, chunk, dt, dec = c
    return f"B{B}H{H}T{T}d{d}dv{dv}c{chunk}-{dt}{'-decay' if dec else ''}"


def upstream(torch, B, H, T, dv, seed):
    do = synth.make_upstream_grad(B, H, T, dv, seed)
    return do, torch.from_numpy(do).cuda()


@pytest.mark.parametrize("case", SMALL, ids=[case_id(c) for c in SMALL])
def test_bwd_matches_autograd(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dt, decay = case
    say("backward case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dt, seed=500 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    do_h, do = upstream(torch, B, H, T, dv, 500 + T)
    dq, dk, dvv = hla.bwd(q, k, v, do, chunk, g)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    want = BO.grad_autograd(uq, uk, uv, do_h.reshape(B * H, T, dv), ug)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dvv), want):
        e = rel_err(host(got).reshape(w.shape), w)
        tol = 1e-4 if dt == "f32" else 2e-2
        say(f"  {name} {e:.3e}  (tol {tol})")
        assert e <= tol, name


# (B, H, T, d, dv, chunk, dtype, decay): the ratio-normalised output
NORM = [
    (1, 2, 256, 64, 64, 64, "bf16", True),
    (1, 1, 200, 32, 64, 100, "bf16", False),      # ragged tiles, d < dv
    (1, 2, 384, 128, 128, 96, "bf16", True),      # n = 4, 8-wave forward
    (2, 1, 192, 64, 32, 64, "f32", True),         # fp32, d > dv
    (1, 1, 128, 16, 16, 32, "f32", False),        # d = 16 (the v = 1 sums at width 16)
]


@pytest.mark.parametrize("case", NORM, ids=[case_id(c) + "-norm" for c in NORM])
def test_bwd_normalised_matches_autograd(gpu, case):
    """Gradient of o = num / (den + eps) against float64 autograd of the same
    quotient.  q and k are taken in absolute value (exact in bf16), so every
    q.k is positive and den stays well away from 0: the quotient's gradient
    is then as well conditioned as the numerator's."""
    torch = gpu
    B, H, T, d, dv, chunk, dt, decay = case
    say("normalised backward case", case_id(case))
    eps = 1e-6
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dt, seed=700 + T + d, decay=decay)
    inp.q, inp.k = np.abs(inp.q), np.abs(inp.k)
    if dt == "bf16":
        inp.q_bits = inp.q_bits & np.uint16(0x7FFF)
        inp.k_bits = inp.k_bits & np.uint16(0x7FFF)
    q, k, v, g = to_dev(inp)
    do_h, do = upstream(torch, B, H, T, dv, 700 + T)
    dq, dk, dvv = hla.bwd(q, k, v, do, chunk, g, normalize=True, eps=eps)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    want = BO.grad_autograd(uq, uk, uv, do_h.reshape(B * H, T, dv), ug, normalize=True, eps=eps)
    tol = 1e-4 if dt == "f32" else 2e-2
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dvv), want):
        e = rel_err(host(got).reshape(w.shape), w)
        say(f"  {name} {e:.3e}  (tol {tol})")
        assert e <= tol, name
    # the unnormalised gradient differs (the quotient is not a rescaling)
    dq0, _, _ = hla.bwd(q, k, v, do, chunk, g)
    torch.cuda.synchronize()
    assert rel_err(host(dq0), host(dq)) > 1e-2


def test_bwd_gamma_zero_closed_form(gpu):
    # gamma = 0 keeps only i = j = t: o_t = (q_t.k_t)^2 v_t
    torch = gpu
    B, H, T, d, dv = 1, 2, 192, 64, 64
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=531)
    q, k, v, _ = to_dev(inp)
    g = torch.zeros(H, dtype=torch.float32, device="cuda")
    do_h, do = upstream(torch, B, H, T, dv, 531)
    dq, dk, dvv = hla.bwd(q, k, v, do, 64, g)
    torch.cuda.synchronize()
    qh, kh, vh = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    qk = np.sum(qh * kh, axis=-1)
    dov = np.sum(do_h * vh, axis=-1)
    assert rel_err(host(dvv), (qk ** 2)[..., None] * do_h) <= 2e-2
    assert rel_err(host(dq), (2 * qk * dov)[..., None] * kh) <= 2e-2
    assert rel_err(host(dk), (2 * qk * dov)[..., None] * qh) <= 2e-2


def test_bwd_is_deterministic(gpu):
    torch = gpu
    B, H, T, d, dv = 1, 2, 512, 128, 128
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=532, decay=True)
    q, k, v, g = to_dev(inp)
    _, do = upstream(torch, B, H, T, dv, 532)
    a = hla.bwd(q, k, v, do, 128, g)
    b = hla.bwd(q, k, v, do, 128, g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_chunk_does_not_change_the_result(gpu):
    # the segment length only regroups the sums (fp32 inputs: no bf16 rounding
    # of intermediates that a regrouped sum could tip)
    torch = gpu
    B, H, T, d, dv = 1, 1, 1024, 64, 64
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "f32", seed=533, decay=True)
    q, k, v, g = to_dev(inp)
    _, do = upstream(torch, B, H, T, dv, 533)
    a = hla.bwd(q, k, v, do, 1024, g)
    b = hla.bwd(q, k, v, do, 64, g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert rel_err(host(y), host(x)) <= 1e-5


def test_bwd_full_size_sampled_units(gpu):
    # B4 H16 T16384 d128, decayed: the benchmark's backward workload and chunk
    torch = gpu
    from bench import BWD_CHUNK
    B, H, T, d, dv = 4, 16, 16384, 128, 128
    say("backward full size B4 H16 T16384 d128, chunk", BWD_CHUNK)
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=2, decay=True)
    q, k, v, g = to_dev(inp)
    do_h, do = upstream(torch, B, H, T, dv, 2)
    dq, dk, dvv = hla.bwd(q, k, v, do, BWD_CHUNK, g)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    dou = do_h.reshape(B * H, T, dv)
    for u in (0, 37):
        want = BO.grad_states(uq[u:u + 1], uk[u:u + 1], uv[u:u + 1], dou[u:u + 1], ug[u:u + 1])
        for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dvv), want):
            e = rel_err(host(got.reshape(B * H, T, -1)[u]), w[0])
            say(f"  unit {u} {name} {e:.3e}")
            assert e <= 2e-2, (u, name)

"""GPU parity of the third-order HLA path against the fp64 CPU oracle
(oracle/hla3_oracle.py), through the C ABI.

Stage by stage on small cases: every segment's summary (moments S, Q, P, m
and cross summaries V, Z, z, R, r) against the oracle's segment_summary3;
the exclusive prefixes and inclusive totals of hla3_scan (moments by a
decayed running sum, R and r through the segment map) against the oracle's
Blelloch scan under combine3; hla3_fwd's num and den against the pages-form
serial recurrence serial3.  Then gamma = 0, the decode step, prefill ->
decode, and sampled units of B4 H16 T16384 d128 (decayed) in the launch
configuration the benchmark times.

Tolerances: max|got - want| / max|want| <= 1e-4 (fp32 inputs), <= 2e-2 (bf16
inputs with fp32 state), as for the second order.
"""

import numpy as np
import pytest

from causal_prefix_scan_amd import hla, synth
from oracle import hla3_oracle as O3

from gpu_util import host, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()          # raises if the HIP library is missing: no silent fallback
    return torch


def tol_of(dtype):
    return 1e-4 if dtype == "f32" else 2e-2


# (B, H, T, d, dv, chunk, dtype, decay)
CASES = [
    (1, 2, 256, 16, 16, 64, "f32", False),
    (1, 2, 192, 32, 64, 64, "bf16", True),      # n = 3
    (2, 1, 320, 64, 32, 64, "bf16", True),      # n = 5, d > dv
    (1, 2, 384, 64, 64, 96, "bf16", False),     # a ragged 32-token tile per segment
    (1, 1, 512, 128, 128, 128, "bf16", True),   # n = 4
    (1, 2, 256, 128, 64, 256, "bf16", True),    # n = 1
    (1, 1, 192, 32, 32, 48, "f32", True),       # fp32, n = 4, ragged 16
    (1, 2, 600, 64, 128, 200, "bf16", True),    # 3 tiles + ragged 8, d < dv
    (1, 2, 768, 32, 32, 64, "bf16", True),      # n = 12
    (1, 1, 576, 128, 128, 64, "bf16", True),    # n = 9 at d = 128 (eight waves per segment)
]


def cid(c):
    B, H, T, d, dv, chunk, dt, dec = c
    return f"B{B}H{H}T{T}d{d}dv{dv}c{chunk}-{dt}{'-decay' if dec else ''}"


@pytest.mark.parametrize("case", CASES, ids=[cid(c) for c in CASES])
def test_hla3_stages_match_oracle(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay = case
    say("third-order case", cid(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=4000 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    uq, uk, uv, ug = inp.units()
    U, n = B * H, T // chunk
    tol = tol_of(dtype)
    seg = lambda x, s: x[:, s * chunk:(s + 1) * chunk]
    sums = [O3.segment_summary3(seg(uq, s), seg(uk, s), seg(uv, s), ug) for s in range(n)]
    pre = O3.blelloch_exclusive_scan3(sums)
    num, den, fin = O3.serial3_r(uq, uk, uv, ug)

    gs = hla.hla3_chunk_summaries(q, k, v, chunk, g)
    torch.cuda.synchronize()
    for key in hla.SUMMARY3_FIELDS:
        got = host(gs[key]).reshape(U, n, -1)
        want = np.stack([s_[key].reshape(U, -1) for s_ in sums], axis=1)
        e = rel_err(got, want)
        say(f"  summary {key}: {e:.2e}")
        assert e <= tol, (key, e)

    tot = hla.hla3_scan(gs, q, v, chunk, g, want_total=True)
    torch.cuda.synchronize()
    for key in hla.STATE3_FIELDS:
        got = host(gs[key]).reshape(U, n, -1)
        want = np.stack([p_[key].reshape(U, -1) for p_ in pre], axis=1)
        e = rel_err(got[:, 1:], want[:, 1:]) if n > 1 else 0.0
        et = rel_err(host(tot[key]).reshape(U, -1), fin[key].reshape(U, -1))
        say(f"  prefix {key}: {e:.2e}  total {et:.2e}")
        assert e <= tol and et <= tol, (key, e, et)
        assert not np.any(got[:, 0]), "the first segment's exclusive prefix is zero"
    for key in ("Q", "V", "Z", "z"):     # read only
        want = np.stack([s_[key].reshape(U, -1) for s_ in sums], axis=1)
        assert rel_err(host(gs[key]).reshape(U, n, -1), want) <= tol

    o, dn, fs = hla.hla3_fwd(q, k, v, chunk, g, want_den=True, want_state=True)
    torch.cuda.synchronize()
    pn, pd = O3.serial3(uq, uk, uv, ug)          # the pages' form
    e_num = rel_err(host(o).reshape(U, T, dv), pn)
    e_den = rel_err(host(dn).reshape(U, T), pd)
    say(f"  num {e_num:.2e} den {e_den:.2e}")
    assert e_num <= tol and e_den <= tol
    assert rel_err(pn, num) < 1e-9 and rel_err(pd, den) < 1e-9
    for key in hla.STATE3_FIELDS:
        assert rel_err(host(fs[key]).reshape(U, -1), fin[key].reshape(U, -1)) <= tol, key
    # ratio-normalised: the same kernels, then num / (den + eps)
    eps = 1e-6
    on, dn2, _ = hla.hla3_fwd(q, k, v, chunk, g, normalize=True, eps=eps, want_den=True)
    torch.cuda.synchronize()
    assert torch.equal(dn2, dn)
    assert rel_err(host(on), host(o) / (host(dn)[..., None] + eps)) <= 1e-5


def test_hla3_gamma_zero_is_cubed_diagonal(gpu):
    torch = gpu
    inp = synth.make_fwd_inputs(1, 2, 256, 64, 64, "bf16", seed=4101, decay=True)
    inp.gamma = np.array([0.0, 0.5], np.float32)
    q, k, v, g = to_dev(inp)
    o, dn, _ = hla.hla3_fwd(q, k, v, 64, g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    s = np.sum(uq[0].astype(np.float64) * uk[0], axis=-1)
    num, den, _ = O3.serial3_r(uq, uk, uv, ug)
    assert rel_err(num[0], (s ** 3)[:, None] * uv[0]) < 1e-12     # oracle special case
    assert rel_err(host(o)[0], num) <= 2e-2 and rel_err(host(dn)[0], den) <= 2e-2


DEC = [(3, 2, 64, 32, "f32", True), (2, 2, 128, 128, "bf16", True), (4, 1, 16, 32, "bf16", False),
       (2, 3, 64, 128, "bf16", False), (2, 2, 128, 64, "f32", False)]


@pytest.mark.parametrize("case", DEC, ids=[f"N{c[0]}H{c[1]}d{c[2]}dv{c[3]}-{c[4]}" for c in DEC])
def test_hla3_decode_steps(gpu, case):
    torch = gpu
    N, H, d, dv, dtype, decay = case
    say("third-order decode case", case)
    pre = synth.make_fwd_inputs(N, H, 40, d, dv, dtype, seed=4200 + d, decay=decay)
    uq, uk, uv, ug = pre.units()
    _, _, st = O3.serial3_r(uq[:, :30], uk[:, :30], uv[:, :30], ug)
    st32 = {x: st[x].astype(np.float32) for x in hla.STATE3_FIELDS}
    state = {x: torch.from_numpy(st32[x].reshape(N, H, *st32[x].shape[1:])).cuda() for x in st32}
    state_n = {x: y.clone() for x, y in state.items()}
    q, k, v, g = to_dev(pre)
    ost = {x: st32[x].astype(np.float64) for x in st32}
    tol, eps = tol_of(dtype), 1e-6
    for t in range(30, 40):
        args = (q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
        o, dn = hla.hla3_decode_step(*args, state, g, den=torch.empty(N, H, device="cuda"))
        on, _ = hla.hla3_decode_step(*args, state_n, g, normalize=True, eps=eps)
        torch.cuda.synchronize()
        n_, d_, ost = O3.decode_step3(ost, uq[:, t], uk[:, t], uv[:, t], ug)
        gn, gd = host(o).reshape(N * H, dv), host(dn).reshape(N * H)
        assert rel_err(gn, n_) <= tol and rel_err(gd, d_) <= tol, t
        assert rel_err(host(on).reshape(N * H, dv), gn / (gd[:, None] + eps)) <= 1e-5
    for x in hla.STATE3_FIELDS:
        assert rel_err(host(state[x]).reshape(N * H, -1), ost[x].reshape(N * H, -1)) <= tol, x
        assert torch.equal(state[x], state_n[x]), x


def test_hla3_prefill_then_decode(gpu):
    torch = gpu
    N, H, d, dv, T0, steps, chunk = 2, 2, 64, 64, 256, 8, 64
    inp = synth.make_fwd_inputs(N, H, T0 + steps, d, dv, "bf16", seed=4300, decay=True)
    q, k, v, g = to_dev(inp)
    qp, kp, vp = (x[:, :, :T0].contiguous() for x in (q, k, v))
    _, _, state = hla.hla3_fwd(qp, kp, vp, chunk, g, want_state=True)
    outs = []
    for t in range(T0, T0 + steps):
        o, dn = hla.hla3_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                     v[:, :, t].contiguous(), state, g,
                                     den=torch.empty(N, H, device="cuda"))
        outs.append((host(o).reshape(N * H, dv), host(dn).reshape(N * H)))
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, den, _ = O3.serial3_r(uq, uk, uv, ug)      # uninterrupted
    got_n = np.stack([x[0] for x in outs], 1)
    got_d = np.stack([x[1] for x in outs], 1)
    e1, e2 = rel_err(got_n, num[:, T0:]), rel_err(got_d, den[:, T0:])
    say(f"  prefill -> decode: num {e1:.2e} den {e2:.2e}")
    assert e1 <= 2e-2 and e2 <= 2e-2


def test_hla3_full_size_sampled_units(gpu):
    """B4 H16 T16384 d128, decayed, bf16 (the second order's headline
    inputs), at the benchmark's segment length, on sampled units."""
    torch = gpu
    from bench import HLA3_CHUNK
    cfg = synth.FWD_WORKLOADS["fwd_decay_bf16_b4h16t16384d128"]
    B, H, T, d, dv = (cfg[x] for x in ("B", "H", "T", "d", "dv"))
    say("third order full size, chunk", HLA3_CHUNK)
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", cfg["seed"], decay=True)
    q, k, v, g = to_dev(inp)
    o, dn, _ = hla.hla3_fwd(q, k, v, HLA3_CHUNK, g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    sample = np.array([0, 21, 63])
    num, den, _ = O3.serial3_r(uq[sample], uk[sample], uv[sample], ug[sample])
    idx = torch.as_tensor(sample).cuda()
    e1 = rel_err(host(o.reshape(B * H, T, dv)[idx]), num)
    e2 = rel_err(host(dn.reshape(B * H, T)[idx]), den)
    say(f"  sampled units: num {e1:.2e} den {e2:.2e}")
    assert e1 <= 2e-2 and e2 <= 2e-2

"""GPU parity of the asymmetric variant AHLA against the fp64 oracle.

Calls go through the C ABI (hla_ahla_fwd and its three stages, via the
ctypes binding).  Small cases are compared element by element with the
oracle's serial recurrence (ragged tiles, one or many segments, decay, both
dtypes), some stage by stage; the decayed B4 H16 T16384 d128 inputs run at
full size and are compared on sampled (batch, head) units.  Tolerances:
1e-4 (fp32 inputs) and 2e-2 (bf16 inputs, fp32 state) on
max|got - want| / max|want|, numerator and denominator gated separately.
"""

import numpy as np
import pytest

from causal_prefix_scan_amd import hla, synth
from oracle import hla_oracle as O

from gpu_util import host, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()          # raises if the HIP library is missing: no silent fallback
    return torch


# (B, H, T, d, dv, chunk, dtype, decay, normalize)
SMALL = [
    (1, 2, 256, 16, 16, 64, "f32", False, False),
    (1, 1, 256, 16, 32, 32, "f32", True, True),
    (2, 1, 320, 32, 64, 64, "bf16", True, False),     # n = 5
    (1, 3, 384, 64, 32, 96, "bf16", True, True),      # ragged 32-token tile; n = 4
    (1, 2, 600, 64, 64, 200, "bf16", False, True),    # 3 tiles + ragged 8; n = 3
    (2, 2, 512, 128, 128, 128, "bf16", True, False),
    (1, 2, 512, 128, 64, 256, "bf16", True, True),
    (1, 1, 96, 64, 128, 32, "bf16", False, False),    # chunk shorter than a tile
    (1, 2, 192, 64, 64, 64, "f32", True, True),
    (1, 1, 128, 32, 16, 128, "bf16", False, False),   # n = 1
    (1, 2, 640, 32, 32, 32, "bf16", True, True),      # n = 20
    (1, 2, 288, 128, 128, 96, "bf16", True, True),    # 32-token last tile per segment
]


def case_id(c):
    B, H, T, d, dv, chunk, dt, dec, nrm = c
    return f"B{B}H{H}T{T}d{d}dv{dv}c{chunk}-{dt}{'-decay' if dec else ''}{'-norm' if nrm else ''}"


@pytest.mark.parametrize("case", SMALL, ids=[case_id(c) for c in SMALL])
def test_ahla_matches_oracle(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dt, decay, norm = case
    say("ahla case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dt, seed=900 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    o, dn = hla.ahla_fwd(q, k, v, chunk, g, normalize=False, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, den, _ = O.serial_ahla(uq, uk, uv, ug)
    tol = 1e-4 if dt == "f32" else 2e-2
    e_num = rel_err(host(o).reshape(num.shape), num)
    e_den = rel_err(host(dn).reshape(den.shape), den)
    say(f"  num {e_num:.3e}  den {e_den:.3e}  (tol {tol})")
    assert e_num <= tol and e_den <= tol
    if norm:
        eps = 1e-6
        on, _ = hla.ahla_fwd(q, k, v, chunk, g, normalize=True, eps=eps)
        torch.cuda.synchronize()
        ratio = host(o) / (host(dn)[..., None] + eps)
        assert rel_err(host(on), ratio) <= 1e-5


STAGED = [SMALL[1], SMALL[2], SMALL[5], SMALL[10]]


@pytest.mark.parametrize("case", STAGED, ids=[case_id(c) for c in STAGED])
def test_ahla_stages_match_oracle(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dt, decay, norm = case
    say("ahla stages", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dt, seed=950 + T, decay=decay)
    q, k, v, g = to_dev(inp)
    st = hla.ahla_chunk_summaries(q, k, v, chunk, g)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    U, n = B * H, T // chunk
    tol = 1e-4 if dt == "f32" else 2e-2
    _, _, pre = O.ahla_chunk_forward(uq, uk, uv, chunk, ug)
    for s in range(n):
        sl = slice(s * chunk, (s + 1) * chunk)
        want = O.ahla_segment_summary(uq[:, sl], uk[:, sl], uv[:, sl], ug)
        for key in ("P", "m", "E", "n", "X"):
            got = host(st[key]).reshape(U, n, *want[key].shape[1:])[:, s]
            assert rel_err(got, want[key]) <= tol, ("summary", s, key)
    hla.ahla_scan(st, q.shape, dv, chunk, hla.HLA_F32 if dt == "f32" else hla.HLA_BF16, g)
    torch.cuda.synchronize()
    for s in range(1, n):
        for key in ("P", "m", "E", "n"):
            got = host(st[key]).reshape(U, n, *pre[s][key].shape[1:])[:, s]
            assert rel_err(got, pre[s][key]) <= tol, ("prefix", s, key)
    assert float(np.abs(host(st["E"]).reshape(U, n, -1)[:, 0]).max()) == 0.0   # P_0 = 0
    o, dn = hla.ahla_output(q, k, v, st, chunk, g, want_den=True)
    torch.cuda.synchronize()
    num, den, _ = O.serial_ahla(uq, uk, uv, ug)
    assert rel_err(host(o).reshape(num.shape), num) <= tol
    assert rel_err(host(dn).reshape(den.shape), den) <= tol


def test_ahla_gamma_zero_keeps_the_current_token(gpu):
    torch = gpu
    inp = synth.make_fwd_inputs(1, 2, 192, 64, 64, "bf16", seed=61, decay=True)
    inp.gamma = np.array([0.0, 0.5], np.float32)
    q, k, v, g = to_dev(inp)
    o, dn = hla.ahla_fwd(q, k, v, 64, g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, den, _ = O.serial_ahla(uq, uk, uv, ug)
    s = np.sum(uq[0].astype(np.float64) * uk[0], axis=-1)
    assert rel_err(num[0], (s * s)[:, None] * uv[0]) < 1e-12     # oracle special case
    assert rel_err(host(o).reshape(num.shape), num) <= 2e-2
    assert rel_err(host(dn).reshape(den.shape), den) <= 2e-2


def test_ahla_is_deterministic(gpu):
    torch = gpu
    inp = synth.make_fwd_inputs(2, 2, 512, 128, 128, "bf16", seed=62, decay=True)
    q, k, v, g = to_dev(inp)
    o1, d1 = hla.ahla_fwd(q, k, v, 128, g, want_den=True)
    o2, d2 = hla.ahla_fwd(q, k, v, 128, g, want_den=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(d1, d2)


def test_ahla_workload_b4h16t16384d128_decayed(gpu):
    torch = gpu
    cfg = synth.FWD_WORKLOADS["fwd_decay_bf16_b4h16t16384d128"]
    B, H, T, d, dv = cfg["B"], cfg["H"], cfg["T"], cfg["d"], cfg["dv"]
    say("ahla workload B4 H16 T16384 d128 decayed, sample [0, 29, 63]")
    inp = synth.make_fwd_inputs(B, H, T, d, dv, cfg["dtype"], cfg["seed"],
                                k_l2norm=cfg["k_l2norm"], decay=cfg["decay"])
    q, k, v, g = to_dev(inp)
    o, dn = hla.ahla_fwd(q, k, v, cfg["chunk"], g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    idx = np.array([0, 29, 63])
    num, den, _ = O.serial_ahla(uq[idx], uk[idx], uv[idx], ug[idx])
    sel = torch.as_tensor(idx).cuda()
    e_num = rel_err(host(o.reshape(B * H, T, dv)[sel]), num)
    e_den = rel_err(host(dn.reshape(B * H, T)[sel]), den)
    say(f"  num {e_num:.3e}  den {e_den:.3e}  (tol {cfg['tol']})")
    assert e_num <= cfg["tol"] and e_den <= cfg["tol"]


# (N, H, d, dv, dtype, decay)
DECODE = [
    (2, 3, 64, 64, "bf16", True),
    (1, 2, 128, 128, "bf16", False),
    (2, 2, 16, 32, "f32", True),
    (1, 4, 128, 64, "bf16", True),
    (2, 1, 32, 32, "f32", False),
]


@pytest.mark.parametrize("case", DECODE, ids=[f"N{c[0]}H{c[1]}d{c[2]}dv{c[3]}-{c[4]}"
                                              f"{'-decay' if c[5] else ''}" for c in DECODE])
def test_ahla_decode_matches_oracle(gpu, case):
    # both sides start from the same fp32 state (the oracle's prefix state
    # rounded to fp32) and apply the same tokens one at a time
    torch = gpu
    N, H, d, dv, dt, decay = case
    say("ahla decode", case)
    T0, steps, eps = 80, 12, 1e-6
    inp = synth.make_fwd_inputs(N, H, T0 + steps, d, dv, dt, seed=800 + d + dv, decay=decay)
    uq, uk, uv, ug = inp.units()
    _, _, st = O.serial_ahla(uq[:, :T0], uk[:, :T0], uv[:, :T0], ug)
    keys = ("P", "m", "E", "n")
    st32 = {key: st[key].astype(np.float32) for key in keys}
    state = {key: torch.from_numpy(st32[key].reshape(N, H, *st32[key].shape[1:])).cuda() for key in keys}
    ref = {key: st32[key].astype(np.float64) for key in keys}
    q, k, v, g = to_dev(inp)
    tol = 1e-4 if dt == "f32" else 2e-2
    den = torch.empty(N, H, device="cuda")
    for t in range(T0, T0 + steps):
        o, _ = hla.ahla_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                    v[:, :, t].contiguous(), state, g, den=den)
        torch.cuda.synchronize()
        num_r, den_r, ref = O.serial_ahla(uq[:, t:t + 1], uk[:, t:t + 1], uv[:, t:t + 1], ug, ref)
        assert rel_err(host(o).reshape(N * H, dv), num_r[:, 0]) <= tol, t
        assert rel_err(host(den).reshape(N * H), den_r[:, 0]) <= tol, t
    for key in keys:
        assert rel_err(host(state[key]).reshape(ref[key].shape), ref[key]) <= 1e-5, key
    on, _ = hla.ahla_decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(),
                                 v[:, :, 0].contiguous(), state, g, normalize=True, eps=eps, den=den)
    torch.cuda.synchronize()
    num_r, den_r, _ = O.serial_ahla(uq[:, :1], uk[:, :1], uv[:, :1], ug, ref)
    assert rel_err(host(den).reshape(N * H), den_r[:, 0]) <= tol
    got_num = host(on).reshape(N * H, dv) * (host(den).reshape(N * H, 1) + eps)
    assert rel_err(got_num, num_r[:, 0]) <= tol


def test_ahla_prefill_then_decode(gpu):
    # the summary of a prefix (one segment) is the state after it; decode steps
    # from there give the forward's outputs for the following tokens
    torch = gpu
    N, H, d, dv, T0, steps = 2, 2, 64, 64, 128, 8
    inp = synth.make_fwd_inputs(N, H, T0 + steps, d, dv, "bf16", seed=88, decay=True)
    q, k, v, g = to_dev(inp)
    st = hla.ahla_chunk_summaries(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(),
                                  v[:, :, :T0].contiguous(), T0, g)
    state = {key: st[key][:, :, 0].contiguous() for key in ("P", "m", "E", "n")}
    outs = []
    for t in range(T0, T0 + steps):
        o, _ = hla.ahla_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                    v[:, :, t].contiguous(), state, g)
        outs.append(o.clone())
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, _, _ = O.serial_ahla(uq, uk, uv, ug)
    got = np.stack([host(x).reshape(N * H, dv) for x in outs], axis=1)
    assert rel_err(got, num[:, T0:]) <= 2e-2

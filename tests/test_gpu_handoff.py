"""GPU parity of the prefill -> decode handoff and of the ratio-normalised
decode output, through the C ABI, against the fp64 CPU oracle.

* The decode workload (64 sequences x 32 heads, d = dv = 128, 2048-token
  prefix) is prefilled on the GPU exactly as the benchmark does it (hla_fwd
  with one segment per prefix and a final state), then decoded for several
  steps twice from copies of that state: once unnormalised (num and den) and
  once ratio-normalised.  Sampled units are compared with the oracle's serial
  recurrence run uninterrupted over prefix + steps; every unit is compared
  for every step with the oracle's decode step continued from the GPU's own
  prefill state.
* The long-context forward (B1 H32 T65536 d64, 512 segments of 128 tokens per
  head) asks hla_fwd for a final state, which takes the per-segment exclusive
  scan over all 512 segments; sampled units' outputs, final states and the
  decode steps that follow are compared with the oracle.
* Small decode cases with normalize = 1.

Gates: num and den at the workload tolerance (2e-2 for bf16 inputs with fp32
state; the normalised output is ill-conditioned where den crosses zero, so
it is gated through num and den).  The GPU's normalised o must equal its own
num / (den + eps) to 1e-5, and agree with the oracle's normalise within the
error that the gated num and den errors propagate to:
|do_t| <= tol (max|num| + |o_t| max|den|) / (|den_t + eps| - tol max|den|) on the
tokens where that denominator is positive.  The literal
max|do| / max|o|, the same on tokens with |den_t| >= 1e-2 t / d and min|den|
are printed.
"""

import numpy as np
import pytest

from causal_prefix_scan_amd import hla, synth
from oracle import hla_oracle as O

from gpu_util import bits_to_dev, host, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("S", "C", "m", "G", "h")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()          # raises if the HIP library is missing: no silent fallback
    return torch


def check_normalised(got_o, num_gpu, den_gpu, num_ref, den_ref, eps, tol, t_index, d, tag):
    """Normalised output: self-consistency with the GPU's num and den, and the
    propagated-error check against the oracle's normalise (see module doc)."""
    assert rel_err(got_o, num_gpu / (den_gpu[..., None] + eps)) <= 1e-5, tag
    want_o = O.normalise(num_ref, den_ref, eps)
    # |dn| <= tol max|num| and |dd| <= tol max|den| (the gates) give
    # |do| <= (|dn| + |o| |dd|) / (|den + eps| - |dd|) wherever that is positive
    D = tol * np.max(np.abs(den_ref))
    room = np.abs(den_ref + eps) - D
    ok = room > 0
    bound = tol * np.max(np.abs(num_ref)) + np.abs(want_o) * D
    excess = float(np.max(np.abs(got_o - want_o)[ok] / (bound[ok] / room[ok][..., None])))
    good = np.abs(den_ref) >= 1e-2 * t_index / d
    frac = float(np.mean(good))
    lit = rel_err(got_o, want_o)
    on_good = rel_err(got_o[good], want_o[good]) if np.any(good) else float("nan")
    say(f"  {tag}: normalised o literal max|do|/max|o| {lit:.3e}; on |den| >= 1e-2 t/d "
        f"({100 * frac:.1f}% of tokens) {on_good:.3e}; min|den| {np.min(np.abs(den_ref)):.3e}; "
        f"|do| / propagated bound <= {excess:.3f}")
    assert excess <= 1.0, (tag, excess)


DEC_NORM = [(3, 2, 64, 32, "f32", True), (2, 2, 128, 128, "bf16", True),
            (4, 1, 16, 32, "bf16", False), (2, 3, 64, 128, "bf16", False)]


@pytest.mark.parametrize("case", DEC_NORM, ids=[f"N{c[0]}H{c[1]}d{c[2]}dv{c[3]}-{c[4]}" for c in DEC_NORM])
def test_decode_normalised_small(gpu, case):
    torch = gpu
    N, H, d, dv, dtype, decay = case
    say("normalised decode case", case)
    eps = 1e-6
    pre = synth.make_fwd_inputs(N, H, 40, d, dv, dtype, seed=60 + d, decay=decay)
    uq, uk, uv, ug = pre.units()
    _, _, st = O.serial(uq[:, :30], uk[:, :30], uv[:, :30], ug)
    st32 = {key: st[key].astype(np.float32) for key in FIELDS}
    mk = lambda: {key: torch.from_numpy(st32[key].reshape(N, H, *st32[key].shape[1:])).cuda()
                  for key in FIELDS}
    s_num, s_nrm = mk(), mk()
    q, k, v, g = to_dev(pre)
    ost = {key: st32[key].astype(np.float64) for key in FIELDS}
    tol = 1e-4 if dtype == "f32" else 2e-2
    for t in range(30, 40):
        args = (q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
        o, dn = hla.decode_step(*args, s_num, g, normalize=False, den=torch.empty(N, H, device="cuda"))
        on, dn2 = hla.decode_step(*args, s_nrm, g, normalize=True, eps=eps,
                                  den=torch.empty(N, H, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(dn, dn2), "the denominator does not depend on normalize"
        n_, d_, ost = O.decode_step(ost, uq[:, t], uk[:, t], uv[:, t], ug)
        got_n, got_d = host(o).reshape(N * H, dv), host(dn).reshape(N * H)
        assert rel_err(got_n, n_) <= tol and rel_err(got_d, d_) <= tol
        check_normalised(host(on).reshape(N * H, dv), got_n, got_d, n_, d_, eps, tol,
                         np.full(N * H, t + 1.0), d, f"step {t}")
    for key in FIELDS:
        assert torch.equal(s_num[key], s_nrm[key]), ("state must not depend on normalize", key)


def test_decode_workload_prefill_then_normalised_decode(gpu):
    """The decode workload end to end: GPU prefill of all 2048 distinct
    2048-token prefixes (hla_fwd, one segment, final state), then decode steps
    unnormalised and ratio-normalised from copies of that state."""
    torch = gpu
    name, cfg = synth.DECODE_WORKLOAD
    Nq, H, d, dv, P, seed, eps = (cfg[x] for x in ("n_seq", "H", "d", "dv", "prefix_len",
                                                     "seed", "eps"))
    U, steps, tol = Nq * H, 8, cfg["tol"]
    say("workload", name, "prefill on the GPU, then", steps, "decode steps")
    pre = synth.make_fwd_inputs(Nq, H, P, d, dv, "bf16", seed)
    pq, pk, pv = (bits_to_dev(b) for b in (pre.q_bits, pre.k_bits, pre.v_bits))
    o_pre, den_pre, state = hla.fwd(pq, pk, pv, P, None, want_den=True, want_state=True)
    torch.cuda.synchronize()
    del pq, pk, pv
    state2 = {key: val.clone() for key, val in state.items()}
    prefill64 = {key: host(state[key]).reshape(U, *state[key].shape[2:]) for key in FIELDS}
    toks = [synth.make_decode_step(Nq, H, d, dv, seed, s) for s in range(steps)]
    den_a = torch.empty(Nq, H, device="cuda")
    den_b = torch.empty(Nq, H, device="cuda")
    rec = []
    for s in range(steps):
        qd, kd, vd = (bits_to_dev(b).reshape(Nq, H, -1) for b in toks[s][3])
        o, dn = hla.decode_step(qd, kd, vd, state, None, normalize=False, den=den_a)
        on, dn2 = hla.decode_step(qd, kd, vd, state2, None, normalize=True, eps=eps, den=den_b)
        torch.cuda.synchronize()
        assert torch.equal(dn, dn2)
        rec.append((host(o).reshape(U, dv), host(dn).reshape(U), host(on).reshape(U, dv)))
    for key in FIELDS:
        assert torch.equal(state[key], state2[key]), key

    # every unit, every step: the oracle's decode step continued from the GPU's prefill state
    ost = prefill64
    for s in range(steps):
        qh, kh, vh = toks[s][:3]
        n_, d_, ost = O.decode_step(ost, qh, kh, vh)
        e1, e2 = rel_err(rec[s][0], n_), rel_err(rec[s][1], d_)
        say(f"  step {s}, all {U} units: num {e1:.2e} den {e2:.2e}")
        assert e1 <= tol and e2 <= tol
        check_normalised(rec[s][2], rec[s][0], rec[s][1], n_, d_, eps, tol,
                         np.full(U, P + s + 1.0), d, f"step {s}")

    # sampled units: the oracle's serial recurrence uninterrupted over prefix + steps
    sample = np.array([0, 1, 63, 64, 511, 1000, 1337, 2047])
    uq, uk, uv, _ = pre.units()
    cat = lambda x, i: np.concatenate([x[sample], np.stack([toks[s][i][sample] for s in range(steps)], 1)], 1)
    num, den, fin = O.serial(cat(uq, 0), cat(uk, 1), cat(uv, 2))
    e_pre = rel_err(host(o_pre).reshape(U, P, dv)[sample], num[:, :P])
    e_pre_d = rel_err(host(den_pre).reshape(U, P)[sample], den[:, :P])
    got_n = np.stack([rec[s][0][sample] for s in range(steps)], 1)
    got_d = np.stack([rec[s][1][sample] for s in range(steps)], 1)
    got_o = np.stack([rec[s][2][sample] for s in range(steps)], 1)
    e1, e2 = rel_err(got_n, num[:, P:]), rel_err(got_d, den[:, P:])
    say(f"  sampled units uninterrupted: prefill num {e_pre:.2e} den {e_pre_d:.2e}; "
        f"decode num {e1:.2e} den {e2:.2e}")
    assert e_pre <= tol and e_pre_d <= tol and e1 <= tol and e2 <= tol
    t_idx = np.broadcast_to(np.arange(P + 1, P + steps + 1, dtype=np.float64), got_d.shape)
    check_normalised(got_o, got_n, got_d, num[:, P:], den[:, P:], eps, tol, t_idx, d,
                     "sampled units")
    for key in FIELDS:
        e = rel_err(host(state[key]).reshape(U, -1)[sample], fin[key].reshape(len(sample), -1))
        assert e <= tol, ("state after the steps", key, e)


def test_long_context_final_state_and_decode(gpu):
    """B1 H32 T65536 d64 with a final state: the per-segment scan over all 512
    segments of 128 tokens, then decode steps from the GPU's final state."""
    torch = gpu
    cfg = synth.FWD_WORKLOADS["fwd_bf16_b1h32t65536d64"]
    B, H, T, d, dv, chunk = (cfg[x] for x in ("B", "H", "T", "d", "dv", "chunk"))
    steps, tol = 4, cfg["tol"]
    say("long context with a final state: n =", T // chunk, "segments per head")
    inp = synth.make_fwd_inputs(B, H, T + steps, d, dv, "bf16", cfg["seed"])
    q, k, v, _ = to_dev(inp)
    qp, kp, vp = (x[:, :, :T].contiguous() for x in (q, k, v))
    o, dn, state = hla.fwd(qp, kp, vp, chunk, None, want_den=True, want_state=True)
    outs = []
    for t in range(T, T + steps):
        od, dd = hla.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                 v[:, :, t].contiguous(), state, None, normalize=False,
                                 den=torch.empty(B, H, device="cuda"))
        outs.append((host(od).reshape(B * H, dv), host(dd).reshape(B * H)))
    torch.cuda.synchronize()
    sample = np.array([0, 17, 31])
    uq, uk, uv, _ = inp.units()
    num, den, fin = O.serial(uq[sample, :T], uk[sample, :T], uv[sample, :T])
    e1 = rel_err(host(o).reshape(B * H, T, dv)[sample], num)
    e2 = rel_err(host(dn).reshape(B * H, T)[sample], den)
    say(f"  outputs over the per-segment scan: num {e1:.2e} den {e2:.2e}")
    assert e1 <= tol and e2 <= tol
    ost = fin
    for s, t in enumerate(range(T, T + steps)):
        n_, d_, ost = O.decode_step(ost, uq[sample, t], uk[sample, t], uv[sample, t])
        e3, e4 = rel_err(outs[s][0][sample], n_), rel_err(outs[s][1][sample], d_)
        say(f"  decode step {s}: num {e3:.2e} den {e4:.2e}")
        assert e3 <= tol and e4 <= tol
    for key in FIELDS:
        e = rel_err(host(state[key]).reshape(B * H, -1)[sample], ost[key].reshape(len(sample), -1))
        assert e <= tol, ("state after prefill and decode", key, e)


def test_per_segment_scan_n512(gpu):
    """hla_scan on 512 segment summaries per head (d = 64): exclusive prefixes
    of sampled segments and the inclusive totals against the oracle's Blelloch
    scan of the oracle's summaries."""
    torch = gpu
    B, H, T, d, dv, chunk = 1, 2, 65536, 64, 64, 128
    n = T // chunk
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=31, decay=True)
    q, k, v, g = to_dev(inp)
    uq, uk, uv, ug = inp.units()
    gs = hla.fwd_chunk_summaries(q, k, v, chunk, g)
    total = hla.scan(gs, q.shape, dv, chunk, hla.HLA_BF16, g, want_total=True)
    torch.cuda.synchronize()
    sums = O.chunk_summaries(uq, uk, uv, chunk, ug)
    pre = O.blelloch_exclusive_scan(sums, ug)
    _, _, fin = O.serial(uq, uk, uv, ug)
    U = B * H
    pick = [0, 1, 31, 32, 255, 256, 300, 511]
    for key in FIELDS:
        got = host(gs[key]).reshape(U, n, -1)[:, pick]
        want = np.stack([pre[i][key].reshape(U, -1) for i in pick], axis=1)
        e = rel_err(got[:, 1:], want[:, 1:])
        et = rel_err(host(total[key]).reshape(U, -1), fin[key].reshape(U, -1))
        say(f"  n = {n}: prefix {key} {e:.2e}, total {et:.2e}")
        assert e <= 2e-2 and et <= 2e-2, key
        assert not np.any(got[:, 0]), "the first segment's exclusive prefix is zero"

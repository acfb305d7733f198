"""GPU parity of the HIP path against the fp64 CPU oracle.

Every call goes through the C ABI (ctypes binding).  Small cases are
compared element by element, stage by stage (segment summaries, exclusive
prefixes, outputs); the full-size workloads run in the launch configuration
the benchmark times and are compared on sampled (batch, head) units that the
oracle recomputes from scratch.

Tolerances: max|got - want| / max|want| <= 1e-4 for fp32 inputs and <= 2e-2
for bf16 inputs with fp32 state.  Ratio-normalised outputs are gated on the
numerator and the denominator separately (the denominator changes sign, so
num / (den + eps) is ill-conditioned); the literal metric is printed.
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


def tol_of(dtype):
    return 1e-4 if dtype == "f32" else 2e-2


def dcode(dtype):
    return hla.HLA_F32 if dtype == "f32" else hla.HLA_BF16


# (B, H, T, d, dv, chunk, dtype, decay, normalize)
SMALL = [
    (1, 2, 256, 16, 16, 64, "f32", False, False),
    (1, 1, 256, 16, 16, 32, "f32", True, True),
    (2, 1, 320, 32, 64, 64, "bf16", True, False),     # n = 5 (not a power of two)
    (1, 3, 384, 64, 32, 96, "bf16", True, True),      # ragged 32-token tile; n = 4
    (1, 2, 600, 64, 64, 200, "bf16", False, True),    # 3 tiles + ragged 8; n = 3
    (2, 2, 512, 128, 128, 128, "bf16", True, False),
    (1, 2, 512, 128, 64, 256, "bf16", True, True),
    (1, 1, 96, 64, 128, 32, "bf16", False, False),    # chunk shorter than a tile
    (1, 2, 192, 64, 64, 64, "f32", True, True),
    (1, 1, 128, 32, 16, 128, "bf16", False, False),   # n = 1
    # more than 16 segments: runs of 8, a scan over the run totals
    (1, 2, 640, 32, 32, 32, "bf16", True, True),      # n = 20: runs 8, 8, 4; tree pads 3 -> 4
    (1, 1, 640, 16, 16, 16, "f32", True, False),      # n = 40: 5 runs, tree pads 5 -> 8
    (1, 1, 544, 128, 128, 32, "bf16", True, False),   # n = 17: runs 8, 8, 1
    (1, 2, 1536, 64, 64, 64, "bf16", True, True),     # n = 24 at d = 64: runs of 8 side by side
                                                      # (16-wave rescan, 8 waves idle), from prefixes
    (1, 2, 288, 128, 128, 96, "bf16", True, True),    # 8 waves, a 32-token last tile per segment
    (2, 1, 200, 128, 64, 100, "bf16", False, True),   # 8 waves, d > dv, 36-token last tile
    # more than 256 workgroups: the 4-wave d = 64 kernels (the cases above with
    # d = 64 run the 8-wave ones, a grid of at most one workgroup per CU)
    (4, 16, 320, 64, 64, 64, "bf16", True, True),     # 64 units x 5 segments = 320 workgroups
    (4, 16, 480, 64, 32, 96, "bf16", False, False),   # 320 workgroups, d > dv, ragged 32-token tile
]


def case_id(c):
    B, H, T, d, dv, chunk, dt, dec, nrm = c
    return f"B{B}H{H}T{T}d{d}dv{dv}c{chunk}-{dt}{'-decay' if dec else ''}{'-norm' if nrm else ''}"


@pytest.mark.parametrize("case", SMALL, ids=[case_id(c) for c in SMALL])
def test_stages_match_oracle(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay, norm = case
    say("case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=1000 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    uq, uk, uv, ug = inp.units()
    U, n = B * H, T // chunk
    tol = tol_of(dtype)

    num, den, final = O.serial(uq, uk, uv, ug)
    sums = O.chunk_summaries(uq, uk, uv, chunk, ug)
    pre = O.blelloch_exclusive_scan(sums, ug)

    gs = hla.fwd_chunk_summaries(q, k, v, chunk, g)
    torch.cuda.synchronize()
    for key in FIELDS:
        got = host(gs[key]).reshape(U, n, -1)
        want = np.stack([s[key].reshape(U, -1) for s in sums], axis=1)
        e = rel_err(got, want)
        say(f"  summary {key}: {e:.2e}")
        assert e <= tol, (key, e)
    gs0 = {key: val.clone() for key, val in gs.items()}
    keep = {key: val.clone() for key, val in gs.items()}

    total = hla.scan(gs, q.shape, dv, chunk, dcode(dtype), g, want_total=True)
    torch.cuda.synchronize()
    for key in FIELDS:
        got = host(gs[key]).reshape(U, n, -1)
        want = np.stack([p[key].reshape(U, -1) for p in pre], axis=1)
        e = rel_err(got, want) if np.any(want) else float(np.max(np.abs(got)))
        say(f"  prefix {key}: {e:.2e}")
        assert e <= tol, (key, e)
        et = rel_err(host(total[key]).reshape(U, -1), final[key].reshape(U, -1))
        assert et <= tol, ("total", key, et)
    assert not torch.any(gs["S"][:, :, 0]).item(), "exclusive prefix of segment 0 must be zero"
    # out of place: the in-place scan's bits, the summaries only read
    pre2, tot2 = hla.scan_into(gs0, q.shape, dv, chunk, dcode(dtype), g, want_total=True)
    torch.cuda.synchronize()
    for key in FIELDS:
        assert torch.equal(pre2[key], gs[key]), ("scan_into", key)
        assert torch.equal(tot2[key], total[key]), ("scan_into total", key)
        assert torch.equal(gs0[key], keep[key]), ("scan_into wrote its input", key)
    # without a total the walk neither loads nor combines a unit's last
    # segment: the prefixes are the same bits
    pre3, tot3 = hla.scan_into(gs0, q.shape, dv, chunk, dcode(dtype), g, want_total=False)
    gs3 = {key: val.clone() for key, val in keep.items()}
    tot4 = hla.scan(gs3, q.shape, dv, chunk, dcode(dtype), g, want_total=False)
    torch.cuda.synchronize()
    assert tot3 is None and tot4 is None
    for key in FIELDS:
        assert torch.equal(pre3[key], gs[key]), ("scan_into without a total", key)
        assert torch.equal(gs3[key], gs[key]), ("scan without a total", key)

    o, dn = hla.fwd_output(q, k, v, gs, chunk, g, normalize=False, want_den=True)
    torch.cuda.synchronize()
    e_num = rel_err(host(o).reshape(U, T, dv), num)
    e_den = rel_err(host(dn).reshape(U, T), den)
    say(f"  num {e_num:.2e} den {e_den:.2e}")
    assert e_num <= tol and e_den <= tol

    if norm:
        eps = 1e-6
        on, dn2 = hla.fwd_output(q, k, v, gs, chunk, g, normalize=True, eps=eps, want_den=True)
        torch.cuda.synchronize()
        assert torch.equal(dn2, dn)
        ratio = host(o) / (host(dn)[..., None] + eps)
        assert rel_err(host(on), ratio) <= 1e-5

    # the composed entry point gives the same bits as the three calls (these
    # problems have too few units for spans of several chunks; the minimum
    # workspace keeps hla_fwd on these calls' plan for every shape)
    assert hla.fwd_span_chunks(q, v, chunk, g) == 1
    o3, dn3, fs = hla.fwd(q, k, v, chunk, g, normalize=False, want_den=True, want_state=True,
                          workspace=hla.fwd_workspace(q, v, chunk, g, with_p=False))
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(dn3, dn)
    for key in FIELDS:
        assert torch.equal(fs[key], total[key]), key


# (B, H, T, d, dv, chunk, dtype, decay, normalize): more than 16 segments, so
# more than one run; the first four have whole runs (R divides n)
RUNS = [
    (1, 2, 1024, 32, 32, 32, "bf16", True, True),     # n = 32: 4 runs of 8
    (1, 1, 512, 16, 16, 16, "f32", True, False),      # n = 32, fp32
    (1, 1, 1024, 128, 128, 32, "bf16", True, False),  # 8-wave kernels walking 256-token runs
    (2, 1, 2048, 64, 64, 64, "bf16", False, True),    # n = 32, gamma = 1
    (1, 2, 640, 32, 32, 32, "bf16", True, False),     # n = 20: runs 8, 8, 4 (prefixes only)
]


@pytest.mark.parametrize("case", RUNS, ids=[case_id(c) for c in RUNS])
def test_run_prefixes_and_run_length_outputs(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay, norm = case
    say("case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=2000 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    uq, uk, uv, ug = inp.units()
    U, n = B * H, T // chunk
    R = hla.scan_run_length(T, chunk)
    runs = (n + R - 1) // R
    assert R > 1 and runs > 1
    tol = tol_of(dtype)
    num, den, _ = O.serial(uq, uk, uv, ug)
    pre = O.blelloch_exclusive_scan(O.chunk_summaries(uq, uk, uv, chunk, ug), ug)

    gs = hla.fwd_chunk_summaries(q, k, v, chunk, g)
    before = {key: gs[key].clone() for key in FIELDS}
    rp = hla.scan_runs(gs, q.shape, dv, chunk, dcode(dtype), g)
    torch.cuda.synchronize()
    for key in FIELDS:
        assert torch.equal(gs[key], before[key]), ("summaries must be left as they are", key)
        got = host(rp[key]).reshape(U, runs, -1)
        want = np.stack([pre[r * R][key].reshape(U, -1) for r in range(runs)], axis=1)
        e = rel_err(got, want)
        say(f"  run prefix {key}: {e:.2e}")
        assert e <= tol, (key, e)
    assert not torch.any(rp["S"][:, :, 0]).item(), "the first run starts from zero"
    if runs * R != n:
        return
    # outputs with the output kernel walking whole runs from the run prefixes
    o, dn = hla.fwd_output(q, k, v, rp, chunk * R, g, normalize=False, want_den=True)
    torch.cuda.synchronize()
    e_num = rel_err(host(o).reshape(U, T, dv), num)
    e_den = rel_err(host(dn).reshape(U, T), den)
    say(f"  run-length spans: num {e_num:.2e} den {e_den:.2e}")
    assert e_num <= tol and e_den <= tol
    if norm:
        eps = 1e-6
        on, _ = hla.fwd_output(q, k, v, rp, chunk * R, g, normalize=True, eps=eps)
        torch.cuda.synchronize()
        ratio = host(o) / (host(dn)[..., None] + eps)
        assert rel_err(host(on), ratio) <= 1e-5


# (B, H, T, d, dv, chunk, dtype, decay, normalize): enough units for hla_fwd
# to walk spans of several chunks per workgroup
SPANS = [
    (4, 4, 2048, 32, 32, 32, "bf16", True, True),      # n = 64 -> spans of 4 chunks, 16 per head
    (2, 8, 1024, 64, 64, 16, "bf16", False, False),    # n = 64 -> spans of 4
    (1, 16, 4096, 64, 64, 32, "bf16", True, False),    # n = 128 -> spans of 8, 16 per head
    (1, 4, 8192, 32, 32, 32, "bf16", True, True),      # n = 256 -> spans of 2, 128 per head: 8 runs
    (4, 8, 512, 16, 32, 16, "f32", True, True),        # n = 32 -> spans of 2
]


@pytest.mark.parametrize("case", SPANS, ids=[case_id(c) for c in SPANS])
def test_fwd_spans_of_several_chunks(gpu, case):
    """hla_fwd with spans of R > 1 chunks: the same bits as the three calls at
    chunk R * chunk, the oracle's outputs and final state at the tolerance."""
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay, norm = case
    say("case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=3000 + T + d, decay=decay)
    q, k, v, g = to_dev(inp)
    R = hla.fwd_span_chunks(q, v, chunk, g)
    n = T // chunk
    assert R > 1 and n % R == 0 and B * H * (n // R) >= 256
    say(f"  spans of {R} chunks, {n // R} per head")
    eps = 1e-6
    o, dn, fs = hla.fwd(q, k, v, chunk, g, normalize=norm, eps=eps, want_den=True, want_state=True)
    gs = hla.fwd_chunk_summaries(q, k, v, chunk * R, g)
    tot = hla.scan(gs, q.shape, dv, chunk * R, dcode(dtype), g, want_total=True)
    o3, dn3 = hla.fwd_output(q, k, v, gs, chunk * R, g, normalize=norm, eps=eps, want_den=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o3) and torch.equal(dn, dn3)
    for key in FIELDS:
        assert torch.equal(fs[key], tot[key]), key
    uq, uk, uv, ug = inp.units()
    U = B * H
    num, den, fin = O.serial(uq, uk, uv, ug)
    tol = tol_of(dtype)
    e_den = rel_err(host(dn).reshape(U, T), den)
    if norm:
        assert rel_err(host(o), host(o3)) == 0.0
        on, _, _ = hla.fwd(q, k, v, chunk, g, normalize=False)
        torch.cuda.synchronize()
        e_num = rel_err(host(on).reshape(U, T, dv), num)
        assert rel_err(host(o), host(on) / (host(dn)[..., None] + eps)) <= 1e-5
    else:
        e_num = rel_err(host(o).reshape(U, T, dv), num)
    say(f"  num {e_num:.2e} den {e_den:.2e}")
    assert e_num <= tol and e_den <= tol
    for key in FIELDS:
        e = rel_err(host(fs[key]).reshape(U, -1), fin[key].reshape(U, -1))
        assert e <= tol, ("final state", key, e)


def local_p(uq, uk, ug, chunk):
    """p_t = S_t q_t with S_t = sum_{i<=t} g^(t-i) k_i k_i^T restarted at every
    segment start (the definition; fp64), [U, T, d]."""
    U, T, d = uq.shape
    q64, k64 = uq.astype(np.float64), uk.astype(np.float64)
    g = np.ones(U) if ug is None else ug.astype(np.float64)
    out = np.zeros((U, T, d))
    S = np.zeros((U, d, d))
    for t in range(T):
        if t % chunk == 0:
            S[:] = 0.0
        S = g[:, None, None] * S + k64[:, t, :, None] * k64[:, t, None, :]
        out[:, t] = np.einsum("uij,uj->ui", S, q64[:, t])
    return out


# (B, H, T, d, dv, chunk, dtype, decay, normalize): bf16, d = dv = 128, the
# shape whose outputs come from the segment-local p
PCASES = [
    (2, 2, 512, 128, 128, 128, "bf16", True, False),
    (1, 2, 288, 128, 128, 96, "bf16", True, True),     # a 32-token last tile per segment
    (1, 1, 600, 128, 128, 200, "bf16", False, True),   # 3 tiles + ragged 8, gamma = 1
    (1, 1, 544, 128, 128, 32, "bf16", True, False),    # n = 17, chunks shorter than a tile
    (1, 2, 256, 128, 128, 256, "bf16", True, False),   # n = 1
]


@pytest.mark.parametrize("case", PCASES, ids=[case_id(c) for c in PCASES])
def test_outputs_from_segment_local_p(gpu, case):
    """hla_fwd_chunk_summaries_p writes the same summaries as
    hla_fwd_chunk_summaries and the segment-local p of the definition (zeros
    past each segment's end); hla_fwd_output_from_p gives the oracle's outputs;
    hla_fwd with room for p gives the same bits as these three calls."""
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay, norm = case
    say("case", case_id(case))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=3500 + T + chunk, decay=decay)
    q, k, v, g = to_dev(inp)
    uq, uk, uv, ug = inp.units()
    U, n, tol, eps = B * H, T // chunk, tol_of(dtype), 1e-6
    ntiles = (chunk + 63) // 64
    assert hla.p_bytes(q, v, chunk) == U * n * ntiles * d * 64 * 2
    gs = hla.fwd_chunk_summaries(q, k, v, chunk, g)
    gp, pl = hla.fwd_chunk_summaries_p(q, k, v, chunk, g)
    torch.cuda.synchronize()
    for key in FIELDS:
        assert torch.equal(gs[key], gp[key]), key
    # p: per tile, (column block cb, row block r) fragments of 64 groups of 4,
    # group l = tokens 16 r + 4 (l // 16) + [0, 4) of column 16 cb + l % 16
    blocks = host(pl.float()).reshape(U, n, ntiles, d // 16, 4, 4, 16, 4)   # [.., cb, r, lg, lr, j]
    want = local_p(uq, uk, ug, chunk).reshape(U, n, chunk, d)
    tiles = blocks.transpose(0, 1, 2, 4, 5, 7, 3, 6).reshape(U, n, ntiles, 64, d)   # [.., r, lg, j, cb, lr]
    got = tiles.reshape(U, n, ntiles * 64, d)
    e = rel_err(got[:, :, :chunk], want)
    say(f"  segment-local p {e:.2e}")
    assert e <= tol
    assert not np.any(got[:, :, chunk:]), "rows past the segment end are zeros"
    tot = hla.scan(gp, q.shape, dv, chunk, dcode(dtype), g, want_total=True)
    o, dn = hla.fwd_output_from_p(q, v, pl, gp, chunk, g, normalize=False, want_den=True)
    torch.cuda.synchronize()
    num, den, fin = O.serial(uq, uk, uv, ug)
    e_num = rel_err(host(o).reshape(U, T, dv), num)
    e_den = rel_err(host(dn).reshape(U, T), den)
    say(f"  num {e_num:.2e} den {e_den:.2e}")
    assert e_num <= tol and e_den <= tol
    # against the path with the S recurrence, at the tolerance
    hla.scan(gs, q.shape, dv, chunk, dcode(dtype), g)
    o_old, dn_old = hla.fwd_output(q, k, v, gs, chunk, g, normalize=False, want_den=True)
    torch.cuda.synchronize()
    assert rel_err(host(o), host(o_old)) <= tol and rel_err(host(dn), host(dn_old)) <= tol
    if norm:
        on, dn2 = hla.fwd_output_from_p(q, v, pl, gp, chunk, g, normalize=True, eps=eps,
                                        want_den=True)
        torch.cuda.synchronize()
        assert torch.equal(dn2, dn)
        assert rel_err(host(on), host(o) / (host(dn)[..., None] + eps)) <= 1e-5
    # hla_fwd with room for p: the same bits as the three calls above
    assert hla.fwd_span_chunks(q, v, chunk, g) == 1
    o3, dn3, fs = hla.fwd(q, k, v, chunk, g, normalize=False, want_den=True, want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(dn3, dn)
    for key in FIELDS:
        assert torch.equal(fs[key], tot[key]), key


def test_outputs_from_p_gamma_zero(gpu):
    """gamma = 0 on the segment-local p path: each output is (q.k)^2 v of its own token."""
    torch = gpu
    inp = synth.make_fwd_inputs(1, 2, 256, 128, 128, "bf16", seed=71, decay=True)
    inp.gamma = np.array([0.0, 0.5], np.float32)
    q, k, v, g = to_dev(inp)
    o, dn, _ = hla.fwd(q, k, v, 128, g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, den, _ = O.serial(uq, uk, uv, ug)
    s = np.sum(uq[0].astype(np.float64) * uk[0], axis=-1)
    assert rel_err(num[0], (s * s)[:, None] * uv[0]) < 1e-12     # oracle special case
    assert rel_err(host(o).reshape(2, 256, 128), num) <= 2e-2
    assert rel_err(host(dn).reshape(2, 256), den) <= 2e-2


def full_or_sampled(name, sample_units):
    cfg = synth.FWD_WORKLOADS[name]
    return cfg, sample_units


def run_workload(gpu, name, sample_units=None):
    torch = gpu
    cfg = synth.FWD_WORKLOADS[name]
    B, H, T, d, dv = cfg["B"], cfg["H"], cfg["T"], cfg["d"], cfg["dv"]
    say("workload", name, "sample", sample_units)
    inp = synth.make_fwd_inputs(B, H, T, d, dv, cfg["dtype"], cfg["seed"],
                                k_l2norm=cfg["k_l2norm"], decay=cfg["decay"])
    q, k, v, g = to_dev(inp)
    o, dn, _ = hla.fwd(q, k, v, cfg["chunk"], g, normalize=False, want_den=True)
    on = None
    if cfg["normalize"]:
        on, _, _ = hla.fwd(q, k, v, cfg["chunk"], g, normalize=True, eps=cfg["eps"])
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    U = B * H
    idx = np.arange(U) if sample_units is None else np.asarray(sample_units)
    num, den, _ = O.serial(uq[idx], uk[idx], uv[idx], None if ug is None else ug[idx])
    got_num = host(o.reshape(U, T, dv)[torch.as_tensor(idx).cuda()])
    got_den = host(dn.reshape(U, T)[torch.as_tensor(idx).cuda()])
    e_num, e_den = rel_err(got_num, num), rel_err(got_den, den)
    say(f"  num {e_num:.3e}  den {e_den:.3e}  (tol {cfg['tol']})")
    assert e_num <= cfg["tol"]
    if cfg["normalize"]:
        assert e_den <= cfg["tol"]
        want_o = O.normalise(num, den, cfg["eps"])
        got_o = host(on.reshape(U, T, dv)[torch.as_tensor(idx).cuda()])
        t = np.arange(1, T + 1)
        good = np.abs(den) >= 1e-2 * t[None, :] / d
        say(f"  literal max|do|/max|o| {rel_err(got_o, want_o):.3e}; on |den| >= 1e-2 t/d: "
            f"{rel_err(got_o[good], want_o[good]):.3e}; min|den| {np.min(np.abs(den)):.3e}")
        # the GPU's own ratio is consistent with its numerator and denominator
        assert rel_err(got_o, got_num / (got_den[..., None] + cfg["eps"])) <= 1e-5


def test_workload_fwd_f32_b1h1t256d16(gpu):
    run_workload(gpu, "fwd_f32_b1h1t256d16")


def test_workload_fwd_norm_bf16_b2h8t4096d64(gpu):
    run_workload(gpu, "fwd_norm_bf16_b2h8t4096d64")


def test_workload_fwd_decay_bf16_b4h16t16384d128(gpu):
    run_workload(gpu, "fwd_decay_bf16_b4h16t16384d128", sample_units=[0, 21, 63])


def test_workload_fwd_bf16_b1h32t65536d64(gpu):
    run_workload(gpu, "fwd_bf16_b1h32t65536d64", sample_units=[0, 31])


def test_fwd_gamma_zero_keeps_the_diagonal(gpu):
    torch = gpu
    inp = synth.make_fwd_inputs(1, 2, 256, 64, 64, "bf16", seed=7, decay=True)
    inp.gamma = np.array([0.0, 0.5], np.float32)
    q, k, v, g = to_dev(inp)
    o, dn, _ = hla.fwd(q, k, v, 128, g, want_den=True)
    torch.cuda.synchronize()
    uq, uk, uv, ug = inp.units()
    num, den, _ = O.serial(uq, uk, uv, ug)
    s = np.sum(uq[0].astype(np.float64) * uk[0], axis=-1)
    assert rel_err(num[0], (s * s)[:, None] * uv[0]) < 1e-12     # oracle special case
    assert rel_err(host(o)[0], num) <= 2e-2
    assert rel_err(host(dn)[0], den) <= 2e-2


def test_fwd_is_deterministic_and_causal(gpu):
    torch = gpu
    inp = synth.make_fwd_inputs(2, 2, 512, 64, 64, "bf16", seed=8, decay=True)
    q, k, v, g = to_dev(inp)
    o1, _, _ = hla.fwd(q, k, v, 128, g)
    o2, _, _ = hla.fwd(q, k, v, 128, g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    t0 = 300                                  # inside the third segment
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, :, t0 + 1:] = -q2[:, :, t0 + 1:]
    k2[:, :, t0 + 1:] = 2 * k2[:, :, t0 + 1:]
    v2[:, :, t0 + 1:] = 0.5
    o3, _, _ = hla.fwd(q2, k2, v2, 128, g)
    torch.cuda.synchronize()
    assert torch.equal(o3[:, :, :t0 + 1], o1[:, :, :t0 + 1])
    assert not torch.equal(o3[:, :, t0 + 1:], o1[:, :, t0 + 1:])


def test_empty_problem(gpu):
    torch = gpu
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, _, _ = hla.fwd(q, q, q, 64)
    assert o.shape == (1, 2, 0, 64)


# ---- decode -------------------------------------------------------------------

DEC_SMALL = [(3, 2, 64, 32, "f32", True), (2, 2, 128, 128, "bf16", True),
             (4, 1, 16, 32, "bf16", False), (2, 3, 64, 128, "bf16", False)]


@pytest.mark.parametrize("case", DEC_SMALL, ids=[f"N{c[0]}H{c[1]}d{c[2]}dv{c[3]}-{c[4]}" for c in DEC_SMALL])
def test_decode_steps_match_oracle(gpu, case):
    torch = gpu
    N, H, d, dv, dtype, decay = case
    say("decode case", case)
    pre = synth.make_fwd_inputs(N, H, 40, d, dv, dtype, seed=50 + d, decay=decay)
    uq, uk, uv, ug = pre.units()
    _, _, st = O.serial(uq[:, :30], uk[:, :30], uv[:, :30], ug)
    st32 = {key: st[key].astype(np.float32) for key in FIELDS}
    state = {key: torch.from_numpy(st32[key].reshape(N, H, *st32[key].shape[1:])).cuda()
             for key in FIELDS}
    q, k, v, g = to_dev(pre)
    ost = {key: st32[key].astype(np.float64) for key in FIELDS}
    tol = tol_of(dtype)
    for t in range(30, 40):
        o, dn = hla.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                v[:, :, t].contiguous(), state, g, normalize=False,
                                den=torch.empty(N, H, device="cuda"))
        torch.cuda.synchronize()
        n_, d_, ost = O.decode_step(ost, uq[:, t], uk[:, t], uv[:, t], ug)
        assert rel_err(host(o).reshape(N * H, dv), n_) <= tol
        assert rel_err(host(dn).reshape(N * H), d_) <= tol
    for key in FIELDS:
        assert rel_err(host(state[key]).reshape(N * H, -1), ost[key].reshape(N * H, -1)) <= tol


def test_workload_decode_bf16_n64h32d128(gpu):
    torch = gpu
    name, cfg = synth.DECODE_WORKLOAD
    Nq, H, d, dv, P, steps, seed = (cfg[x] for x in ("n_seq", "H", "d", "dv", "prefix_len",
                                                     "steps", "seed"))
    U, n_unique = Nq * H, 64
    say("workload", name)
    pre = synth.make_decode_prefix(Nq, H, d, dv, P, seed, n_unique=n_unique)
    uq, uk, uv, _ = pre.units()
    st64 = O.segment_summary_sums(uq, uk, uv)
    st32 = {key: st64[key].astype(np.float32) for key in FIELDS}
    rep = U // n_unique

    def tiled(x):
        return np.tile(x, (rep,) + (1,) * (x.ndim - 1))

    state = {key: torch.from_numpy(tiled(st32[key]).reshape(Nq, H, *st32[key].shape[1:])).cuda()
             for key in FIELDS}
    sample = np.array([0, 1, 63, 64, 511, 1000, 1337, 2047])
    sidx = torch.as_tensor(sample).cuda()
    den_buf = torch.empty(Nq, H, device="cuda")
    rec_o, rec_d, full = [], [], []
    toks = []
    for s in range(steps):
        qh, kh, vh, bits = synth.make_decode_step(Nq, H, d, dv, seed, s)
        qd, kd, vd = (bits_to_dev(b).reshape(Nq, H, -1) for b in bits)
        o, dn = hla.decode_step(qd, kd, vd, state, None, normalize=False, den=den_buf)
        rec_o.append(o.reshape(U, dv)[sidx].clone())
        rec_d.append(dn.reshape(U)[sidx].clone())
        if s < 3:
            full.append((host(o).reshape(U, dv), host(dn).reshape(U), qh, kh, vh))
        toks.append((qh[sample], kh[sample], vh[sample]))
    torch.cuda.synchronize()
    tol = cfg["tol"]
    # all units, first steps
    ost = {key: tiled(st32[key]).astype(np.float64) for key in FIELDS}
    for s, (go, gd, qh, kh, vh) in enumerate(full):
        n_, d_, ost = O.decode_step(ost, qh, kh, vh)
        e1, e2 = rel_err(go, n_), rel_err(gd, d_)
        say(f"  step {s} all units: num {e1:.2e} den {e2:.2e}")
        assert e1 <= tol and e2 <= tol
    # sampled units, every step
    sst = {key: tiled(st32[key])[sample].astype(np.float64) for key in FIELDS}
    worst = 0.0
    for s in range(steps):
        n_, d_, sst = O.decode_step(sst, *toks[s])
        e1, e2 = rel_err(host(rec_o[s]), n_), rel_err(host(rec_d[s]), d_)
        worst = max(worst, e1, e2)
        assert e1 <= tol and e2 <= tol, (s, e1, e2)
    say(f"  sampled units, {steps} steps: worst {worst:.2e}")

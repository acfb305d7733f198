"""C-ABI contract checks that need no GPU.

Every declared symbol is exported; argument validation returns the documented
status before anything is launched (fake, never-dereferenced device
pointers are used); on a host without a HIP device a valid call returns
HLA_ERR_HIP instead of crashing.
"""

import ctypes
import os
import re

import pytest

from causal_prefix_scan_amd import hla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla.h")

OK, NULLP, SHAPE, DTYPE, MISAL, UNSUP, WS, ALIAS, HIP, VALUE = range(10)

# Fake device addresses: 16-byte aligned, far apart, never dereferenced on the host.
Q, K, V, O, DEN, GAM = (0x10000000 * (i + 1) for i in range(6))
S_BASE = 0x100000000


def state(base=S_BASE):
    step = 0x1000000
    return hla.State(base, base + step, base + 2 * step, base + 3 * step, base + 4 * step)


def problem(**kw):
    p = dict(B=2, H=3, T=256, d=64, dv=64, chunk=64, in_dtype=hla.HLA_BF16, normalize=0,
             eps=0.0, gamma=None)
    p.update(kw)
    return hla.Problem(**p)


@pytest.fixture(scope="module")
def L():
    return hla.lib()


def no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


def test_every_declared_symbol_is_exported(L):
    decl = set(re.findall(r"\b(hla3?_[a-z0-9_]+)\s*\(", open(HEADER).read()))
    assert decl == set(hla.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in hla.STATUS.items():
        assert hla.status_string(code).startswith(name)
    assert hla.status_string(12345) == "HLA_ERR_UNKNOWN"
    assert "gfx950" in hla.version()


def summaries(L, p, out=None, q=Q, k=K, v=V):
    return L.hla_fwd_chunk_summaries(ctypes.byref(p) if p is not None else None, q, k, v,
                                     ctypes.byref(out or state()), None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=250), SHAPE),                 # T % chunk != 0
    (dict(chunk=0), SHAPE),
    (dict(B=-1), SHAPE),
    (dict(d=0), SHAPE),
    (dict(in_dtype=7), DTYPE),
    (dict(normalize=2), VALUE),
    (dict(eps=float("nan")), VALUE),
    (dict(eps=float("inf")), VALUE),
    (dict(d=48), UNSUP),
    (dict(d=256, dv=256), UNSUP),
    (dict(d=16, dv=64), UNSUP),           # ratio 4 not built
    (dict(d=128, dv=128, in_dtype=hla.HLA_F32), UNSUP),
    (dict(gamma=GAM + 4), MISAL),
    (dict(B=70000, H=1, T=64), VALUE),    # grid.y of the scan
])
def test_problem_validation(L, kw, code):
    assert summaries(L, problem(**kw)) == code
    assert L.hla_fwd_output(ctypes.byref(problem(**kw)), Q, K, V, ctypes.byref(state()), O, None,
                            None, 0, None) == code


def test_pointer_validation(L):
    p = problem()
    assert summaries(L, None) == NULLP
    assert summaries(L, p, q=None) == NULLP
    assert summaries(L, p, v=V + 8) == MISAL
    bad = state()
    bad.G = None
    assert summaries(L, p, out=bad) == NULLP
    bad = state()
    bad.m = bad.m + 4
    assert summaries(L, p, out=bad) == MISAL
    # summaries overlapping an input
    assert summaries(L, p, out=state(base=Q)) == ALIAS
    # o overlapping q
    assert L.hla_fwd_output(ctypes.byref(p), Q, K, V, ctypes.byref(state()), Q + 64, None,
                            None, 0, None) == ALIAS
    assert L.hla_fwd_output(ctypes.byref(p), Q, K, V, ctypes.byref(state()), None, None,
                            None, 0, None) == NULLP


def test_workspace_sizes(L):
    per = 32 * 32 + 2 * 32 * 16 + 2 * 32
    # up to 16 segments per unit: one run, rescanned in place, no scratch
    for n in (4, 5, 16):
        p = problem(B=1, H=2, T=n * 64, chunk=64, d=32, dv=16)
        assert L.hla_scan_workspace_bytes(ctypes.byref(p)) == 0
        assert L.hla_fwd_workspace_bytes(ctypes.byref(p)) == 2 * n * per * 4
    # n = 40: runs of 8 segments (8^2 >= 40), 5 run totals + 3 padding slots
    # of the tree over them = 8 summaries per unit
    p = problem(B=1, H=2, T=40 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_workspace_bytes(ctypes.byref(p)) == 2 * 8 * per * 4
    summ = 2 * 40 * per * 4
    assert L.hla_fwd_workspace_bytes(ctypes.byref(p)) == summ + 2 * 8 * per * 4
    # n = 512: runs of 32, 16 run totals (a power of two: no padding)
    p = problem(B=1, H=2, T=512 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_workspace_bytes(ctypes.byref(p)) == 2 * 16 * per * 4
    assert L.hla_scan_workspace_bytes(ctypes.byref(problem(T=10))) == 0   # invalid -> 0
    # too small a workspace is rejected before anything runs
    assert L.hla_scan(ctypes.byref(p), ctypes.byref(state()), None, 0x7000000000, 16, None) == WS
    assert L.hla_fwd(ctypes.byref(p), Q, K, V, O, None, None, 0x7000000000, 16, None) == WS


def test_noalloc_limits_and_checks(L):
    cap = L.hla_fwd_noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    f = L.hla_fwd_noalloc
    # a problem whose workspace exceeds the fixed scratch is refused up front
    big = problem(B=4, H=16, T=16384, d=128, dv=128, chunk=128)
    assert L.hla_fwd_workspace_bytes(ctypes.byref(big)) > cap
    assert f(ctypes.byref(big), Q, K, V, O, None, None, None) == WS
    # the same argument checks as hla_fwd, before any HIP call
    p = problem()
    assert f(ctypes.byref(problem(T=10)), Q, K, V, O, None, None, None) == SHAPE
    assert f(ctypes.byref(p), None, K, V, O, None, None, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, None, None, None, None) == NULLP
    assert f(ctypes.byref(p), Q + 8, K, V, O, None, None, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, Q, None, None, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, O, None, ctypes.byref(state(base=K)), None) == ALIAS
    # an empty problem is a no-op
    assert f(ctypes.byref(problem(T=0)), None, None, None, None, None, None, None) == OK


def test_segment_local_p_sizes_and_checks(L):
    # bf16 with d = dv = 128 only: [B, H, n, ceil(chunk / 64), d, 64] bf16
    p = problem(B=1, H=2, T=576, d=128, dv=128, chunk=96)
    assert L.hla_fwd_p_bytes(ctypes.byref(p)) == 2 * 6 * 2 * 128 * 64 * 2
    for kw in (dict(d=64, dv=64), dict(d=128, dv=64), dict(in_dtype=hla.HLA_F32, d=64, dv=64),
               dict(T=10)):
        q = problem(**dict(dict(B=1, H=2, T=576, d=128, dv=128, chunk=96), **kw))
        assert L.hla_fwd_p_bytes(ctypes.byref(q)) == 0, kw
    # hla_fwd's fastest plan: the summaries (and scan scratch, none here)
    # rounded up to 256 bytes, then p over hla_fwd's spans, then room for the
    # exclusive prefixes out of place, as large as the summaries (R = 1 here:
    # 2 units of 6 segments, so the summaries fill the minimum workspace)
    r256 = lambda x: (x + 255) // 256 * 256
    base = L.hla_fwd_workspace_bytes(ctypes.byref(p))
    assert L.hla_fwd_p_workspace_bytes(ctypes.byref(p)) == \
        r256(r256(base) + L.hla_fwd_p_bytes(ctypes.byref(p))) + base
    q64 = problem()   # no p path; spans of one chunk
    base = L.hla_fwd_workspace_bytes(ctypes.byref(q64))
    assert L.hla_fwd_p_workspace_bytes(ctypes.byref(q64)) == r256(base) + base
    # spans of 4 chunks: the minimum workspace, sized for one summary per
    # chunk, has room for the span prefixes
    w = problem(B=4, H=16, T=4096, d=64, dv=64, chunk=64)
    assert L.hla_fwd_span_chunks(ctypes.byref(w)) == 4
    assert L.hla_fwd_p_workspace_bytes(ctypes.byref(w)) == L.hla_fwd_workspace_bytes(ctypes.byref(w))
    # argument checks before anything runs
    st = ctypes.byref(state())
    assert L.hla_fwd_chunk_summaries_p(ctypes.byref(q64), Q, K, V, st, DEN, None) == UNSUP
    assert L.hla_fwd_chunk_summaries_p(ctypes.byref(p), Q, K, V, st, None, None) == NULLP
    assert L.hla_fwd_chunk_summaries_p(ctypes.byref(p), Q, K, V, st, DEN + 8, None) == MISAL
    assert L.hla_fwd_chunk_summaries_p(ctypes.byref(p), Q, K, V, st, Q, None) == ALIAS
    assert L.hla_fwd_output_from_p(ctypes.byref(q64), Q, V, DEN, st, O, None, None) == UNSUP
    assert L.hla_fwd_output_from_p(ctypes.byref(p), Q, V, None, st, O, None, None) == NULLP
    assert L.hla_fwd_output_from_p(ctypes.byref(p), Q, V, DEN, st, O + 4, None, None) == MISAL
    assert L.hla_fwd_output_from_p(ctypes.byref(p), Q, V, DEN, st, DEN, None, None) == ALIAS
    assert L.hla_fwd_output_from_p(ctypes.byref(p), Q, V, DEN, st, O, Q, None) == ALIAS
    # empty problems are no-ops
    e = problem(T=0, d=128, dv=128)
    assert L.hla_fwd_chunk_summaries_p(ctypes.byref(e), None, None, None, None, None, None) == OK
    assert L.hla_fwd_output_from_p(ctypes.byref(e), None, None, None, None, None, None, None) == OK


def test_run_prefix_scan_sizes_and_checks(L):
    per = 32 * 32 + 2 * 32 * 16 + 2 * 32
    # run length: n up to 16 is one run; above, the power of two R with R^2 >= n
    for n, R in ((1, 1), (5, 5), (16, 16), (17, 8), (64, 8), (65, 16), (512, 32)):
        p = problem(B=1, H=2, T=n * 64, chunk=64, d=32, dv=16)
        assert L.hla_scan_run_length(ctypes.byref(p)) == R, n
    assert L.hla_scan_run_length(ctypes.byref(problem(T=10))) == 0   # invalid -> 0
    # one run: no scratch; n = 40: 5 runs of 8, the tree pads them to 8 (3 slots)
    p = problem(B=1, H=2, T=16 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_runs_workspace_bytes(ctypes.byref(p)) == 0
    p = problem(B=1, H=2, T=40 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_runs_workspace_bytes(ctypes.byref(p)) == 2 * 3 * per * 4
    # n = 512: 16 runs, a power of two: no padding
    p = problem(B=1, H=2, T=512 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_runs_workspace_bytes(ctypes.byref(p)) == 0
    # argument checks before anything runs
    p = problem(B=1, H=2, T=40 * 64, chunk=64, d=32, dv=16)
    assert L.hla_scan_runs(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(state(base=0x7100000000)),
                           0x7000000000, 16, None) == WS
    assert L.hla_scan_runs(ctypes.byref(p), None, ctypes.byref(state()), None, 0, None) == NULLP
    # run prefixes overlapping the summaries
    assert L.hla_scan_runs(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(state()),
                           0x7000000000, 1 << 20, None) == ALIAS


def test_out_of_place_scan_checks(L):
    pre = state(base=0x7100000000)
    p = problem(d=128, dv=96)   # a head size that is not built
    assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(pre), None,
                           None, 0, None) == UNSUP
    p = problem()
    assert L.hla_scan_into(ctypes.byref(p), None, ctypes.byref(pre), None, None, 0, None) == NULLP
    assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), None, None, None, 0, None) == NULLP
    # prefixes over the summaries, or a total over the prefixes
    assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(state()), None,
                           None, 0, None) == ALIAS
    assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(pre),
                           ctypes.byref(pre), None, 0, None) == ALIAS
    # n = 64: four runs of 16, whose totals need scratch
    p = problem(T=64 * 64)
    assert L.hla_scan_workspace_bytes(ctypes.byref(p)) > 0
    assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(pre), None,
                           0x7000000000, 16, None) == WS
    if no_gpu():
        p = problem()
        assert L.hla_scan_into(ctypes.byref(p), ctypes.byref(state()), ctypes.byref(pre), None,
                               None, 0, None) == HIP


def test_empty_problem_is_a_no_op(L):
    for kw in (dict(T=0), dict(B=0), dict(H=0)):
        assert summaries(L, problem(**kw)) == OK
        assert L.hla_fwd(ctypes.byref(problem(**kw)), Q, K, V, O, None, None, None, 0, None) == OK
    assert L.hla_decode_step(0, 4, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V,
                             ctypes.byref(state()), O, None, None) == OK


def test_decode_validation(L):
    st = state()
    args = lambda **kw: dict(dict(N=2, H=2, d=128, dv=128, dt=hla.HLA_BF16, norm=1, eps=1e-6,
                                  gamma=None, q=Q, k=K, v=V, st=st, o=O, den=None), **kw)

    def call(a):
        return L.hla_decode_step(a["N"], a["H"], a["d"], a["dv"], a["dt"], a["norm"], a["eps"],
                                 a["gamma"], a["q"], a["k"], a["v"], ctypes.byref(a["st"]),
                                 a["o"], a["den"], None)
    assert call(args(N=-1)) == SHAPE
    assert call(args(dt=3)) == DTYPE
    assert call(args(norm=5)) == VALUE
    assert call(args(eps=float("nan"))) == VALUE
    assert call(args(d=96)) == UNSUP
    assert call(args(k=None)) == NULLP
    assert call(args(o=None)) == NULLP
    assert call(args(o=O + 2)) == MISAL
    assert call(args(o=Q)) == ALIAS
    assert call(args(den=O + 64)) == ALIAS
    assert call(args(st=state(base=Q))) == ALIAS


@pytest.mark.skipif(not no_gpu(), reason="checks the behaviour on a host without a GPU")
def test_valid_call_without_device_returns_hip_error(L):
    assert summaries(L, problem()) == HIP
    assert L.hla_fwd(ctypes.byref(problem()), Q, K, V, O, None, None, 0x7000000000, 1 << 40,
                     None) == HIP
    assert L.hla_fwd_noalloc(ctypes.byref(problem()), Q, K, V, O, None, None, None) == HIP
    assert L.hla_decode_step(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V,
                             ctypes.byref(state()), O, None, None) == HIP


def test_unmasked_sizes_and_checks(L):
    p = problem()                       # B2 H3 T256 d64 dv64 chunk 64: n = 4
    per = 64 * 64 + 64 * 64 + 64
    assert L.hla_unmasked_fwd_workspace_bytes(ctypes.byref(p)) == 2 * 3 * 4 * per * 4
    assert L.hla_unmasked_fwd_workspace_bytes(ctypes.byref(problem(T=10))) == 0
    need = 2 * 3 * 4 * per * 4
    W = 0x7000000000
    f = L.hla_unmasked_fwd
    assert f(ctypes.byref(problem(T=10)), Q, K, V, O, None, W, need, None) == SHAPE
    assert f(ctypes.byref(problem(d=48)), Q, K, V, O, None, W, need, None) == UNSUP
    assert f(ctypes.byref(problem(in_dtype=hla.HLA_F32, d=128, dv=128)), Q, K, V, O, None, W,
             1 << 40, None) == UNSUP
    assert f(ctypes.byref(p), None, K, V, O, None, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, None, None, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, O, None, None, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, O, None, W, need - 4, None) == WS
    assert f(ctypes.byref(p), Q, K, V, O + 4, None, W, need, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, O, None, W + 8, need, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, Q + 64, None, W, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, O, None, K, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, O, O, W, need, None) == ALIAS
    assert f(ctypes.byref(problem(B=0)), None, None, None, None, None, None, 0, None) == OK
    # the three stages: S, C, m required, G and h ignored
    mo = hla.State(S_BASE, S_BASE + 0x1000000, S_BASE + 0x2000000, None, None)
    no_m = hla.State(S_BASE, S_BASE + 0x1000000, None, None, None)
    assert L.hla_unmasked_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(no_m), None) == NULLP
    assert L.hla_unmasked_chunk_summaries(ctypes.byref(p), Q, K, V, None, None) == NULLP
    bad = hla.State(Q, S_BASE + 0x1000000, S_BASE + 0x2000000, None, None)
    assert L.hla_unmasked_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(bad), None) == ALIAS
    mis = hla.State(S_BASE + 4, S_BASE + 0x1000000, S_BASE + 0x2000000, None, None)
    assert L.hla_unmasked_scan(ctypes.byref(p), ctypes.byref(mis), None) == MISAL
    assert L.hla_unmasked_scan(ctypes.byref(problem(chunk=0)), ctypes.byref(mo), None) == SHAPE
    assert L.hla_unmasked_output(ctypes.byref(p), Q, K, V, ctypes.byref(mo), None, None, None) == NULLP
    assert L.hla_unmasked_output(ctypes.byref(p), Q, K, V, ctypes.byref(mo), S_BASE, None, None) == ALIAS
    if no_gpu():
        assert f(ctypes.byref(p), Q, K, V, O, None, W, need, None) == HIP
        assert L.hla_unmasked_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(mo), None) == HIP
        assert L.hla_unmasked_scan(ctypes.byref(p), ctypes.byref(mo), None) == HIP
        assert L.hla_unmasked_output(ctypes.byref(p), Q, K, V, ctypes.byref(mo), O, DEN, None) == HIP


def test_unmasked_decode_validation(L):
    f = L.hla_unmasked_decode_step
    mo = hla.State(S_BASE, S_BASE + 0x1000000, S_BASE + 0x2000000, None, None)
    no_c = hla.State(S_BASE, None, S_BASE + 0x2000000, None, None)
    assert f(-1, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(mo), O, None, None) == SHAPE
    assert f(2, 2, 64, 64, 7, 0, 0.0, None, Q, K, V, ctypes.byref(mo), O, None, None) == DTYPE
    assert f(2, 2, 48, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(mo), O, None, None) == UNSUP
    assert f(2, 2, 64, 64, hla.HLA_BF16, 2, 0.0, None, Q, K, V, ctypes.byref(mo), O, None, None) == VALUE
    assert f(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(no_c), O, None, None) == NULLP
    assert f(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(mo), None, None, None) == NULLP
    assert f(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, GAM + 4, Q, K, V, ctypes.byref(mo), O, None, None) == MISAL
    assert f(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(mo), Q, None, None) == ALIAS
    assert f(0, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, None, None, None, None, None, None, None) == OK
    if no_gpu():
        assert f(2, 2, 64, 64, hla.HLA_BF16, 1, 1e-6, None, Q, K, V, ctypes.byref(mo), O, DEN,
                 None) == HIP


def test_ahla_sizes_and_checks(L):
    p = problem()                       # B2 H3 T256 d64 dv64 chunk 64: n = 4
    per = 2 * 64 * 64 + 2 * 64 + 64 * 64
    need = 2 * 3 * 4 * per * 4
    assert L.hla_ahla_fwd_workspace_bytes(ctypes.byref(p)) == need
    assert L.hla_ahla_fwd_workspace_bytes(ctypes.byref(problem(T=10))) == 0
    W = 0x7000000000
    f = L.hla_ahla_fwd
    assert f(ctypes.byref(problem(T=10)), Q, K, V, O, None, W, need, None) == SHAPE
    assert f(ctypes.byref(problem(d=48)), Q, K, V, O, None, W, need, None) == UNSUP
    assert f(ctypes.byref(p), Q, K, V, None, None, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, O, None, W, need - 4, None) == WS
    assert f(ctypes.byref(p), Q, K, V, O + 4, None, W, need, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, O, None, K, need, None) == ALIAS
    step = 0x1000000
    st = hla.AhlaState(S_BASE, S_BASE + step, S_BASE + 2 * step, S_BASE + 3 * step, S_BASE + 4 * step)
    no_x = hla.AhlaState(S_BASE, S_BASE + step, S_BASE + 2 * step, S_BASE + 3 * step, None)
    assert L.hla_ahla_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(no_x), None) == NULLP
    over = hla.AhlaState(S_BASE, S_BASE + 8, S_BASE + 2 * step, S_BASE + 3 * step, S_BASE + 4 * step)
    assert L.hla_ahla_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(over), None) == MISAL
    over16 = hla.AhlaState(S_BASE, S_BASE + 16, S_BASE + 2 * step, S_BASE + 3 * step, S_BASE + 4 * step)
    assert L.hla_ahla_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(over16), None) == ALIAS
    assert L.hla_ahla_scan(ctypes.byref(problem(chunk=0)), ctypes.byref(st), None) == SHAPE
    assert L.hla_ahla_output(ctypes.byref(p), Q, K, V, ctypes.byref(st), S_BASE, None, None) == ALIAS
    assert f(ctypes.byref(problem(B=0)), None, None, None, None, None, None, 0, None) == OK
    dec = L.hla_ahla_decode_step
    no_n = hla.AhlaState(S_BASE, S_BASE + step, S_BASE + 2 * step, None, None)
    assert dec(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(no_n), O, None, None) == NULLP
    assert dec(2, 2, 48, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(st), O, None, None) == UNSUP
    assert dec(2, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, Q, K, V, ctypes.byref(st), Q, None, None) == ALIAS
    assert dec(0, 2, 64, 64, hla.HLA_BF16, 0, 0.0, None, None, None, None, None, None, None, None) == OK
    if no_gpu():
        assert dec(2, 2, 64, 64, hla.HLA_BF16, 1, 1e-6, None, Q, K, V, ctypes.byref(no_x), O, DEN,
                   None) == HIP
        assert f(ctypes.byref(p), Q, K, V, O, None, W, need, None) == HIP
        assert L.hla_ahla_chunk_summaries(ctypes.byref(p), Q, K, V, ctypes.byref(st), None) == HIP
        assert L.hla_ahla_scan(ctypes.byref(p), ctypes.byref(st), None) == HIP
        assert L.hla_ahla_output(ctypes.byref(p), Q, K, V, ctypes.byref(st), O, DEN, None) == HIP


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 64, 16)
    with pytest.raises(RuntimeError, match="CUDA/HIP"):
        hla.fwd(q, q, q, 64)


def test_bwd_sizes_and_checks(L):
    p = problem()                       # B2 H3 T256 d64 dv64 chunk 64: n = 4
    # p, dp (fp32 slots), segment states, k k^T prefixes, and (bf16 inputs) a bf16 copy of dout
    need = (2 * 6 * 256 * 64 + 2 * 6 * 4 * 64 * 64) * 4 + 6 * 256 * 64 * 2
    assert L.hla_bwd_workspace_bytes(ctypes.byref(p)) == need
    assert L.hla_bwd_workspace_bytes(ctypes.byref(problem(dv=128))) == \
        (2 * 6 * 256 * 64 + 6 * 4 * 128 * 128 + 6 * 4 * 64 * 64) * 4 + 6 * 256 * 128 * 2
    assert L.hla_bwd_workspace_bytes(ctypes.byref(problem(in_dtype=hla.HLA_F32))) == \
        (2 * 6 * 256 * 64 + 2 * 6 * 4 * 64 * 64) * 4
    assert L.hla_bwd_workspace_bytes(ctypes.byref(problem(T=10))) == 0
    DO, DQ, DK, DV = S_BASE, S_BASE + 0x1000000, S_BASE + 0x2000000, S_BASE + 0x3000000
    W = 0x7000000000
    f = L.hla_bwd
    assert f(ctypes.byref(problem(T=10)), Q, K, V, DO, DQ, DK, DV, W, need, None) == SHAPE
    # the ratio-normalised backward needs more workspace (recomputed num and
    # den, the two upstream gradients, the v = 1 channel, bf16 dp, the forward's
    # workspace); too little is refused before anything runs
    pn = problem(normalize=1, eps=1e-6)
    need_n = L.hla_bwd_workspace_bytes(ctypes.byref(pn))
    tok = 6 * 256
    assert need_n >= need + tok * 64 * 4 + tok * 4 + tok * 64 * 2 + 2 * tok * 16 * 2 + tok * 64 * 2
    assert f(ctypes.byref(pn), Q, K, V, DO, DQ, DK, DV, W, need, None) == WS
    assert f(ctypes.byref(problem(d=48)), Q, K, V, DO, DQ, DK, DV, W, need, None) == UNSUP
    assert f(ctypes.byref(p), None, K, V, DO, DQ, DK, DV, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, None, DQ, DK, DV, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, None, DV, W, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DV, None, need, None) == NULLP
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DV, W, need - 4, None) == WS
    assert f(ctypes.byref(p), Q, K, V, DO, DQ + 4, DK, DV, W, need, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, DO + 8, DQ, DK, DV, W, need, None) == MISAL
    assert f(ctypes.byref(p), Q, K, V, DO, Q + 64, DK, DV, W, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DQ + 64, DV, W, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DO, W, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DV, DV - 16, need, None) == ALIAS
    assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DV, K, need, None) == ALIAS
    assert f(ctypes.byref(problem(B=0)), None, None, None, None, None, None, None, None, 0, None) == OK
    if no_gpu():
        assert f(ctypes.byref(p), Q, K, V, DO, DQ, DK, DV, W, need, None) == HIP

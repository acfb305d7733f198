"""The forward, the decode step, the backward and the third-order forward
captured in a HIP graph (torch.cuda.CUDAGraph over the C-ABI calls on the
capturing stream) and replayed: every replay,
with eager work and synchronisations between replays, must give the same
bits as the same calls launched directly.  The library records no
hipMemsetAsync (its scratch is cleared by its own kernels), allocates nothing
inside the calls when the caller passes the workspace and outputs, and only
checks arguments on the host, so the captured calls are the eager ones."""

import pytest

from causal_prefix_scan_amd import hla, synth

from gpu_util import bits_to_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()          # raises if the HIP library is missing: no silent fallback
    return torch


# (B, H, T, d, dv, chunk, dtype, decay, normalize)
FWD_CASES = [
    (1, 2, 2048, 128, 128, 512, "bf16", True, False),   # segment-local p path, 4 segments
    (1, 2, 1024, 64, 64, 64, "bf16", False, True),      # spans of chunks, ratio-normalised
    (2, 8, 1024, 64, 64, 16, "bf16", True, True),       # spans of 4 chunks: the one-launch rescan
    (1, 1, 256, 16, 16, 32, "f32", True, True),         # fp32, 8 segments
]


def _capture(torch, fn):
    """fn run once on a side stream, then captured; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"B{c[0]}H{c[1]}T{c[2]}d{c[3]}c{c[5]}-{c[6]}")
def test_forward_graph_replays_match_eager(gpu, case):
    torch = gpu
    B, H, T, d, dv, chunk, dtype, decay, norm = case
    say("case", case)
    q, k, v, g = to_dev(synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=4100 + T + d, decay=decay))
    q2, k2, v2, g2 = to_dev(synth.make_fwd_inputs(B, H, T, d, dv, dtype, seed=4200 + T + d, decay=decay))
    eps = 1e-6
    ws = hla.fwd_workspace(q, v, chunk, g)
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    o_ref, den_ref, _ = hla.fwd(q, k, v, chunk, g, normalize=norm, eps=eps, want_den=True, workspace=ws)
    torch.cuda.synchronize()
    o_ref, den_ref = o_ref.clone(), den_ref.clone()

    graph = _capture(torch, lambda: hla.fwd(q, k, v, chunk, g, normalize=norm, eps=eps, want_den=True,
                                            workspace=ws, o=o, den=den))
    for rep in range(3):
        o.fill_(float("nan"))
        den.fill_(float("nan"))
        # eager work between replays: another forward through the same workspace
        hla.fwd(q2, k2, v2, chunk, g2, normalize=norm, eps=eps, workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), ("replay", rep, "o")
        assert torch.equal(den, den_ref), ("replay", rep, "den")


def test_decode_graph_replays_match_eager(gpu):
    """One decode step captured with fixed token buffers; each replay, after
    the next token is copied in, advances the state exactly as the eager
    steps do (the state is updated in place by both)."""
    torch = gpu
    N, H, d, dv, P, steps = 4, 4, 128, 128, 256, 5
    inp = synth.make_fwd_inputs(N, H, P, d, dv, "bf16", seed=4300)
    q, k, v, _ = to_dev(inp)
    _, _, state0 = hla.fwd(q, k, v, P, None, want_state=True)
    toks = [synth.make_decode_step(N, H, d, dv, 4301, s)[3] for s in range(steps)]
    dev = [tuple(bits_to_dev(b).reshape(N, H, -1) for b in t) for t in toks]
    eps = 1e-6

    st_e = {key: val.clone() for key, val in state0.items()}
    outs = []
    for s in range(steps):
        o, den = hla.decode_step(*dev[s], st_e, None, True, eps,
                                 den=torch.empty(N, H, dtype=torch.float32, device="cuda"))
        outs.append((o.clone(), den.clone()))
    torch.cuda.synchronize()

    st_g = {key: val.clone() for key, val in state0.items()}
    tq, tk, tv = (x.clone() for x in dev[0])
    o = torch.empty(N, H, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(N, H, dtype=torch.float32, device="cuda")
    # _capture runs the step once before capturing it: undo that update
    saved = {key: val.clone() for key, val in st_g.items()}
    graph = _capture(torch, lambda: hla.decode_step(tq, tk, tv, st_g, None, True, eps, o=o, den=den))
    for key in st_g:
        st_g[key].copy_(saved[key])
    torch.cuda.synchronize()
    for s in range(steps):
        for dst, src in zip((tq, tk, tv), dev[s]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, outs[s][0]), ("step", s, "o")
        assert torch.equal(den, outs[s][1]), ("step", s, "den")
    for key in st_g:
        assert torch.equal(st_g[key], st_e[key]), ("state", key)


def test_backward_graph_replays_match_eager(gpu):
    """hla_bwd (its 14 launches, the workspace passed in) captured once and
    replayed: the same bits as the eager call on every replay."""
    import ctypes

    import numpy as np
    torch = gpu
    B, H, T, d, dv, chunk = 1, 2, 512, 64, 64, 128
    say("backward graph", (B, H, T, d, dv, chunk))
    q, k, v, g = to_dev(synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=4400, decay=True))
    rng = np.random.default_rng(4401)
    dout = torch.from_numpy(rng.standard_normal((B, H, T, dv)).astype(np.float32)).cuda()
    dout2 = torch.from_numpy(rng.standard_normal((B, H, T, dv)).astype(np.float32)).cuda()
    p = hla.make_problem(q, v, chunk, g)
    ws = torch.empty(max(hla.lib().hla_bwd_workspace_bytes(ctypes.byref(p)), 16), dtype=torch.uint8,
                     device="cuda")
    ref = [x.clone() for x in hla.bwd(q, k, v, dout, chunk, g, workspace=ws)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(x) for x in ref]
    graph = _capture(torch, lambda: hla.bwd(q, k, v, dout, chunk, g, workspace=ws, dq=outs[0], dk=outs[1],
                                            dv=outs[2]))
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        hla.bwd(q, k, v, dout2, chunk, g, workspace=ws)   # eager work through the same workspace
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, want), ("replay", rep, name)


def test_third_order_graph_replays_match_eager(gpu):
    """hla3_fwd captured once and replayed: the same bits as the eager call."""
    torch = gpu
    B, H, T, d, dv, chunk = 1, 2, 768, 64, 64, 128
    say("third-order graph", (B, H, T, d, dv, chunk))
    q, k, v, g = to_dev(synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=4500, decay=True))
    o_ref, den_ref, _ = hla.hla3_fwd(q, k, v, chunk, g, want_den=True)
    torch.cuda.synchronize()
    o_ref, den_ref = o_ref.clone(), den_ref.clone()
    o = torch.empty_like(o_ref)
    den = torch.empty_like(den_ref)
    graph = _capture(torch, lambda: hla.hla3_fwd(q, k, v, chunk, g, want_den=True, o=o, den=den))
    for rep in range(3):
        o.fill_(float("nan"))
        den.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), ("replay", rep, "o")
        assert torch.equal(den, den_ref), ("replay", rep, "den")

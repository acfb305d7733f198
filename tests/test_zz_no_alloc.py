"""hla_fwd_noalloc (the forward with the library's own fixed scratch) against
hla_fwd (the same forward with a caller workspace), through the C ABI: two
calls in a row on one device, the second with a smaller problem, each equal
bit for bit to hla_fwd on the same inputs given the minimum workspace (the
same kernels and launches: without room for the segment-local p, hla_fwd
takes the plan the fixed scratch holds); the first also against the fp64
oracle at the bf16 tolerance."""

import numpy as np
import pytest

from causal_prefix_scan_amd import hla, synth
from oracle import hla_oracle as O

from gpu_util import host, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("S", "C", "m", "G", "h")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hla.lib()
    return torch


# (B, H, T, d, dv, chunk, decay, normalize, want_state): the first is the
# larger; the third has 40 segments per head, so the scan's scratch is used
CASES = [
    (2, 8, 4096, 128, 128, 1024, True, False, True),
    (1, 3, 768, 64, 64, 256, False, True, False),
    (1, 2, 2560, 64, 64, 64, True, False, True),
    (1, 1, 256, 32, 32, 64, True, True, False),
]


def one(torch, case, seed, check_oracle):
    B, H, T, d, dv, chunk, decay, norm, want_state = case
    say("noalloc case", case)
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", seed=seed, decay=decay)
    q, k, v, g = to_dev(inp)
    p = hla.make_problem(q, v, chunk, g, norm, 1e-6)
    import ctypes
    need = hla.lib().hla_fwd_workspace_bytes(ctypes.byref(p))
    assert 0 < need <= hla.lib().hla_fwd_noalloc_max_workspace_bytes()
    ws = hla.fwd_workspace(q, v, chunk, g, with_p=False)
    assert ws.numel() == need
    o1, d1, s1 = hla.fwd(q, k, v, chunk, g, normalize=norm, eps=1e-6, want_den=True,
                         want_state=want_state, workspace=ws)
    o2, d2, s2 = hla.fwd_noalloc(q, k, v, chunk, g, normalize=norm, eps=1e-6, want_den=True,
                                 want_state=want_state)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(d1, d2)
    if want_state:
        for key in FIELDS:
            assert torch.equal(s1[key], s2[key]), key
    if check_oracle:
        uq, uk, uv, ug = inp.units()
        num, den, _ = O.serial(uq, uk, uv, ug)
        if not norm:
            e = rel_err(host(o2).reshape(num.shape), num)
            say(f"  num vs oracle {e:.2e}")
            assert e <= 2e-2
        e = rel_err(host(d2).reshape(den.shape), den)
        assert e <= 2e-2


def test_noalloc_matches_fwd_two_calls_shrinking(gpu):
    torch = gpu
    for i, case in enumerate(CASES):
        one(torch, case, seed=500 + i, check_oracle=(i % 2 == 1))

"""Helpers shared by the GPU tests: device copies of the seeded inputs and
error metrics.  No attention arithmetic lives here."""

import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(inp):
    """FwdInputs -> (q, k, v, gamma) device tensors with the exact same values."""
    torch = torch_mod()
    if inp.dtype == "bf16":
        cv = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (inp.q, inp.k, inp.v))
    g = None if inp.gamma is None else torch.from_numpy(inp.gamma).cuda()
    return q, k, v, g


def bits_to_dev(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    scale = np.max(np.abs(want))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / scale)


def state_host(st, lead_slice=None):
    out = {}
    for key in ("S", "C", "m", "G", "h"):
        x = st[key]
        if lead_slice is not None:
            x = x[lead_slice]
        out[key] = host(x)
    return out

"""Helpers shared by the GPU tests: move seeded inputs to the device, call the
library through the C ABI, and compute the matching oracle result on the host.

The device gets Omega from the library's generator and the oracle gets it from
its own generator; both implement the same published stream (their agreement
is a host test).  Everything else (q, k, v, M, mask) is the same array.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import Workload, make_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def device_inputs(w: Workload, inp: dict):
    import torch
    dt = torch_dtype(w.dtype)
    dev = {
        "q": to_dev(inp["q"], dt), "k": to_dev(inp["k"], dt), "v": to_dev(inp["v"], dt),
        "M": to_dev(inp["M"], torch.float32),
        "omega": to_dev(bd.dark_prf_omega(w.seed, w.m, w.r, w.orthogonal), torch.float32),
        "mask": to_dev(inp["mask"]) if inp["mask"] is not None else None,
    }
    return dev


def oracle_omega(w: Workload) -> np.ndarray:
    return oracle.omega(w.seed, w.m, w.r, w.orthogonal)


def run_device(w: Workload, dev: dict, return_state=False):
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    res = bd.prf_attention(dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"], mask=dev["mask"],
                           causal=w.causal, return_state=return_state, proj_tag=tag)
    return res


def host(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()

"""Helpers for the GPU tests: move seeded inputs to the device and compare
against the float64 oracle with the stated tolerances."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from mla_latent_kv_05_amd import binding, inputs

# bf16 / fp8 caches with fp32 accumulation: max-abs and mean-abs bounds
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# self-imposed, tighter checks (norm-relative error, lse)
BF16_NORM_REL = 1e-2
LSE_ABS = 1e-3
# fp32 inputs: relative error max|g-o| / max|o|
F32_REL = 1e-5


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a hard failure still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def case_to_device(case: inputs.DecodeCase, device="cuda") -> dict:
    q = bf16_dev if case.q_dtype == "bf16" else f32_dev
    if case.kv_dtype == "bf16":
        cache = bf16_dev(case.cache, device)
        kvdt = binding.MLA_BF16
    elif case.kv_dtype == "f32":
        cache = f32_dev(case.cache, device)
        kvdt = binding.MLA_F32
    else:
        cache = torch.from_numpy(np.ascontiguousarray(case.cache)).to(device)
        kvdt = {"fp8": binding.MLA_FP8_E4M3, "int4": binding.MLA_INT4, "int2": binding.MLA_INT2}[case.kv_dtype]
    table = np.where(case.block_table >= 0, case.block_table, 0).astype(np.int32)
    return dict(q_lat=q(case.q_lat, device), q_rope=q(case.q_rope, device), kv_cache=cache,
                block_table=torch.from_numpy(table).to(device),
                seq_lens=torch.from_numpy(case.seq_lens.astype(np.int32)).to(device), kv_dtype=kvdt,
                d_r=case.d_r, block_size=case.block_size, softmax_scale=case.softmax_scale)


def run_decode(case, out_dtype=torch.float32, **kw):
    d = case_to_device(case)
    o, lse = binding.decode(d["q_lat"], d["q_rope"], d["kv_cache"], d["block_table"], d["seq_lens"],
                            d["softmax_scale"], kv_dtype=d["kv_dtype"], d_r=d["d_r"],
                            block_size=d["block_size"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def errors(g: np.ndarray, o: np.ndarray) -> dict:
    d = np.abs(g - o)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "norm_rel": float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300)),
            "max_rel": float(d.max() / max(np.abs(o).max(), 1e-300))}


def assert_bf16_close(g, o, what=""):
    e = errors(g, o)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {e}"
    assert e["norm_rel"] <= BF16_NORM_REL, f"{what}: {e}"
    return e


def assert_f32_close(g, o, what="", tol=F32_REL):
    e = errors(g, o)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert e["max_rel"] <= tol, f"{what}: {e}"
    return e


def assert_lse_close(g, o, what="", tol=LSE_ABS):
    fin = np.isfinite(o)
    assert np.array_equal(fin, np.isfinite(g)), f"{what}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(g[fin] - o[fin]).max())
        assert err <= tol, f"{what}: lse err {err}"

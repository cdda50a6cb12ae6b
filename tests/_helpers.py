"""Shared helpers for the GPU parity tests: upload a workload, run the HIP path
through the C ABI, run the oracle on the same bytes, compare."""
from __future__ import annotations

import os

import numpy as np
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import c_oracle

# Parity bounds of the decode output against the fp64 oracle: bf16/fp32 cache:
# max-abs <= 1e-2 and mean-abs <= 1e-3; fp8 e4m3 cache: max-abs <= 3e-2
# (mean-abs reported).  int8 and int4 caches (no stated figure): their values
# widen to bf16 exactly and take the bf16 path's arithmetic, so the bf16
# bounds apply.
TOL = {"f32": (1e-2, 1e-3), "bf16": (1e-2, 1e-3), "fp8": (3e-2, None), "i8": (1e-2, 1e-3), "i4": (1e-2, 1e-3)}
DECODE_SCALED = {"fp8": "paged_attn_decode_fp8", "i8": "paged_attn_decode_int8", "i4": "paged_attn_decode_int4"}
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# (what, kv dtype, elements, max-abs, mean-abs) of every full-workload comparison
# made with ``report=True``; conftest prints them at the end of the run.
PARITY_LOG: list = []


def dev_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def host_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


class DeviceWorkload:
    """A workload's tensors resident in HBM."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.q = dev_tensor(wl.q, device)
        self.k_pool = dev_tensor(wl.k_pool, device)
        self.v_pool = dev_tensor(wl.v_pool, device)
        self.bt = dev_tensor(wl.block_tables, device)
        self.sl = dev_tensor(wl.seq_lens, device)
        self.ks = None if wl.k_scales is None else dev_tensor(wl.k_scales, device)
        self.vs = None if wl.v_scales is None else dev_tensor(wl.v_scales, device)
        odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
        self.out = torch.empty((wl.B, wl.Hq, wl.D), dtype=odt, device=device)
        nbytes = pkv.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D)
        self.ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)

    def decode(self, seq_lens=None, partition_tokens=None, out=None):
        wl = self.wl
        sl = self.sl if seq_lens is None else seq_lens
        pt = wl.partition_tokens if partition_tokens is None else partition_tokens
        out = self.out if out is None else out
        if wl.kv_dtype in DECODE_SCALED:
            fn = getattr(pkv, DECODE_SCALED[wl.kv_dtype])
            fn(self.q, wl.q_dtype, self.k_pool, self.v_pool, self.ks, self.vs, self.bt, sl, wl.Hq, wl.Hkv,
               wl.D, wl.P, wl.scale, out, wl.out_dtype, self.ws, pt)
        else:
            pkv.paged_attn_decode(self.q, wl.q_dtype, self.k_pool, self.v_pool, wl.kv_dtype, self.bt,
                                  sl, wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype,
                                  self.ws, pt)
        return out

    def step(self, k_new, v_new, seq_lens, partition_tokens=None, out=None):
        """Fused append + decode (decode_step entry point)."""
        wl = self.wl
        pt = wl.partition_tokens if partition_tokens is None else partition_tokens
        out = self.out if out is None else out
        pkv.decode_step(self.q, wl.q_dtype, k_new, v_new, self.k_pool, self.v_pool, wl.kv_dtype, self.bt,
                        seq_lens, wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, self.ws,
                        k_scales=self.ks, v_scales=self.vs, partition_tokens=pt)
        return out

    def append(self, k_new, v_new, seq_lens):
        wl = self.wl
        pkv.kv_append(k_new, v_new, wl.kv_dtype, self.bt, seq_lens, self.k_pool, self.v_pool,
                      wl.Hkv, wl.D, wl.P)


# Logit of token t (q = ones, K rows c_t / D, scale 1) for tests of the
# softmax reference: it grows every tile, every few tiles, once, only in the
# last tile, or at alternating tiles; and logits near 900.
LOGIT_PROFILES = {
    "fast_ramp_up": lambda t, L, r: 0.5 * t,                 # the reference grows every tile
    "slow_ramp_up": lambda t, L, r: 0.02 * t,                # grows every few tiles, lags in between
    "ramp_down": lambda t, L, r: 100.0 - 0.5 * t,            # the first tile sets it for good
    "large_offset": lambda t, L, r: 900.0 + 2.0 * r.standard_normal(len(t)),
    "last_token_spike": lambda t, L, r: np.where(t == L - 1, 60.0, 0.0),
    "alternating": lambda t, L, r: np.where((t // 32) % 2 == 0, 0.0, 30.0),
}


def oracle_decode(wl, k_pool=None, v_pool=None, seq_lens=None, pairs=None):
    return c_oracle.decode(wl.q, wl.q_dtype, wl.k_pool if k_pool is None else k_pool,
                           wl.v_pool if v_pool is None else v_pool, wl.kv_dtype, wl.block_tables,
                           wl.seq_lens if seq_lens is None else seq_lens, wl.Hq, wl.P, wl.scale,
                           wl.k_scales, wl.v_scales, pairs=pairs, nthreads=ORACLE_THREADS)


def gpu_out(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (the most that rounding a value to bf16 can move it)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 8)


def check_close(got: np.ndarray, ref: np.ndarray, kv_dtype: str, what: str = "",
                out_rounding: bool = False, report: bool = False):
    """Element-wise comparison at the parity bounds above; returns (max, mean).

    With ``out_rounding`` (bf16 outputs of large magnitude in edge-case tests),
    each element may additionally differ by the half-ulp that storing the exact
    result as bf16 costs, and the mean bound grows by the mean of that allowance.
    """
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(ref).all(), f"{what}: oracle produced non-finite values"
    assert np.isfinite(got).all(), f"{what}: GPU produced non-finite values"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    if report:
        PARITY_LOG.append((what, kv_dtype, int(err.size), mx, mean))
    tmax, tmean = TOL[kv_dtype]
    allow = bf16_half_ulp(ref) if out_rounding else np.zeros_like(ref)
    worst = float((err - allow).max()) if err.size else 0.0
    assert worst <= tmax, f"{what}: max-abs {mx:.3e} exceeds {tmax} (+ output rounding {out_rounding})"
    if tmean is not None:
        lim = tmean + (float(allow.mean()) if err.size else 0.0)
        assert mean <= lim, f"{what}: mean-abs {mean:.3e} > {lim:.3e}"
    return mx, mean

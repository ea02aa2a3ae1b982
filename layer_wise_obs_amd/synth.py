"""Seeded synthetic inputs for the layer-pruning path.

This module only draws input tensors (weights W and token-major calibration
activations X). It holds none of the pruning arithmetic. The same function runs
on the CPU and on the GPU and produces the same bytes on both, because every
value comes from integer arithmetic on a counter (the element's flat index)
followed by exactly rounded fp32 multiplies and one round-to-nearest-even cast:

* ``_mix32`` is a 32-bit integer finaliser (xorshift-multiply, constants chosen
  below 2**31 so the products never leave int64);
* a normal-like variate is the Irwin-Hall sum of eight 16-bit uniforms taken
  from two mixed 32-bit words, centred and scaled to unit variance;
* outlier channels are the ``k`` channels with the smallest mixed channel key
  (ties broken by index), multiplied by a fixed factor before rounding;
* "ReLU-like" activations are ``max(0, z)``.

The pages measure on LLaMA models calibrated with 128 C4 sequences of 2048
tokens ("Pruning LLMs with Thanos", section "What the experiments show"; the
Wanda section of the weight-pruning explainer). Neither the weights nor C4 are
used here: these generators stand in for them with the same layer shapes and
token counts, and with a few channels that are much larger than average (the
explainer's section on magnitude pruning describes activation outliers up to
100x the average).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

M32 = 0xFFFFFFFF
_MUL1 = 0x21F0AAAD
_MUL2 = 0x735A2D97
# Irwin-Hall(8) of 16-bit uniforms: mean 8*32767.5, variance 8*(65536**2-1)/12.
_IH_MEAN = 8 * 65535 // 2
_IH_STD = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """32-bit avalanche mix of an int64 tensor holding values in [0, 2**32)."""
    x = x ^ (x >> 16)
    x = (x * _MUL1) & M32
    x = x ^ (x >> 15)
    x = (x * _MUL2) & M32
    x = x ^ (x >> 15)
    return x


def _key(seed: int, tensor_id: int, lane: int) -> int:
    v = (seed * 0x9E3779B1 + tensor_id * 0x85EBCA6B + lane * 0xC2B2AE35) & M32
    v ^= v >> 16
    v = (v * _MUL1) & M32
    v ^= v >> 15
    v = (v * _MUL2) & M32
    v ^= v >> 15
    return v


def _word(e: torch.Tensor, key: int) -> torch.Tensor:
    lo = e & M32
    hi = e >> 32
    return _mix32(_mix32((lo + key) & M32) ^ ((hi * 0x27D4EB2F + key) & M32))


def normal_like(e: torch.Tensor, seed: int, tensor_id: int) -> torch.Tensor:
    """Unit-variance, zero-mean fp32 variates for flat element indices ``e``.

    The value is an integer in [-262140, 262140] times one fp32 constant, so it
    is reproduced bit for bit on any device.
    """
    w0 = _word(e, _key(seed, tensor_id, 0))
    w1 = _word(e, _key(seed, tensor_id, 1))
    s = (w0 & 0xFFFF) + (w0 >> 16) + (w1 & 0xFFFF) + (w1 >> 16)
    w2 = _mix32(w0 ^ w1)
    w3 = _mix32((w1 + 0x9E3779B9) & M32)
    s = s + (w2 & 0xFFFF) + (w2 >> 16) + (w3 & 0xFFFF) + (w3 >> 16)
    return (s - _IH_MEAN).to(torch.float32)


def _scale_const(x: float, device) -> torch.Tensor:
    return torch.tensor(x, dtype=torch.float32, device=device)


def outlier_channels(b: int, count: int, seed: int, tensor_id: int) -> torch.Tensor:
    """Indices of ``count`` outlier channels out of ``b`` (sorted ascending)."""
    if count <= 0:
        return torch.zeros(0, dtype=torch.int64)
    ch = torch.arange(b, dtype=torch.int64)
    k = _mix32((ch + _key(seed, tensor_id, 7)) & M32)
    order = torch.argsort(k * b + ch)  # unique keys: ties broken by index
    return torch.sort(order[:count]).values


def weights(c: int, b: int, sigma: float, seed: int, tensor_id: int,
            dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """W [c, b] row-major, ~N(0, sigma^2) (Irwin-Hall approximation)."""
    out = torch.empty((c, b), dtype=dtype, device=device)
    rows = max(1, (1 << 24) // max(b, 1))
    k_sig = _scale_const(sigma / _IH_STD, device)
    for r0 in range(0, c, rows):
        r1 = min(c, r0 + rows)
        e = torch.arange(r0 * b, r1 * b, dtype=torch.int64, device=device)
        v = normal_like(e, seed, tensor_id) * k_sig
        out[r0:r1] = v.view(r1 - r0, b).to(dtype)
    return out


def activations(n: int, b: int, seed: int, tensor_id: int, outlier_count: int,
                outlier_scale: float, relu: bool = False, dtype=torch.bfloat16,
                device="cpu", token_offset: int = 0, chunk_tokens: int = 8192,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Token-major calibration activations X^T [n, b] (X is b x n with tokens as columns).

    Tokens ``token_offset .. token_offset+n`` of the stream are produced, so any
    token range can be regenerated on its own.
    """
    if out is None:
        out = torch.empty((n, b), dtype=dtype, device=device)
    k_one = _scale_const(1.0 / _IH_STD, device)
    col_scale = torch.ones(b, dtype=torch.float32)
    oc = outlier_channels(b, outlier_count, seed, tensor_id)
    if len(oc):
        col_scale[oc] = float(outlier_scale)
    col_scale = col_scale.to(device)
    has_out = len(oc) > 0
    step = max(1, min(chunk_tokens, (1 << 25) // max(b, 1)))
    for t0 in range(0, n, step):
        t1 = min(n, t0 + step)
        e = torch.arange((token_offset + t0) * b, (token_offset + t1) * b,
                         dtype=torch.int64, device=device)
        v = (normal_like(e, seed, tensor_id) * k_one).view(t1 - t0, b)
        if has_out:
            v = v * col_scale
        if relu:
            v = torch.clamp_min(v, 0.0)
        out[t0:t1] = v.to(dtype)
    return out


@dataclass
class Layer:
    name: str
    c: int
    b: int
    hessian: str  # name of the input stream whose Hessian this layer uses


@dataclass
class Stream:
    name: str
    b: int
    n: int
    outlier_count: int
    outlier_scale: float
    relu: bool
    tensor_id: int


@dataclass
class Config:
    """One workload: layers, calibration streams and pruning settings."""
    cid: int
    seed: int
    wdtype: torch.dtype
    xdtype: torch.dtype
    sigma: float
    layers: list = field(default_factory=list)
    streams: dict = field(default_factory=dict)
    patterns: list = field(default_factory=list)  # ("unstructured", p) or ("nm", n, m)
    block: int = 128
    lambda_rel: float = 0.01

    def weights(self, layer: Layer, device="cpu") -> torch.Tensor:
        tid = 100 + [l.name for l in self.layers].index(layer.name)
        return weights(layer.c, layer.b, self.sigma, self.seed, tid, self.wdtype, device)

    def activations(self, stream: str, device="cpu", n: int | None = None,
                    token_offset: int = 0, out=None) -> torch.Tensor:
        s = self.streams[stream]
        return activations(s.n if n is None else n, s.b, self.seed, s.tensor_id,
                           s.outlier_count, s.outlier_scale, s.relu, self.xdtype,
                           device, token_offset=token_offset, out=out)


def _round_frac(frac: float, b: int) -> int:
    return int(round(frac * b))


def config(cid: int) -> Config:
    """The five synthetic workloads (shapes of LLaMA-7B / LLaMA-2-70B layers)."""
    seed = 20250406 + cid
    if cid == 1:
        cfg = Config(1, seed, torch.float32, torch.float32, 0.02, block=32)
        cfg.streams["x"] = Stream("x", 256, 512, 4, 20.0, False, 1)
        cfg.layers = [Layer("fc", 128, 256, "x")]
        cfg.patterns = [("unstructured", 0.5)]
        return cfg
    if cid == 2:
        cfg = Config(2, seed, torch.bfloat16, torch.bfloat16, 0.02)
        cfg.streams["attn_in"] = Stream("attn_in", 4096, 262144, _round_frac(0.01, 4096), 50.0, False, 1)
        cfg.layers = [Layer("q_proj", 4096, 4096, "attn_in")]
        cfg.patterns = [("nm", 2, 4)]
        return cfg
    if cid == 3:
        cfg = Config(3, seed, torch.bfloat16, torch.bfloat16, 0.02)
        cfg.streams["down_in"] = Stream("down_in", 11008, 262144, _round_frac(0.01, 11008), 30.0, True, 1)
        cfg.layers = [Layer("down_proj", 4096, 11008, "down_in")]
        cfg.patterns = [("nm", 2, 4), ("nm", 4, 8)]
        return cfg
    if cid == 4:
        cfg = Config(4, seed, torch.bfloat16, torch.bfloat16, 0.02)
        n = 131072
        cfg.streams["attn_in"] = Stream("attn_in", 4096, n, 41, 50.0, False, 1)
        cfg.streams["o_in"] = Stream("o_in", 4096, n, 41, 50.0, False, 2)
        cfg.streams["mlp_in"] = Stream("mlp_in", 4096, n, 41, 50.0, False, 3)
        cfg.streams["down_in"] = Stream("down_in", 11008, n, 110, 30.0, True, 4)
        cfg.layers = [Layer("q_proj", 4096, 4096, "attn_in"), Layer("k_proj", 4096, 4096, "attn_in"),
                      Layer("v_proj", 4096, 4096, "attn_in"), Layer("o_proj", 4096, 4096, "o_in"),
                      Layer("gate_proj", 11008, 4096, "mlp_in"), Layer("up_proj", 11008, 4096, "mlp_in"),
                      Layer("down_proj", 4096, 11008, "down_in")]
        cfg.patterns = [("unstructured", 0.5)]
        return cfg
    if cid == 5:
        cfg = Config(5, seed, torch.bfloat16, torch.bfloat16, 0.015)
        n = 65536
        cfg.streams["attn_in"] = Stream("attn_in", 8192, n, 82, 100.0, False, 1)
        cfg.streams["o_in"] = Stream("o_in", 8192, n, 82, 100.0, False, 2)
        cfg.streams["down_in"] = Stream("down_in", 28672, n, 287, 100.0, False, 3)
        cfg.layers = [Layer("k_proj", 1024, 8192, "attn_in"), Layer("v_proj", 1024, 8192, "attn_in"),
                      Layer("q_proj", 8192, 8192, "attn_in"), Layer("o_proj", 8192, 8192, "o_in"),
                      Layer("down_proj", 8192, 28672, "down_in")]
        cfg.patterns = [("unstructured", 0.6), ("nm", 2, 4)]
        return cfg
    raise ValueError(f"unknown config {cid}")


def small_problem(c: int, b: int, n: int, seed: int, outliers: int = 2,
                  outlier_scale: float = 20.0, relu: bool = False,
                  wdtype=torch.float32, xdtype=torch.float32, sigma: float = 0.02,
                  device="cpu"):
    """A small (W, X^T) pair for tests: W [c,b], X^T [n,b]."""
    W = weights(c, b, sigma, seed, 100, wdtype, device)
    X = activations(n, b, seed, 1, outliers, outlier_scale, relu, xdtype, device)
    return W, X

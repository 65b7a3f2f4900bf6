"""Seeded synthetic inputs of diffusion-transformer linear layers at 1K images.

This module only draws inputs: it holds none of the method's arithmetic (no
quantisation, transform, GEMM or epilogue), so both the CPU oracle's tests and
the GPU path take their inputs from here.

The pages run their models on trained weights and image datasets that are not
available; these synthetic tensors stand in for them.  A 1K image is 4096
tokens; hidden sizes 3072 / 4096 and the FFN width 12288 are DiT-typical.
Recipe (every stream seeded by numpy.random.default_rng([workload, stream])):

* activations: N(0, 1) in float32; round(0.005 * K) channels, drawn without
  replacement, are multiplied by 20 (the activation outliers the KroQuant
  page names as the obstacle to W4A4); then rounded to bfloat16 where the
  workload's activations are bfloat16.
* weights: N(0, 1/sqrt(K)) (standard deviation 1/sqrt(K)), float32, logical
  layout [K, N] of y = x @ W.
* RMSNorm gains: U(0.5, 1.5), one vector of head_dim for Q and one for K,
  repeated over the heads.
* block transforms: T_b = Q1 diag(s) Q2 with Haar-random orthogonal Q1, Q2
  and singular values s log-uniform in [1, 9.5] with both end points present,
  rounded to bfloat16 and drawn again until cond(T_b) < 10.

Stream ids: 0 activations (QKV input), 1 QKV / first weight, 2 FFN up weight,
3 outlier channels, 4 RMSNorm gains, 5 / 9 / 10 block transforms of the QKV /
FFN-up / FFN-down inputs, 6 FFN down weight, 7 activations of the FFN input,
8 FFN gate weight, 11 stand-in activations of the FFN down input.
"""

from dataclasses import dataclass, field

import numpy as np

EPS = 1e-6


def rng(workload: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([workload, stream])


def to_bf16_values(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned
    as float32 arrays holding exactly representable bf16 values."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def activations(workload: int, stream: int, rows: int, cols: int, outlier_stream: int = 3,
                bf16: bool = True) -> np.ndarray:
    x = rng(workload, stream).standard_normal((rows, cols), dtype=np.float32)
    n_out = int(round(0.005 * cols))
    if n_out:
        ch = rng(workload, outlier_stream).choice(cols, n_out, replace=False)
        x[:, ch] *= 20.0
    return to_bf16_values(x) if bf16 else x


def weight(workload: int, stream: int, k: int, n: int) -> np.ndarray:
    w = rng(workload, stream).standard_normal((k, n), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(k))
    return w


def norm_gains(workload: int, head_dim: int, heads_q: int, heads_k: int) -> np.ndarray:
    g = rng(workload, 4).uniform(0.5, 1.5, 2 * head_dim).astype(np.float32)
    wq, wk = g[:head_dim], g[head_dim:]
    return np.concatenate([np.tile(wq, heads_q), np.tile(wk, heads_k)])


def _haar(r: np.random.Generator, n: int) -> np.ndarray:
    q, rr = np.linalg.qr(r.standard_normal((n, n)))
    return q * np.sign(np.diag(rr))[None, :]


def transforms(workload: int, n_t: int, stream: int = 5, cond_max: float = 10.0) -> np.ndarray:
    """n_t random invertible 32x32 matrices, bfloat16 values (float32 array)."""
    r = rng(workload, stream)
    out = np.empty((n_t, 32, 32), dtype=np.float32)
    for b in range(n_t):
        while True:
            s = np.exp(r.uniform(0.0, np.log(9.5), 32))
            s[0], s[1] = 1.0, 9.5
            t = (_haar(r, 32) * s[None, :]) @ _haar(r, 32)
            tb = to_bf16_values(t.astype(np.float32))
            if np.linalg.cond(tb.astype(np.float64)) < cond_max:
                out[b] = tb
                break
    return out


@dataclass
class Workload:
    """Inputs of one fused linear layer (or of the three linears of a block)."""
    name: str
    m: int
    k: int
    x: np.ndarray                      # [M, K] float32 holding fp32 or bf16 values
    x_bf16: bool
    epilogue: str                      # "none" | "rmsnorm_head" | "swiglu"
    w: np.ndarray = None               # [K, N] logical weight (none / rmsnorm)
    w_gate: np.ndarray = None          # [K, N/2] (swiglu)
    w_up: np.ndarray = None
    head_dim: int = 0
    n_norm: int = 0
    norm_w: np.ndarray = None
    eps: float = EPS
    requant: bool = False
    t: np.ndarray = None               # [n_t, 32, 32] bf16 values, or None
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        """Physical GEMM width (both SwiGLU halves)."""
        if self.epilogue == "swiglu":
            return 2 * self.w_gate.shape[1]
        return self.w.shape[1]

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


def tiny(rows: int = 256) -> Workload:
    """X fp32 [256, 512], W [512, 512], per-head RMSNorm on 4 heads of 128."""
    x = rng(1, 0).standard_normal((256, 512), dtype=np.float32)[:rows]
    return Workload("tiny_rmsnorm_hd128", rows, 512, x, False, "rmsnorm_head",
                    w=weight(1, 1, 512, 512), head_dim=128, n_norm=512,
                    norm_w=np.tile(rng(1, 4).uniform(0.5, 1.5, 128).astype(np.float32), 4))


def qkv_hd128(rows: int = 4096) -> Workload:
    """X bf16 [4096, 3072] with outliers, W [3072, 9216] = 24 Q | 24 K | 24 V heads of 128."""
    return Workload("qkv_hd128", rows, 3072, activations(2, 0, rows, 3072), True, "rmsnorm_head",
                    w=weight(2, 1, 3072, 9216), head_dim=128, n_norm=6144,
                    norm_w=norm_gains(2, 128, 24, 24))


def qkv_hd256(rows: int = 4096) -> Workload:
    """X bf16 [4096, 4096] with outliers, W [4096, 12288] = 16 Q | 16 K | 16 V heads of 256."""
    return Workload("qkv_hd256", rows, 4096, activations(3, 0, rows, 4096), True, "rmsnorm_head",
                    w=weight(3, 1, 4096, 12288), head_dim=256, n_norm=8192,
                    norm_w=norm_gains(3, 256, 16, 16))


def ffn_up_swiglu(rows: int = 4096, requant: bool = True) -> Workload:
    """X bf16 [4096, 3072] with outliers, W_gate and W_up [3072, 12288]."""
    return Workload("ffn_up_swiglu_requant" if requant else "ffn_up_swiglu", rows, 3072,
                    activations(4, 0, rows, 3072), True, "swiglu",
                    w_gate=weight(4, 1, 3072, 12288), w_up=weight(4, 2, 3072, 12288),
                    requant=requant)


def dit_block(rows: int = 16384):
    """Batch of 4 images (16384 tokens): block transform + quantise on every
    input, QKV (RMSNorm hd 128), FFN up (SwiGLU, bf16 out), FFN down (none).
    Returns the three Workloads.  In the block the down layer's activations
    are the up layer's bf16 output; its x here (stream 11) is a seeded
    stand-in of the same shape for checking the down layer on its own."""
    qkv = Workload("dit_block_qkv", rows, 3072, activations(5, 0, rows, 3072), True, "rmsnorm_head",
                   w=weight(5, 1, 3072, 9216), head_dim=128, n_norm=6144,
                   norm_w=norm_gains(5, 128, 24, 24), t=transforms(5, 96, stream=5))
    up = Workload("dit_block_up", rows, 3072, activations(5, 7, rows, 3072), True, "swiglu",
                  w_gate=weight(5, 8, 3072, 12288), w_up=weight(5, 2, 3072, 12288),
                  t=transforms(5, 96, stream=9))
    down = Workload("dit_block_down", rows, 12288, activations(5, 11, rows, 12288), True, "none",
                    w=weight(5, 6, 12288, 3072), t=transforms(5, 384, stream=10))
    return qkv, up, down

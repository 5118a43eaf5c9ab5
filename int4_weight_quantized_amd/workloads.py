"""Seeded synthetic inputs for the int4-weight quantized linear layer.

This module only draws random data in the shapes, dtypes and value ranges of
the layers the pages discuss. It holds none of the method's arithmetic: weight
codes are drawn as uniform random bits, so every 4-bit field of a packed word
is a uniform code in 0..15 without any packing step, and floats are drawn in
fp32 and rounded to bf16/fp16 by torch's round-to-nearest-even cast.

It is shared by the oracle-side tests and the GPU side; nothing here may
depend on either of them.

Workloads (sizes from the layer shapes the pages use as examples):
  w4a8_tiny        M=16,   K=256,   N=256,   group 128, bf16 activations
  w4a8_up_proj     M=4096, K=4096,  N=14336, group 128, bf16 activations
  w4a8_down_proj   M=8192, K=14336, N=4096,  per-channel (group -1), fp16
                   activations with 1% of the K channels scaled by 20
  w4a16_decode     M in {1, 8}, K=4096, N=14336, group 64, bf16, asymmetric
  w4afp8_moe       64 experts, K=7168, N=2048, group 128, 8192 tokens routed
                   to 8 distinct experts each (uniform)
"""
from __future__ import annotations

import numpy as np
import torch

SEEDS = {
    "w4a8_tiny": 1001,
    "w4a8_up_proj": 1002,
    "w4a8_down_proj": 1003,
    "w4a16_decode": 1004,
    "w4afp8_moe": 1005,
    "w4a16_prefill": 1006,
}

SHAPES = {
    "w4a8_tiny": dict(M=16, K=256, N=256, group=128, x_dtype="bf16"),
    "w4a8_up_proj": dict(M=4096, K=4096, N=14336, group=128, x_dtype="bf16"),
    "w4a8_down_proj": dict(M=8192, K=14336, N=4096, group=-1, x_dtype="f16"),
    "w4a16_decode": dict(M=8, K=4096, N=14336, group=64, x_dtype="bf16"),
    "w4afp8_moe": dict(E=64, K=7168, N=2048, group=128, T=8192, topk=8, x_dtype="bf16"),
    # the decode layer's weights at a prefill batch (the asymmetric grid's large-batch path)
    "w4a16_prefill": dict(M=4096, K=4096, N=14336, group=64, x_dtype="bf16"),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_half_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 to bf16 or fp16 (RNE, torch's cast); return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(tdt).view(torch.int16).numpy().view(np.uint16)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """int32 words whose eight 4-bit fields are independent uniform codes 0..15."""
    return rng.integers(0, 2**32, size=shape, dtype=np.uint32).view(np.int32)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    """uint8 bytes whose two 4-bit fields are independent uniform codes 0..15."""
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def uniform_f16(rng, shape, lo=0.005, hi=0.02) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32).astype(np.float16)


def w4a8_inputs(M: int, K: int, N: int, group: int, x_dtype: str = "bf16",
                seed: int = 0, outlier_frac: float = 0.0, outlier_mult: float = 20.0,
                with_bias: bool = False) -> dict:
    """Activations x [M,K], GPTQ qweight int32 [K/8, N], fp16 scales [G, N].

    G = K / group, or 1 for group -1 (one scale per output column).
    Outliers: round(outlier_frac*K) K-columns, chosen by a seeded permutation,
    are multiplied by outlier_mult for every token.
    """
    assert K % 8 == 0 and N % 8 == 0
    rng = _rng(seed)
    G = 1 if group == -1 else K // group
    x32 = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    cols = rng.permutation(K)[:n_out] if n_out else np.zeros(0, dtype=np.int64)
    if n_out:
        x32[:, cols] *= np.float32(outlier_mult)
    qweight = random_words(rng, (K // 8, N))
    scales = uniform_f16(rng, (G, N))
    bias = None
    if with_bias:
        bias = to_half_bits(rng.standard_normal(N, dtype=np.float32), x_dtype)
    return dict(M=M, K=K, N=N, group=group, x_dtype=x_dtype, seed=seed,
                x=to_half_bits(x32, x_dtype), qweight=qweight, scales=scales,
                bias=bias, outlier_cols=np.sort(cols))


def w4a16_inputs(M: int, K: int, N: int, group: int = 64, seed: int = 0,
                 zero_std: float = 0.01) -> dict:
    """x bf16 [M,K]; weight bytes uint8 [N, K/2] (two codes per byte, low
    nibble first); scale bf16 [N, K/group] U[0.005,0.02]; zero bf16 N(0, std)."""
    assert K % group == 0 and group % 2 == 0
    rng = _rng(seed)
    G = K // group
    x32 = rng.standard_normal((M, K), dtype=np.float32)
    w = random_bytes(rng, (N, K // 2))
    scale = rng.uniform(0.005, 0.02, size=(N, G)).astype(np.float32)
    zero = (rng.standard_normal((N, G), dtype=np.float32) * np.float32(zero_std))
    return dict(M=M, K=K, N=N, group=group, seed=seed,
                x=to_half_bits(x32, "bf16"), w=w,
                scale=to_half_bits(scale, "bf16"), zero=to_half_bits(zero, "bf16"))


def route_topk(T: int, E: int, topk: int, rng: np.random.Generator):
    """Each token picks `topk` distinct experts uniformly at random.

    Returns the routed rows sorted by expert (stable in token id) as
    row_token int32 [T*topk] and expert_offsets int32 [E+1] (prefix sums of
    the per-expert row counts)."""
    keys = rng.random((T, E))
    experts = np.argsort(keys, axis=1)[:, :topk]          # distinct, uniform subset
    tok = np.repeat(np.arange(T, dtype=np.int64), topk)
    exp = experts.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))                           # by expert, then token
    row_token = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_token, offsets


def moe_inputs(E: int, K: int, N: int, group: int, T: int, topk: int,
               seed: int = 0) -> dict:
    """Routed-expert inputs: x bf16 [T,K]; expert weights in the
    compressed-tensors layout int32 [E, N, K/8] (8 codes per word along K);
    fp16 scales [E, G, N]; routing (row_token, expert_offsets)."""
    assert K % group == 0
    rng = _rng(seed)
    G = K // group
    x32 = rng.standard_normal((T, K), dtype=np.float32)
    w = random_words(rng, (E, N, K // 8))
    scales = uniform_f16(rng, (E, G, N))
    row_token, offsets = route_topk(T, E, topk, rng)
    return dict(E=E, K=K, N=N, group=group, T=T, topk=topk, seed=seed,
                x=to_half_bits(x32, "bf16"), x_dtype="bf16", w=w, scales=scales,
                row_token=row_token, expert_offsets=offsets)


def named(name: str, **override) -> dict:
    """The workload of that name with its fixed seed (sizes may be overridden)."""
    shp = dict(SHAPES[name])
    shp.update(override)
    seed = SEEDS[name]
    if name in ("w4a8_tiny", "w4a8_up_proj"):
        return w4a8_inputs(shp["M"], shp["K"], shp["N"], shp["group"], shp["x_dtype"], seed)
    if name == "w4a8_down_proj":
        return w4a8_inputs(shp["M"], shp["K"], shp["N"], shp["group"], shp["x_dtype"], seed,
                           outlier_frac=0.01, outlier_mult=20.0)
    if name in ("w4a16_decode", "w4a16_prefill"):
        return w4a16_inputs(shp["M"], shp["K"], shp["N"], shp["group"], seed)
    if name == "w4afp8_moe":
        return moe_inputs(shp["E"], shp["K"], shp["N"], shp["group"], shp["T"], shp["topk"], seed)
    raise KeyError(name)

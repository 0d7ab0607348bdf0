"""Seeded synthetic inputs for the grouped NVFP4 cast.

This module only draws random numbers and lays them out: it holds none of the
quantisation arithmetic, and it is the one module that both the HIP path's
tests/benchmark and the CPU oracle's tests take their inputs from.

The pages measure on no public dataset or routing trace, so every workload is
synthetic: a packed bf16 (sum_M, K) buffer of MoE expert activations (or
gradients) whose rows are grouped by expert, each expert's row count a multiple
of 128 (the token dispatcher pads every group to a multiple of 128 rows, as the
grouped-experts converter page, "Design notes", requires).  numpy's PCG64
``default_rng(seed)`` draws everything in float32; values are rounded to bf16
with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROW_ALIGN = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 to bf16 (nearest, ties to even); returns uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # chunked to bound temporaries on the large workloads
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 26
    for i in range(0, flat_u.size, step):
        c = flat_u[i:i + step]
        flat_o[i:i + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def largest_remainder(weights: np.ndarray, units: int) -> np.ndarray:
    """Split ``units`` among the weights in proportion to them: floor shares,
    then one extra unit each to the largest fractional parts (ties to the lower
    index)."""
    w = np.asarray(weights, dtype=np.float64)
    q = w / w.sum() * units
    base = np.floor(q).astype(np.int64)
    left = units - int(base.sum())
    frac = q - base
    order = sorted(range(w.size), key=lambda i: (-frac[i], i))
    for i in order[:left]:
        base[i] += 1
    return base


def zipf_splits(rng: np.random.Generator, num_experts: int, sum_m: int,
                exponent: float = 1.1, zeros: int = 2) -> np.ndarray:
    """Zipf-skewed routing: rank weights r^-exponent over a seeded permutation
    of the experts, the ``zeros`` smallest set to zero, rounded to 128-row
    units by largest remainder."""
    perm = rng.permutation(num_experts)
    w = np.empty(num_experts, dtype=np.float64)
    w[perm] = np.arange(1, num_experts + 1, dtype=np.float64) ** (-exponent)
    if zeros:
        w[perm[num_experts - zeros:]] = 0.0
    return largest_remainder(w, sum_m // ROW_ALIGN) * ROW_ALIGN


@dataclass
class Workload:
    """One synthetic input: bf16 bits (sum_m, k), host splits, directions."""
    name: str
    x: np.ndarray            # uint16 bf16 bit patterns, (sum_m, k), C-contiguous
    splits: np.ndarray       # int64 rows per expert, multiples of 128
    rowwise: bool = True
    columnwise: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def sum_m(self) -> int:
        return int(self.x.shape[0])

    @property
    def k(self) -> int:
        return int(self.x.shape[1])

    @property
    def num_experts(self) -> int:
        return int(self.splits.size)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def tiny(seed: int = 1) -> Workload:
    """4 experts, K=256, sum_M=512, splits [128, 256, 0, 128], values N(0,1);
    both directions."""
    splits = np.array([128, 256, 0, 128], dtype=np.int64)
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_normal(rng, (512, 256)))
    return Workload("tiny_e4_k256_m512", x, splits, True, True, {"seed": seed})


def outliers(seed: int = 2) -> Workload:
    """8 experts, K=2048, sum_M=8192; splits lognormal(0, 0.5) weights rounded
    to 128-row units; values N(0,1) with 0.1% of entries scaled by 100;
    rowwise only."""
    rng = np.random.default_rng(seed)
    splits = largest_remainder(rng.lognormal(0.0, 0.5, 8), 8192 // ROW_ALIGN) * ROW_ALIGN
    v = _normal(rng, (8192, 2048))
    mask = rng.random((8192, 2048), dtype=np.float32) < np.float32(0.001)
    v[mask] *= np.float32(100.0)
    return Workload("outliers_e8_k2048_m8192_rowwise", f32_to_bf16_bits(v), splits, True, False,
                    {"seed": seed})


def deepseek_share(seed: int = 3, sum_m: int = 65536, k: int = 7168, num_experts: int = 32) -> Workload:
    """DeepSeek-V3-style one-GPU expert share: 32 experts, K=7168 (hidden),
    sum_M=65536, Zipf(1.1) routing in 128-row units with the 2 smallest
    experts empty; values N(0,1) times a per-row lognormal(0,1) scale; both
    directions."""
    rng = np.random.default_rng(seed)
    splits = zipf_splits(rng, num_experts, sum_m)
    v = _normal(rng, (sum_m, k))
    row_scale = np.exp(_normal(rng, (sum_m, 1)))
    v *= row_scale.astype(np.float32)
    return Workload(f"deepseek_share_e{num_experts}_k{k}_m{sum_m}", f32_to_bf16_bits(v), splits,
                    True, True, {"seed": seed})


def down_proj(seed: int = 4, sum_m: int = 131072, k: int = 2048, num_experts: int = 64) -> Workload:
    """Down-projection input: 64 experts, K=2048, sum_M=131072, uniform random
    128-aligned splits (multinomial over 128-row units); values SiLU(a)*b with
    a, b ~ N(0,1); both directions."""
    rng = np.random.default_rng(seed)
    units = rng.multinomial(sum_m // ROW_ALIGN, np.full(num_experts, 1.0 / num_experts))
    splits = units.astype(np.int64) * ROW_ALIGN
    a = _normal(rng, (sum_m, k))
    b = _normal(rng, (sum_m, k))
    # SiLU(a) = a * sigmoid(a), evaluated in float32 (input synthesis only)
    a = a / (np.float32(1.0) + np.exp(-a))
    a *= b
    del b
    return Workload(f"down_proj_e{num_experts}_k{k}_m{sum_m}", f32_to_bf16_bits(a), splits, True, True,
                    {"seed": seed})


def gradient_like(seed: int = 5, sum_m: int = 65536, k: int = 7168) -> np.ndarray:
    """Gradient-like values: Student-t(3) * 1e-3, as bf16 bits (sum_m, k)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_t(3.0, size=(sum_m, k)).astype(np.float32)
    v *= np.float32(1e-3)
    return f32_to_bf16_bits(v)


def replay_splits(i: int, num_experts: int = 32, sum_m: int = 65536) -> np.ndarray:
    """Routing for graph replay i: Zipf(1.1) as in the expert-share workload,
    from seed 5000 + i."""
    return zipf_splits(np.random.default_rng(5000 + i), num_experts, sum_m)


def graph_replay(seed: int = 5, sum_m: int = 65536, k: int = 7168, num_experts: int = 32) -> Workload:
    """Graph-safe replay workload: expert-share shapes, gradient-like values,
    routing replaced per replay (``replay_splits``)."""
    return Workload(f"graph_replay_e{num_experts}_k{k}_m{sum_m}", gradient_like(seed, sum_m, k),
                    replay_splits(0, num_experts, sum_m), True, True, {"seed": seed})


def random_case(seed: int, splits, k: int, dist: str = "normal") -> Workload:
    """Small seeded case for parity sweeps: arbitrary 128-aligned splits and
    any K that is a multiple of 16 (ragged against the kernels' tiles)."""
    rng = np.random.default_rng(seed)
    splits = np.asarray(splits, dtype=np.int64)
    sum_m = int(splits.sum())
    if dist == "normal":
        v = _normal(rng, (sum_m, k))
    elif dist == "outliers":
        v = _normal(rng, (sum_m, k))
        mask = rng.random((sum_m, k)) < 0.001
        v[mask] *= np.float32(100.0)
    elif dist == "rowscale":
        v = _normal(rng, (sum_m, k)) * np.exp(_normal(rng, (sum_m, 1)))
    elif dist == "student":
        v = rng.standard_t(3.0, size=(sum_m, k)).astype(np.float32) * np.float32(1e-3)
    elif dist == "sparse":
        v = _normal(rng, (sum_m, k))
        v[rng.random((sum_m, k)) < 0.9] = 0.0
    else:
        raise ValueError(dist)
    return Workload(f"random_{dist}_s{seed}", f32_to_bf16_bits(np.asarray(v, np.float32)), splits,
                    True, True, {"seed": seed})


def _rowscaled_blocks(rng, sum_m: int, k: int, block_rows: int) -> np.ndarray:
    """N(0,1) x per-row exp(N(0,1)) as bf16 bits, drawn block_rows rows at a
    time (bounded host memory for very large buffers)."""
    x = np.empty((sum_m, k), dtype=np.uint16)
    for r0 in range(0, sum_m, block_rows):
        r1 = min(r0 + block_rows, sum_m)
        v = _normal(rng, (r1 - r0, k)) * np.exp(_normal(rng, (r1 - r0, 1)))
        x[r0:r1] = f32_to_bf16_bits(np.asarray(v, np.float32))
    return x


def max_rows(seed: int = 6, k: int = 16) -> Workload:
    """The row limit of the C ABI: sum_M = 2^24 rows, K = 16 (or k), two
    experts (one of 2^24 - 2^17 rows, one of 2^17)."""
    rng = np.random.default_rng(seed)
    sum_m = 1 << 24
    splits = np.array([sum_m - (1 << 17), 1 << 17], dtype=np.int64)
    return Workload(f"max_rows_e2_k{k}_m16777216", _rowscaled_blocks(rng, sum_m, k, 1 << 20), splits,
                    True, True, {"seed": seed})


def max_k(seed: int = 7) -> Workload:
    """The column limit of the C ABI: K = 2^22, one expert of 128 rows."""
    rng = np.random.default_rng(seed)
    sum_m, k = 128, 1 << 22
    return Workload("max_k_e1_k4194304_m128", _rowscaled_blocks(rng, sum_m, k, 16),
                    np.array([sum_m], dtype=np.int64), True, True, {"seed": seed})


def random_encoded(seed: int, nbytes_data: int):
    """Seeded NVFP4-encoded bytes for decode tests: nbytes_data code bytes
    (every byte value) and nbytes_data / 8 scale bytes (the codes a cast
    writes, 0x00 .. 0x7E).  Line amax values come from ``random_amax``."""
    rng = np.random.default_rng(seed)
    data = rng.integers(0, 256, nbytes_data, dtype=np.uint8)
    scale = rng.integers(0, 0x7F, nbytes_data // 8, dtype=np.uint8)
    return data, scale


def random_amax(seed: int, lines: int) -> np.ndarray:
    """Seeded positive line amax values spanning several binades."""
    rng = np.random.default_rng(seed)
    return np.exp2(rng.uniform(-8.0, 8.0, lines)).astype(np.float32)


def exact_nvfp4_lines(seed: int, lines: int, length: int):
    """Seeded encoded lines whose dot products are exact in fp32 for lengths
    up to 2^22: E2M1 codes of 0, +-0.5, +-1 (0, 1, 2, 9, 10), every block
    scale 1.0 (E4M3 0x38) and line amax 2688 (line factor 1), so every
    partial sum is a multiple of 0.25 of magnitude <= 2^22.  Returns
    (data [lines, length/2], scale [lines, length/16], amax [lines])."""
    rng = np.random.default_rng(seed)
    codes = np.array([0, 1, 2, 9, 10], dtype=np.uint8)
    data = np.empty((lines, length // 2), dtype=np.uint8)
    step = max(1, (1 << 24) // length)  # lines per draw
    for i0 in range(0, lines, step):
        i1 = min(i0 + step, lines)
        nib = codes[rng.integers(0, codes.size, (i1 - i0, length))]
        data[i0:i1] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    scale = np.full((lines, length // 16), 0x38, dtype=np.uint8)
    amax = np.full(lines, 2688.0, dtype=np.float32)
    return data, scale, amax


CONFIGS = {
    "tiny": tiny,
    "outliers": outliers,
    "deepseek_share": deepseek_share,
    "down_proj": down_proj,
    "graph_replay": graph_replay,
}

"""Seeded synthetic inputs for the block-scaled linear layer.

This module only draws random numbers and rounds them to the layer's input
dtypes (BF16 activations, FP32 weights); it holds none of the layer's own
arithmetic (no quantization, no GEMM).  Both the parity tests and the
benchmark take their inputs from here, so the two sides see identical bytes.

Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used counter-style: output i of
stream `seed` is mix(seed + (i + 1) * 0x9E3779B97F4A7C15).  Uniforms are the
top 53 bits; normals come from the Box-Muller transform; Student-t(nu=3) is
z0 / sqrt((z1^2 + z2^2 + z3^2) / 3).  Activations are drawn in FP64, rounded
to FP32 and then to BF16 with round-to-nearest-even; weights are rounded to
FP32.

Workload shapes follow the pages' attention output projection: weight
(7168, 8192) with 32-value scale groups ("Kimi-K3 DSpark O-Proj-only MXFP4",
section "Exact quantization coverage"); decode M = 64 (8 concurrent requests
x 8 draft positions, after the fixed-length performance setup in section
"Why O-proj only"); prefill M = 8192 (8 prompts x 1024 input tokens, same
setup).  The pages evaluate on public suites (GSM8K and others); those are
end-to-end model evaluations, and these synthetic tensors stand in only for
the shapes and value ranges the linear layer sees.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

# o_proj shape from the pages (out_features, in_features)
OPROJ_N, OPROJ_K = 7168, 8192


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream `seed` (uint64)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + i * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits."""
    return (splitmix64(seed, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, count: int, std: float = 1.0) -> np.ndarray:
    """`count` N(0, std^2) doubles; normal 2j, 2j+1 come from uniforms 2j, 2j+1."""
    out = np.empty(count, np.float64)
    pairs = (count + 1) // 2
    for p0 in range(0, pairs, _CHUNK):
        n = min(_CHUNK, pairs - p0)
        u = uniform(seed, 2 * p0, 2 * n).reshape(n, 2)
        r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))  # 1 - u in (0, 1]
        th = 2.0 * np.pi * u[:, 1]
        z = np.empty((n, 2), np.float64)
        z[:, 0] = r * np.cos(th)
        z[:, 1] = r * np.sin(th)
        z = z.reshape(-1)
        lo = 2 * p0
        hi = min(count, lo + 2 * n)
        out[lo:hi] = z[: hi - lo]
    return out * std


def student_t3(seed: int, count: int) -> np.ndarray:
    """`count` Student-t(nu=3) doubles, four normals per sample."""
    z = normal(seed, 4 * count).reshape(count, 4)
    return z[:, 0] / np.sqrt((z[:, 1] ** 2 + z[:, 2] ** 2 + z[:, 3] ** 2) / 3.0)


def fisher_yates_prefix(seed: int, n: int, k: int) -> np.ndarray:
    """First k entries of a Fisher-Yates shuffle of range(n) (sorted)."""
    perm = np.arange(n, dtype=np.int64)
    u = uniform(seed, 0, n)
    for i in range(n - 1, 0, -1):
        j = int(u[n - 1 - i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[n - k:])


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """FP64 -> FP32 (RNE) -> BF16 (RNE) bit patterns (uint16).  Finite input only."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------- workloads
def act_normal(seed: int, M: int, K: int) -> np.ndarray:
    """BF16 bits [M, K], N(0, 1)."""
    return f64_to_bf16_bits(normal(seed, M * K)).reshape(M, K)


def act_outlier_t3(seed: int, col_seed: int, M: int, K: int, frac: float = 0.01,
                   factor: float = 50.0) -> np.ndarray:
    """BF16 bits [M, K]: Student-t(3) with round(frac*K) fixed K-channels x factor
    (applied in FP64 before rounding).  Rows are a prefix of the same stream,
    so a smaller M is the first M rows of a larger draw."""
    x = student_t3(seed, M * K).reshape(M, K)
    cols = outlier_channels(col_seed, K, frac)
    x[:, cols] *= factor
    return f64_to_bf16_bits(x)


def outlier_channels(col_seed: int, K: int, frac: float = 0.01) -> np.ndarray:
    return fisher_yates_prefix(col_seed, K, int(round(frac * K)))


def weight_normal(seed: int, N: int, K: int, std: float) -> np.ndarray:
    """FP32 [N, K], N(0, std^2)."""
    return normal(seed, N * K, std).astype(np.float32).reshape(N, K)


# name -> recipe.  Seeds: tiny X 0 / W 1; decode and prefill share W seed 2;
# sweep W 5, X 6, outlier channels 7; ptpc W 8, X 9 (M=64) / 10 (M=8192).
CONFIGS = {
    "tiny_a4w4": dict(kind="a4w4", M=8, N=256, K=512, x=("normal", 0), w=("normal", 1, 0.02)),
    "oproj_decode_a4w4": dict(kind="a4w4", M=64, N=OPROJ_N, K=OPROJ_K, x=("normal", 3), w=("normal", 2, 0.01)),
    "oproj_prefill_a4w4": dict(kind="a4w4", M=8192, N=OPROJ_N, K=OPROJ_K, x=("normal", 4), w=("normal", 2, 0.01)),
    "msweep_outlier_a4w4": dict(kind="a4w4", M=2048, N=OPROJ_N, K=OPROJ_K, Ms=(1, 16, 128, 512, 2048),
                                x=("t3_outlier", 6, 7), w=("normal", 5, 0.02)),
    "ptpc_a8w8_m64": dict(kind="a8w8", M=64, N=OPROJ_N, K=OPROJ_K, x=("normal", 9), w=("normal", 8, 0.01)),
    "ptpc_a8w8_m8192": dict(kind="a8w8", M=8192, N=OPROJ_N, K=OPROJ_K, x=("normal", 10), w=("normal", 8, 0.01)),
    # grouped MoE decode (synthetic: the pages give no expert shapes): 64 tokens x top-8 routed over
    # 32 experts, each expert a [7168, 2048] MXFP4 projection (hidden 7168, intermediate 2048)
    "moe_grouped_a4w4": dict(kind="a4w4_grouped", tokens=64, topk=8, G=32, N=OPROJ_N, K=2048,
                             x=("normal", 11), w=("normal", 12, 0.02), route=13),
    # the same routing into each expert's up (or gate) projection: [2048, 7168], K = the hidden size
    "moe_grouped_up_a4w4": dict(kind="a4w4_grouped", tokens=64, topk=8, G=32, N=2048, K=OPROJ_N,
                                x=("normal", 14), w=("normal", 15, 0.02), route=13),
}


def route_counts(seed: int, tokens: int, topk: int, G: int) -> np.ndarray:
    """Rows per expert when each token picks topk distinct experts uniformly (seeded): the first
    topk entries of a Fisher-Yates shuffle of range(G), one shuffle per token."""
    counts = np.zeros(G, np.int64)
    for t in range(tokens):
        counts[fisher_yates_prefix(seed * 1_000_003 + t, G, topk)] += 1
    return counts


def make_activations(cfg: dict, M: int | None = None) -> np.ndarray:
    M = cfg["M"] if M is None else M
    kind = cfg["x"][0]
    if kind == "normal":
        return act_normal(cfg["x"][1], M, cfg["K"])
    if kind == "t3_outlier":
        return act_outlier_t3(cfg["x"][1], cfg["x"][2], M, cfg["K"])
    raise ValueError(kind)


def make_weight(cfg: dict, N: int | None = None) -> np.ndarray:
    """Rows are a prefix of the full-N draw, so N < cfg['N'] gives its first rows."""
    N = cfg["N"] if N is None else N
    _, seed, std = cfg["w"]
    return weight_normal(seed, N, cfg["K"], std)

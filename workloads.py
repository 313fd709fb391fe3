"""Seeded synthetic inputs for the ternary linear layer.

This module only *draws* inputs: bf16 activations, the per-input-channel sign
table, ternary codes and fp16 group scales.  It holds none of the layer's own
arithmetic (no rotation, no quantisation, no packing, no matmul), so the CPU
oracle and the HIP path can both consume what it returns without sharing any
of the method's code.

Shapes and distributions follow the layers the pages run (ternary 27B hybrid,
hidden 5120, intermediate 17408 = 17 x 1024, prefill steps of 256/512 tokens,
decode batches of up to 24 streams):
  * [P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2"
    (qiita.com/nakanokensetsu/items/ecc183fae033565af7cb), Prerequisites
    (2-bit {-1,0,+1} weights, one scale per 128 elements, block Hadamard on the
    input side, 48 GDN + 16 attention layers), section 1 (down_proj input width
    17408), section 4 (per-row/per-128-group fp16 scales; 256/512-token prefill
    budgets) and section 6 (2.6 MB bf16 all-reduce per 256 tokens, i.e. hidden
    size 5120).
  * [P3] "27B LLM for 24 concurrent users on two 12 GB GPUs"
    (qiita.com/nakanokensetsu/items/66e136acefd5a54b2f1d), appendix environment
    table (24 concurrent sequences).

The real weights, sign tables and prompts are not available, so every value
here is synthetic; the recipe (seeds, draw order, distributions) is fixed so
both sides see identical bytes.

Recipe (numpy PCG64, one Generator per layer, draws in this order):
  1. activations x [M, K] in fp32, then rounded to bf16 (round to nearest even
     on the bit pattern):
       "gauss_outlier": N(0,1), then round(0.02*K) distinct input channels
                        (shared by all tokens) multiplied by 20;
       "silu_gate":     SiLU(a) * b with a, b ~ N(0,1) drawn as two [M, K]
                        arrays (a first);
  2. sign [K]: uniform over {-1, +1} (int8);
  3. code [N, K]: "uniform" = i.i.d. uniform over {-1, 0, +1};
                  "sparse40" = P(0)=0.4, P(+1)=P(-1)=0.3;
  4. s [N, K/128]: exp(N(-4, 0.5)) rounded to fp16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

GROUP = 128          # elements per scale group along K
HBLOCK = 1024        # Hadamard block width along K


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits.

    Inputs are finite by construction (normal draws); NaN handling is not
    needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (a left shift by 16)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Layer:
    """One ternary linear layer's synthetic inputs (host numpy arrays)."""
    M: int
    K: int
    N: int
    x_bits: np.ndarray      # uint16 [M, K]  bf16 bit patterns
    sign: np.ndarray        # int8   [K]     +-1
    code: np.ndarray        # int8   [N, K]  {-1, 0, +1}
    s_bits: np.ndarray      # uint16 [N, K/128] fp16 bit patterns
    seed: int
    act: str
    codes: str

    @property
    def s(self) -> np.ndarray:
        return self.s_bits.view(np.float16)


def draw_activations(rng: np.random.Generator, M: int, K: int, act: str) -> np.ndarray:
    if act == "gauss_outlier":
        x = rng.standard_normal((M, K), dtype=np.float32)
        n_out = int(round(0.02 * K))
        ch = rng.choice(K, size=n_out, replace=False)
        x[:, ch] *= np.float32(20.0)
    elif act == "silu_gate":
        a = rng.standard_normal((M, K), dtype=np.float32)
        b = rng.standard_normal((M, K), dtype=np.float32)
        x = (a / (np.float32(1.0) + np.exp(-a))) * b
    else:
        raise ValueError(f"unknown activation recipe {act!r}")
    return f32_to_bf16_bits(x)


def make_gate_up(seed: int, M: int, K: int):
    """Raw input of the down projection's fused activation step: bf16 bit
    patterns [M, 2K] holding gate (columns 0..K-1) and up (K..2K-1), both
    N(0,1), and a sign table of width K.  No activation is applied here."""
    if K % HBLOCK:
        raise ValueError("K must be a multiple of 1024")
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, 2 * K), dtype=np.float32)
    return f32_to_bf16_bits(g), draw_sign(rng, K)


def draw_sign(rng: np.random.Generator, K: int) -> np.ndarray:
    return rng.choice(np.array([-1, 1], dtype=np.int8), size=K)


def draw_codes(rng: np.random.Generator, N: int, K: int, codes: str) -> np.ndarray:
    if codes == "uniform":
        return rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    if codes == "sparse40":
        return rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(N, K), p=[0.3, 0.4, 0.3])
    raise ValueError(f"unknown code recipe {codes!r}")


def draw_scales(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    s = np.exp(rng.normal(-4.0, 0.5, size=(N, K // GROUP))).astype(np.float16)
    return s.view(np.uint16)


def make_layer(seed: int, M: int, K: int, N: int, act: str = "gauss_outlier",
               codes: str = "uniform", sign: Optional[np.ndarray] = None) -> Layer:
    """Draw one layer.  If `sign` is given it is used instead of drawing one
    (one table per input width shared across layers); the draw is then skipped,
    which keeps the code/scale stream independent of whether it was given."""
    if K % HBLOCK:
        raise ValueError("K must be a multiple of 1024")
    rng = np.random.default_rng(seed)
    x_bits = draw_activations(rng, M, K, act)
    sg = draw_sign(rng, K) if sign is None else np.asarray(sign, dtype=np.int8)
    code = draw_codes(rng, N, K, codes)
    s_bits = draw_scales(rng, N, K)
    return Layer(M, K, N, x_bits, sg, code, s_bits, seed, act, codes)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

HIDDEN = 5120
INTER = 17408
N_LAYERS = 64
DECODE_MS = (1, 4, 8, 16, 24)

CONFIGS: Dict[str, dict] = {
    "tiny": dict(M=16, K=1024, N=256, act="gauss_outlier", codes="uniform", seed=0),
    "prefill_gate_up": dict(M=512, K=HIDDEN, N=INTER, act="gauss_outlier", codes="uniform", seed=1),
    "prefill_down": dict(M=256, K=INTER, N=HIDDEN, act="silu_gate", codes="sparse40", seed=2),
    # Decode sweep: activations drawn once at M=24; smaller M take leading rows.
    "decode_gate_up": dict(M=24, K=HIDDEN, N=INTER, act="gauss_outlier", codes="uniform", seed=3),
    "decode_down": dict(M=24, K=INTER, N=HIDDEN, act="silu_gate", codes="sparse40", seed=30),
}


def make_config(name: str) -> Layer:
    c = CONFIGS[name]
    return make_layer(c["seed"], c["M"], c["K"], c["N"], c["act"], c["codes"])


# 64-layer stack: per layer three linears (attention/GDN projection 5120->5120,
# fused gate+up 5120->34816, down 17408->5120), one sign table per input width.
STACK_LINEARS: List[Tuple[str, int, int, str, str]] = [
    ("proj", HIDDEN, HIDDEN, "gauss_outlier", "uniform"),
    ("gate_up", HIDDEN, 2 * INTER, "gauss_outlier", "uniform"),
    ("down", INTER, HIDDEN, "silu_gate", "sparse40"),
]
STACK_SIGN_SEED = 999


def stack_layer_seed(layer: int, which: int) -> int:
    """Seed of linear `which` (0..2) of decoder layer `layer` (0..63)."""
    return 1000 + 3 * layer + which


def stack_signs() -> Dict[int, np.ndarray]:
    rng = np.random.default_rng(STACK_SIGN_SEED)
    return {HIDDEN: draw_sign(rng, HIDDEN), INTER: draw_sign(rng, INTER)}


def stack_linear_torch(layer: int, which: int, M: int, device, torch_mod=None):
    """Draw one linear of the 64-layer stack directly on `device` with a seeded
    torch generator (the stack holds 18.8 G codes; drawing them with numpy on
    the host would dominate the run).  Same distributions as the numpy recipe,
    different bit stream.  Returns (x_bits int16 [M,K], code int8 [N,K],
    s_bits int16 [N,K/128]) as torch tensors on `device`.
    """
    import torch
    name, K, N, act, codes = STACK_LINEARS[which]
    g = torch.Generator(device=device)
    g.manual_seed(stack_layer_seed(layer, which))
    if act == "gauss_outlier":
        x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
        n_out = int(round(0.02 * K))
        ch = torch.randperm(K, generator=g, device=device)[:n_out]
        x[:, ch] *= 20.0
    else:
        a = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
        b = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
        x = torch.nn.functional.silu(a) * b
    x_bits = x.to(torch.bfloat16).view(torch.int16)
    u = torch.rand((N, K), generator=g, device=device, dtype=torch.float32)
    if codes == "uniform":
        code = (u * 3.0).floor().clamp_(0, 2).to(torch.int8) - 1
    else:
        code = (u >= 0.7).to(torch.int8) - (u < 0.3).to(torch.int8)
    s = torch.exp(torch.randn((N, K // GROUP), generator=g, device=device) * 0.5 - 4.0)
    s_bits = s.to(torch.float16).view(torch.int16)
    return x_bits, code.contiguous(), s_bits

"""CPU oracle for the ternary linear layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, step-by-step NumPy.  It exists to check the HIP library; only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it.  The
product path never calls it and it never calls the product path: the two share
no code.  Inputs come from the seeded generator in ``workloads.py`` (which holds
none of this arithmetic).

Sources (cited by page and section; the pages are the text of three blog posts):
  [P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2"
       (qiita.com/nakanokensetsu/items/ecc183fae033565af7cb)
       - Prerequisites: weights are {-1,0,+1} as 2 bits plus one scale per 128
         elements; a block-wise Hadamard rotation sits on the input side.
       - Section 1 (TP=2 port, the Hadamard block split in the middle): the sign
         table of the rotation is keyed by the full input width; the Sylvester
         recursion H1024 [a; b] = [H512 a + H512 b ; H512 a - H512 b]; the
         kernel's final butterfly stage has exactly that sum/difference form.
       - Section 4 (what helped, prefill linear layers to an int8 GEMM): every
         row n and 128-group g has an fp16 scale s[n,g]; it is split into a row
         maximum smax[n] and an 8-bit ratio q[n,g] = round(127 s[n,g] / smax[n]);
         W_int8[n,k] = code[n,k] * q[n, k/128] fits int8 exactly; the prefill
         matmul becomes one int8 GEMM with int32 accumulation followed by a
         per-row and per-token rescale; activations are quantised to int8 per
         token after the rotation.

Readings taken where the pages are silent (each is listed in the design notes):
  R1 rotation is orthonormal: r = (1/32) H1024 (sign * x) per 1024-block;
  R2 the sign multiplies before H;  R3 butterfly stages run h = 1, 2, ..., 512
  (ascending; the last stage is the page's sum/difference of 512-halves), each
  as (lo, hi) -> (lo + hi, lo - hi) in fp32;  R4 the FWHT runs in fp32 on the
  exactly widened bf16 input;  R5 the activation scale is per token over the
  whole row;  R6 int8 range is symmetric +-127 with a_scale = absmax / 127 and
  x_i8 = rint(r / a_scale) (IEEE division, ties to even);  R7 "round" is ties to
  even;  R8 q is evaluated as rint(fl32(127 s) / smax) in fp32, smax = max_g |s|
  stored exactly as fp32;  R9 an all-zero token gives a_scale = 0, x_i8 = 0, an
  all-zero scale row gives smax = 0, q = 0;  R10 2-bit encoding u = 0 for -1,
  1 for +1, 2 for 0 (3 unused), sixteen codes per little-endian 32-bit word,
  code k = 16w + 4i + b in bits [8b + 2i, 8b + 2i + 1] of word w; a row's 32
  bytes of each 128-group are stored in 2 KB tiles of 64 rows x one group,
  tile (r, g) at byte (r * K/128 + g) * 2048, row 64r + j at 32 j inside it,
  rows past N padded with code 0;  R11 the
  epilogue y = acc * a_scale[t] * smax[n] / 127 is evaluated in float64 and
  rounded to fp32 once;  R12 the optional bf16 output is that fp32 y rounded
  to the nearest bf16 value, ties to even (the pages' consumers take bf16
  activations, [P1] section 4; they do not say how y is narrowed);  R13 the
  down projection's input is SiLU(gate) * up of the gate/up projection's
  output [M, 2K] (gate = columns 0..K-1), rounded to bf16 as an unfused
  pipeline would hand it over (the pages name the 27B model's 17408-wide
  intermediate layer, [P1] section 1, not its activation; SiLU-gated MLPs are
  the reading);  R14 SiLU is evaluated in fp32 as s = g / (1 + e) with
  e = exp(-g) from a fixed sequence of fp32 operations (argument clamped to
  [-87, 88], Cody-Waite reduction by ln 2 split in two, degree-7 Taylor
  polynomial in Horner form, exact scaling by 2^n), so that two
  implementations of the method agree bit for bit;  R15 the bf16 reference
  path ([P1] section 4's pre-int8 path) uses the rotated activation rounded to
  bf16 and the weights code * bf16(s) (the fp16 scale rounded to bf16), with
  fp32 accumulation on the GPU; the oracle sums the exact products in
  float64, and the GPU is held to the fp32 accumulation bound
  K * 2^-24 * sum_k |r W| per output.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
HBLOCK = 1024
INV_NORM = np.float32(1.0 / 32.0)      # 1/sqrt(1024), a power of two (R1)
QMAX = 127


# ---------------------------------------------------------------------------
# Rotation: sign, block FWHT, per-token int8 quantisation  ([P1] Prereq, s.1, s.4)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32, exact (the 16 bits become the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def fwht_f32(v: np.ndarray, n: int = HBLOCK) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform in Sylvester (natural) order over
    consecutive blocks of width n along the last axis, fp32 throughout.

    Stage h (h = 1, 2, 4, ..., n/2, ascending -- R3) pairs positions j and j+h
    for every j with j mod 2h < h and replaces them by (v[j] + v[j+h],
    v[j] - v[j+h]).  With this order the last stage combines the two n/2-halves
    by sum and difference, which is the recursion printed in [P1] section 1.
    """
    v = np.array(v, dtype=np.float32, copy=True)
    if v.shape[-1] % n:
        raise ValueError("last axis must be a multiple of the block width")
    lead = v.shape[:-1]
    nb = v.shape[-1] // n
    h = 1
    while h < n:
        w = v.reshape(lead + (nb, n // (2 * h), 2, h))
        lo = w[..., 0, :].copy()
        hi = w[..., 1, :].copy()
        w[..., 0, :] = lo + hi          # fp32 add, one rounding
        w[..., 1, :] = lo - hi          # fp32 subtract, one rounding
        v = w.reshape(lead + (nb * n,))
        h *= 2
    return v


def rotate(x_bits: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """r = (1/32) H1024 (sign * x) per token and 1024-block, fp32 (R1, R2, R4).
    The sign table is indexed by the full input channel (one table per width,
    [P1] section 1)."""
    x = bf16_to_f32(x_bits)
    if x.shape[-1] % HBLOCK:
        raise ValueError("K must be a multiple of 1024")
    v = x * np.asarray(sign, dtype=np.float32)      # exact: multiply by +-1
    return fwht_f32(v, HBLOCK) * INV_NORM             # exact: power of two


def quantise_per_token(r: np.ndarray):
    """Per-token symmetric int8 quantisation of the rotated activations
    ([P1] section 4; R5, R6, R7, R9).  Returns (x_i8 int8 [M,K], a_scale fp32 [M])."""
    r = np.asarray(r, dtype=np.float32)
    absmax = np.max(np.abs(r), axis=-1)                               # fp32, exact
    a_scale = (absmax / np.float32(QMAX)).astype(np.float32)          # IEEE division
    safe = np.where(a_scale > 0, a_scale, np.float32(1.0)).astype(np.float32)
    ratio = (r / safe[:, None]).astype(np.float32)                     # IEEE division
    x_i8 = np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)       # ties to even
    x_i8[a_scale == 0] = 0
    return x_i8, a_scale


def rotate_quant_act(x_bits: np.ndarray, sign: np.ndarray):
    """bf16 x [M,K] and sign [K] -> (x_i8 [M,K], a_scale [M])."""
    return quantise_per_token(rotate(x_bits, sign))


# ---------------------------------------------------------------------------
# Weight side: scale decomposition and 2-bit packing  ([P1] Prereq, s.4)
# ---------------------------------------------------------------------------

def decompose_scales(s_bits: np.ndarray):
    """fp16 scales s [N, G] -> (q int8 [N, G], smax fp32 [N]).

    smax[n] = max_g |s[n,g]| (R8), q[n,g] = round(127 s[n,g] / smax[n]) with the
    product 127*s exact in fp32 (11-bit significand times 7 bits) and one
    correctly rounded fp32 division, then ties-to-even rounding (R7, R8, R9).
    """
    s = np.asarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    smax = np.max(np.abs(s), axis=-1).astype(np.float32)
    num = (np.float32(QMAX) * s).astype(np.float32)
    den = np.where(smax > 0, smax, np.float32(1.0)).astype(np.float32)
    q = np.rint((num / den[:, None]).astype(np.float32))
    q[smax == 0] = 0
    return q.astype(np.int8), smax


# R10: the 2-bit field value of each code, and its inverse
CODE_TO_FIELD = {-1: 0, 1: 1, 0: 2}
FIELD_TO_CODE = {v: k for k, v in CODE_TO_FIELD.items()}


ROW_BLOCK = 64                        # rows per weight tile (R10)
PAD_BYTE = 0xAA                       # four fields of value 2: code 0 (R10)


def packed_bytes(N: int, K: int) -> int:
    """Size of the tiled packed buffer: ceil(N/64) row blocks of 64 rows x K/4 bytes."""
    return -(-N // ROW_BLOCK) * ROW_BLOCK * K // 4


def pack_rows(code: np.ndarray) -> np.ndarray:
    """{-1,0,+1} codes [N, K] -> one packed row per weight row, [N, K/4] bytes:
    row n is K/16 little-endian 32-bit words and code k = 16w + 4i + b sits in
    bits [8b + 2i, 8b + 2i + 1] of word w, field value CODE_TO_FIELD (R10)."""
    code = np.asarray(code)
    N, K = code.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if np.any((code < -1) | (code > 1)):
        raise ValueError("codes must be in {-1, 0, +1}")
    c = code.astype(np.int64)
    u = np.zeros_like(c)
    for cv, fv in CODE_TO_FIELD.items():
        u[c == cv] = fv
    u = u.reshape(N, K // 16, 4, 4)                                 # [n, w, i, b]
    words = np.zeros((N, K // 16), dtype=np.uint64)
    for i in range(4):
        for b in range(4):
            words |= (u[:, :, i, b].astype(np.uint64) << np.uint64(8 * b + 2 * i))
    return words.astype("<u4").view(np.uint8).reshape(N, K // 4)


def tile_rows(rows: np.ndarray) -> np.ndarray:
    """Packed rows [N, K/4] -> the tiled buffer [ceil(N/64), K/128, 64, 32] (R10):
    tile (r, g) holds the 32 bytes of group g (k = 128g .. 128g + 127) of rows
    64r .. 64r + 63, one row after another; rows past N are code-0 padding."""
    rows = np.asarray(rows, dtype=np.uint8)
    N, KB = rows.shape
    NB, G = -(-N // ROW_BLOCK), KB // 32
    full = np.full((NB * ROW_BLOCK, KB), PAD_BYTE, dtype=np.uint8)
    full[:N] = rows
    return np.ascontiguousarray(full.reshape(NB, ROW_BLOCK, G, 32).transpose(0, 2, 1, 3))


def untile_rows(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of tile_rows (test helper): tiled buffer (any shape with the
    right byte count) -> packed rows [N, K/4]."""
    G = K // GROUP
    t = np.asarray(packed, dtype=np.uint8).reshape(-1, G, ROW_BLOCK, 32)
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3).reshape(-1, K // 4)[:N])


def pack_codes(code: np.ndarray) -> np.ndarray:
    """{-1,0,+1} codes [N, K] -> the tiled packed buffer [ceil(N/64), K/128, 64, 32]."""
    return tile_rows(pack_rows(code))


def unpack_rows(rows: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_rows (test helper): packed rows [N, K/4] -> int8 codes [N, K]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    N = rows.shape[0]
    words = rows.view("<u4").reshape(N, K // 16).astype(np.uint64)
    u = np.zeros((N, K // 16, 4, 4), dtype=np.int64)
    for i in range(4):
        for b in range(4):
            u[:, :, i, b] = ((words >> np.uint64(8 * b + 2 * i)) & np.uint64(3)).astype(np.int64)
    u = u.reshape(N, K)
    if np.any(u == 3):
        raise ValueError("field value 3 does not encode a code")
    code = np.zeros((N, K), dtype=np.int8)
    for fv, cv in FIELD_TO_CODE.items():
        code[u == fv] = cv
    return code


def unpack_codes(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of pack_codes (test helper): tiled buffer -> int8 codes [N, K]."""
    return unpack_rows(untile_rows(packed, N, K), K)


def pack_ternary(code: np.ndarray, s_bits: np.ndarray):
    """(code [N,K], s fp16 [N,K/128]) -> (packed tiled u8 [ceil(N/64), K/128, 64, 32],
    q int8 [N,K/128], smax fp32 [N])."""
    q, smax = decompose_scales(s_bits)
    return pack_codes(code), q, smax


# ---------------------------------------------------------------------------
# The int8 GEMM and its rescale  ([P1] section 4)
# ---------------------------------------------------------------------------

def weight_int8(code: np.ndarray, q: np.ndarray) -> np.ndarray:
    """W_int8[n,k] = code[n,k] * q[n, k // 128]; |W_int8| <= 127 so it is int8."""
    code = np.asarray(code, dtype=np.int16)
    N, K = code.shape
    qe = np.repeat(np.asarray(q, dtype=np.int16), GROUP, axis=1)
    return (code * qe).astype(np.int8)


def linear_acc(x_i8: np.ndarray, code: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc[t,n] = sum_k x_i8[t,k] * W_int8[n,k], exact, int32.

    Evaluated as a float64 matrix product of integer-valued matrices: every
    product and every partial sum is an integer of magnitude <= 127*127*K
    < 2^53 for the supported K, so the library product is exact whatever its
    summation order.
    """
    w = weight_int8(code, q).astype(np.float64)
    a = np.asarray(x_i8, dtype=np.float64)
    acc = a @ w.T
    return acc.astype(np.int64).astype(np.int32)


def linear_acc_at(x_i8: np.ndarray, code: np.ndarray, q: np.ndarray,
                  rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """acc at the sampled (rows[i], cols[i]) pairs, one int64 dot product each."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(rows.shape[0], dtype=np.int64)
    for i, (t, n) in enumerate(zip(rows, cols)):
        w = weight_int8(code[n:n + 1], q[n:n + 1])[0].astype(np.int64)
        out[i] = int(np.dot(np.asarray(x_i8[t], dtype=np.int64), w))
    return out.astype(np.int32)


def epilogue(acc: np.ndarray, a_scale: np.ndarray, smax: np.ndarray) -> np.ndarray:
    """y[t,n] = acc[t,n] * a_scale[t] * smax[n] / 127 in float64, rounded once (R11)."""
    acc = np.asarray(acc, dtype=np.float64)
    y = acc * np.asarray(a_scale, dtype=np.float64)[:, None] * np.asarray(smax, dtype=np.float64)[None, :] / 127.0
    return y.astype(np.float32)


def epilogue_at(acc_s: np.ndarray, a_scale: np.ndarray, smax: np.ndarray, rows, cols) -> np.ndarray:
    acc_s = np.asarray(acc_s, dtype=np.float64)
    y = acc_s * np.asarray(a_scale, dtype=np.float64)[rows] * np.asarray(smax, dtype=np.float64)[cols] / 127.0
    return y.astype(np.float32)


def ternary_linear(x_i8, a_scale, code, q, smax):
    """Full prefill/decode linear: int32 acc then the per-token/per-row rescale."""
    return epilogue(linear_acc(x_i8, code, q), a_scale, smax)


# ---------------------------------------------------------------------------
# SiLU(gate) * up feeding the down projection (R13, R14)
# ---------------------------------------------------------------------------

EXP_LO, EXP_HI = np.float32(-87.0), np.float32(88.0)
LOG2E = np.float32(1.4426950408889634)
LN2_HI = np.float32(0.693145751953125)          # 15 significant bits: n * LN2_HI is exact
LN2_LO = np.float32(0.6931471805599453 - 0.693145751953125)
EXP_TAYLOR = [np.float32(1.0 / np.prod(np.arange(1, k + 1, dtype=np.float64))) for k in range(8)]


def exp_f32(x: np.ndarray) -> np.ndarray:
    """exp in fp32 by the fixed operation sequence of R14: x = clamp(x),
    n = rint(x log2 e), r = (x - n ln2_hi) - n ln2_lo, p = sum_k r^k / k!
    (k <= 7, Horner), exp = p * 2^n."""
    x = np.clip(np.asarray(x, dtype=np.float32), EXP_LO, EXP_HI)
    n = np.rint(x * LOG2E)
    r = (x - n * LN2_HI) - n * LN2_LO
    p = EXP_TAYLOR[7] * np.ones_like(r)
    for k in range(6, -1, -1):
        p = p * r + EXP_TAYLOR[k]
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def silu_mul_bf16(gate_up_bits: np.ndarray) -> np.ndarray:
    """bf16 [M, 2K] (gate | up) -> bf16 bits [M, K] of SiLU(gate) * up (R13, R14)."""
    K = gate_up_bits.shape[1] // 2
    g = bf16_to_f32(gate_up_bits[:, :K])
    u = bf16_to_f32(gate_up_bits[:, K:])
    s = g / (np.float32(1.0) + exp_f32(-g))
    return round_bf16(s * u)


def silu_mul_rotate_quant_act(gate_up_bits: np.ndarray, sign: np.ndarray):
    """The down projection's input step: SiLU(gate) * up, then rotate_quant_act."""
    return rotate_quant_act(silu_mul_bf16(gate_up_bits), sign)


# ---------------------------------------------------------------------------
# bf16 reference path ([P1] section 4's pre-int8 path; R15)
# ---------------------------------------------------------------------------

def rotate_bf16(x_bits: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """The rotation of rotate_quant_act, r rounded to bf16 bits [M, K]."""
    return round_bf16(rotate(x_bits, sign))


def dequant_bf16(code: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """W[n,k] = code[n,k] * bf16(s[n, k/128]) as float64 [N, K] (exact values)."""
    s32 = s_bits.view(np.float16).astype(np.float32)
    sb = bf16_to_f32(round_bf16(s32)).astype(np.float64)
    return np.asarray(code, dtype=np.float64) * np.repeat(sb, GROUP, axis=1)


def reference_linear_bf16(r_bits: np.ndarray, code: np.ndarray, s_bits: np.ndarray):
    """y = r . W^T with the exact products summed in float64; returns (y as
    float64, sum_k |r W| as float64) -- the second is the scale of the GPU's
    fp32 accumulation bound (R15)."""
    r = bf16_to_f32(r_bits).astype(np.float64)
    w = dequant_bf16(code, s_bits)
    return r @ w.T, np.abs(r) @ np.abs(w).T


def round_bf16(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), nearest value, ties to even (R12).

    Written from the definition: the two bf16 neighbours of y (its fp32 bits
    truncated to the top 16, and the next bf16 value away from zero) are
    compared in float64, and on a tie the one with an even last bit wins.
    Finite inputs only."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = y.view(np.uint32)
    lo_bits = u & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)
    y64 = y.astype(np.float64)
    d_lo = np.abs(y64 - lo_bits.view(np.float32).astype(np.float64))
    d_hi = np.abs(hi_bits.view(np.float32).astype(np.float64) - y64)
    lo_odd = ((lo_bits >> 16) & 1) == 1
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)
    return np.where(take_hi, hi_bits >> 16, lo_bits >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Unquantised reference for the sanity error figure ([P1] section 4 reports a
# per-layer relative error of 9.5e-3 for the int8 path)
# ---------------------------------------------------------------------------

def rotate_f64(x_bits: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """Exact (float64) orthonormal block rotation, for the reference only."""
    x = bf16_to_f32(x_bits).astype(np.float64) * np.asarray(sign, dtype=np.float64)
    lead = x.shape[:-1]
    nb = x.shape[-1] // HBLOCK
    v = x.reshape(lead + (nb, HBLOCK)).copy()
    h = 1
    while h < HBLOCK:
        w = v.reshape(lead + (nb, HBLOCK // (2 * h), 2, h))
        lo = w[..., 0, :].copy()
        hi = w[..., 1, :].copy()
        w[..., 0, :] = lo + hi
        w[..., 1, :] = lo - hi
        h *= 2
    return v.reshape(lead + (nb * HBLOCK,)) / 32.0


def float_reference(x_bits, sign, code, s_bits) -> np.ndarray:
    """y_ref = r . (code * s)^T in float64 with the unquantised rotated activation
    r and the unrounded fp16 scales (weights live in the rotated basis)."""
    r = rotate_f64(x_bits, sign)
    s = np.asarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    w = np.asarray(code, dtype=np.float64) * np.repeat(s, GROUP, axis=1)
    return r @ w.T


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))

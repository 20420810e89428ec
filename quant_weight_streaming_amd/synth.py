"""Seeded synthetic inputs for the K-quant decode GEMV.

This module only draws random fields and writes them into GGUF K-quant
super-block bytes (an encoding); it computes no dequantised weight and no
dot product, so the CPU oracle and the GPU path can both consume what it
produces without sharing any of the method's arithmetic.

Formats (public GGUF K-quant layout, the plain reading of "GGUF K-quant" on
the daily.dev summary page, Q&A "How does ExecuTorch export Muse Glimmer GGUF
checkpoints ..."; the byte layout itself is not printed on the pages):

* Q4_K, 144 B per 256 weights: fp16 d, fp16 dmin, 12 B of packed 6-bit
  (scale, min) pairs for 8 sub-blocks of 32, 128 B of 4-bit quants.
* Q5_K, 176 B: Q4_K plus 32 B of fifth bits (bit g of byte i is the high
  bit of element 32*g + i).
* Q6_K, 210 B: 128 B low nibbles, 64 B of 2-bit high parts, 16 int8
  sub-block scales (sub-blocks of 16), fp16 d.

Value distributions follow the five workload descriptions this library is
measured on: d, dmin = fp16(|N(0,1)| * 1e-2); 6-bit scale and min uniform in
[0, 63]; quants uniform over their full range; Q6_K scale uniform in
[-64, 63]; activations N(0,1) rounded to bf16 (or kept fp32).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence

import torch

QK = 256                       # weights per super-block
SB_BYTES = {"q4k": 144, "q5k": 176, "q6k": 210}
TYPES = ("q4k", "q5k", "q6k")


def seed_of(*parts) -> int:
    """Deterministic 63-bit seed from a tuple of labels (config, layer, tensor, field)."""
    h = hashlib.sha256(repr(tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _rand_bytes(n: int, g, device) -> torch.Tensor:
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g, device=device)


def _fp16_abs_normal(n: int, scale: float, g, device) -> torch.Tensor:
    """fp16 bit patterns of fp16_RNE(|N(0,1)| * scale), as int16 tensor."""
    v = torch.randn((n,), generator=g, device=device, dtype=torch.float32).abs_() * scale
    return v.to(torch.float16).view(torch.int16)


def _u16_to_bytes(v: torch.Tensor) -> torch.Tensor:
    """[n] 16-bit tensor -> [n, 2] little-endian bytes."""
    return v.contiguous().view(torch.uint8).view(-1, 2)


# --------------------------------------------------------------------------
# field-level encoders (used for hand-built blocks and for the merged-group
# workload); all arguments are integer tensors with a leading super-block axis
# --------------------------------------------------------------------------

def encode_scales_q4k(sc: torch.Tensor, m: torch.Tensor) -> torch.Tensor:
    """Pack 8 six-bit scales and 8 six-bit mins per super-block into 12 bytes.

    For j = 0..3: byte j holds sc[j] in bits 0-5 and bits 4-5 of sc[j+4] in
    bits 6-7; byte 4+j holds m[j] likewise with m[j+4]; byte 8+j holds the low
    four bits of sc[j+4] and of m[j+4] in its low and high nibble.
    """
    sc = sc.to(torch.int32)
    m = m.to(torch.int32)
    out = torch.empty(sc.shape[0], 12, dtype=torch.int32, device=sc.device)
    out[:, 0:4] = (sc[:, 0:4] & 63) | ((sc[:, 4:8] >> 4) << 6)
    out[:, 4:8] = (m[:, 0:4] & 63) | ((m[:, 4:8] >> 4) << 6)
    out[:, 8:12] = (sc[:, 4:8] & 15) | ((m[:, 4:8] & 15) << 4)
    return out.to(torch.uint8)


def encode_qs_nibbles(q4: torch.Tensor) -> torch.Tensor:
    """Low nibbles of 256 quants -> 128 bytes (element 64c+i low, 64c+32+i high of byte 32c+i)."""
    q4 = q4.to(torch.int32) & 15
    n = q4.shape[0]
    q = q4.view(n, 4, 2, 32)                    # [sb, c, half, i]
    return (q[:, :, 0, :] | (q[:, :, 1, :] << 4)).reshape(n, 128).to(torch.uint8)


def encode_q5_high(q: torch.Tensor) -> torch.Tensor:
    """Fifth bits of 256 quants -> 32 bytes: bit g of byte i = bit 4 of element 32g+i."""
    h = (q.to(torch.int32) >> 4) & 1
    n = h.shape[0]
    h = h.view(n, 8, 32)                        # [sb, g, i]
    out = torch.zeros(n, 32, dtype=torch.int32, device=q.device)
    for g in range(8):
        out |= h[:, g, :] << g
    return out.to(torch.uint8)


def pack_q4k(d: torch.Tensor, dmin: torch.Tensor, sc: torch.Tensor, m: torch.Tensor,
             q: torch.Tensor) -> torch.Tensor:
    """Fields -> Q4_K bytes [n_sb, 144]. d, dmin: fp16 bit patterns (int16/int32)."""
    n = q.shape[0]
    out = torch.empty(n, 144, dtype=torch.uint8, device=q.device)
    out[:, 0:2] = _u16_to_bytes(d.to(torch.int32).to(torch.int16))
    out[:, 2:4] = _u16_to_bytes(dmin.to(torch.int32).to(torch.int16))
    out[:, 4:16] = encode_scales_q4k(sc, m)
    out[:, 16:144] = encode_qs_nibbles(q)
    return out


def pack_q5k(d, dmin, sc, m, q) -> torch.Tensor:
    """Fields -> Q5_K bytes [n_sb, 176]; q in [0, 31]."""
    n = q.shape[0]
    out = torch.empty(n, 176, dtype=torch.uint8, device=q.device)
    out[:, 0:2] = _u16_to_bytes(d.to(torch.int32).to(torch.int16))
    out[:, 2:4] = _u16_to_bytes(dmin.to(torch.int32).to(torch.int16))
    out[:, 4:16] = encode_scales_q4k(sc, m)
    out[:, 16:48] = encode_q5_high(q)
    out[:, 48:176] = encode_qs_nibbles(q)
    return out


def pack_q6k(d: torch.Tensor, sc: torch.Tensor, q: torch.Tensor) -> torch.Tensor:
    """Fields -> Q6_K bytes [n_sb, 210]; sc int8 values [n_sb, 16], q in [0, 63].

    Element e = 128h + 32r + i keeps its low nibble in byte 64h + 32(r&1) + i
    (low nibble for r < 2, high nibble otherwise) and its top two bits in
    bits 2r..2r+1 of byte 128 + 32h + i.
    """
    q = q.to(torch.int32)
    n = q.shape[0]
    out = torch.empty(n, 210, dtype=torch.uint8, device=q.device)
    qv = q.view(n, 2, 4, 32)                    # [sb, h, r, i]
    lo = qv & 15
    ql = torch.empty(n, 2, 2, 32, dtype=torch.int32, device=q.device)  # [sb, h, r&1, i]
    ql[:, :, 0, :] = lo[:, :, 0, :] | (lo[:, :, 2, :] << 4)
    ql[:, :, 1, :] = lo[:, :, 1, :] | (lo[:, :, 3, :] << 4)
    out[:, 0:128] = ql.reshape(n, 128).to(torch.uint8)
    hi = (qv >> 4) & 3
    qh = hi[:, :, 0, :] | (hi[:, :, 1, :] << 2) | (hi[:, :, 2, :] << 4) | (hi[:, :, 3, :] << 6)
    out[:, 128:192] = qh.reshape(n, 64).to(torch.uint8)
    out[:, 192:208] = (sc.to(torch.int32) & 0xFF).to(torch.uint8)
    out[:, 208:210] = _u16_to_bytes(d.to(torch.int32).to(torch.int16))
    return out


# --------------------------------------------------------------------------
# random tensors
# --------------------------------------------------------------------------

def gen_weights(qtype: str, rows: int, cols: int, seed: int, device="cpu",
                merge_frac: float = 0.0) -> torch.Tensor:
    """Random GGUF bytes for a rows x cols matrix, super-blocks in row-major order.

    Returns uint8 [rows, cols/256 * SB_BYTES[qtype]].  Quant bits are uniform
    random bytes (so every quant is uniform over its range); scales and mins
    are drawn as fields and encoded.  With merge_frac > 0 (Q4_K and Q5_K), each
    super-block is selected with that probability and then every aligned
    sub-block pair (2k, 2k+1) gets identical scale and min.
    """
    if cols % QK:
        raise ValueError("cols must be a multiple of 256")
    nsb = rows * (cols // QK)
    g = _gen(seed, device)
    if qtype in ("q4k", "q5k"):
        sbb = SB_BYTES[qtype]
        out = torch.empty(nsb, sbb, dtype=torch.uint8, device=device)
        out[:, 0:2] = _u16_to_bytes(_fp16_abs_normal(nsb, 1e-2, g, device))
        out[:, 2:4] = _u16_to_bytes(_fp16_abs_normal(nsb, 1e-2, g, device))
        sc = torch.randint(0, 64, (nsb, 8), generator=g, device=device, dtype=torch.int32)
        m = torch.randint(0, 64, (nsb, 8), generator=g, device=device, dtype=torch.int32)
        if merge_frac > 0:
            sel = torch.rand((nsb,), generator=g, device=device) < merge_frac
            sel = sel[:, None]
            sc[:, 1::2] = torch.where(sel, sc[:, 0::2], sc[:, 1::2])
            m[:, 1::2] = torch.where(sel, m[:, 0::2], m[:, 1::2])
        out[:, 4:16] = encode_scales_q4k(sc, m)
        out[:, 16:] = _rand_bytes(nsb * (sbb - 16), g, device).view(nsb, sbb - 16)
        return out.view(rows, -1)
    if qtype == "q6k":
        out = torch.empty(nsb, 210, dtype=torch.uint8, device=device)
        out[:, 0:192] = _rand_bytes(nsb * 192, g, device).view(nsb, 192)
        sc = torch.randint(-64, 64, (nsb, 16), generator=g, device=device, dtype=torch.int32)
        out[:, 192:208] = (sc & 0xFF).to(torch.uint8)
        out[:, 208:210] = _u16_to_bytes(_fp16_abs_normal(nsb, 1e-2, g, device))
        return out.view(rows, -1)
    raise ValueError(f"unknown type {qtype}")


def gen_x(batch: int, cols: int, seed: int, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """Activations [batch, cols] ~ N(0,1); bf16 (RNE) or fp32."""
    g = _gen(seed, device)
    x = torch.randn((batch, cols), generator=g, device=device, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# the five measured workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Gemv:
    name: str
    qtype: str
    rows: int
    cols: int
    parts: Sequence[int] = ()       # row split for the multi-projection call (empty = one matrix)
    types: Sequence[str] = ()       # per-part weight types of a mixed-type projection (empty = qtype for all)

    def part_types(self):
        n = len(self.parts) or 1
        return list(self.types) if self.types else [self.qtype] * n

    def weight_bytes(self) -> int:
        parts = list(self.parts) or [self.rows]
        return sum(r * self.cols // QK * SB_BYTES[t] for r, t in zip(parts, self.part_types()))


HIDDEN, INTER, VOCAB = 5120, 31232, 131072
N_LAYERS = 52
QKV = Gemv("qkv", "q4k", 4608, HIDDEN, (4096, 256, 256))     # 32 q heads + 2 kv heads, head_dim 128
O_PROJ = Gemv("o", "q4k", HIDDEN, 4096)
GATE_UP = Gemv("gate_up", "q4k", 2 * INTER, HIDDEN, (INTER, INTER))
DOWN = Gemv("down", "q6k", HIDDEN, INTER)
HEAD = Gemv("head", "q6k", VOCAB, HIDDEN)


def sweep(gate_up_type: str = "q4k"):
    """The 52-layer decode-step weight sweep plus the head, in launch order."""
    gu = dataclasses.replace(GATE_UP, qtype=gate_up_type)
    out = []
    for layer in range(N_LAYERS):
        out += [(layer, QKV), (layer, O_PROJ), (layer, gu), (layer, DOWN)]
    out.append((N_LAYERS, HEAD))
    return out


def sweep_bytes(gate_up_type: str = "q4k") -> int:
    return sum(g.rows * g.cols // QK * SB_BYTES[g.qtype] for _, g in sweep(gate_up_type))


# A mixed-type build in the manner of the GGUF "Q4_K_M" recipe (the SGLang Day-0 post's GGUF checkpoints,
# "Q4KM"; the daily.dev summary's "k-quant" build): most tensors Q4_K, the attention V rows and half of
# the down projections kept at Q6_K.  The exact per-tensor recipe is not on the pages; this reading puts V
# at Q6_K in every layer (so every QKV projection mixes two types in one launch) and down at Q6_K in the
# even layers and Q4_K in the odd ones.
QKV_Q4KM = Gemv("qkv", "q4k", 4608, HIDDEN, (4096, 256, 256), ("q4k", "q4k", "q6k"))
DOWN_Q4K = Gemv("down", "q4k", HIDDEN, INTER)


def sweep_q4km():
    """The 52-layer sweep with the Q4_K_M-style type mix, in launch order."""
    out = []
    for layer in range(N_LAYERS):
        out += [(layer, QKV_Q4KM), (layer, O_PROJ), (layer, GATE_UP), (layer, DOWN if layer % 2 == 0 else DOWN_Q4K)]
    out.append((N_LAYERS, HEAD))
    return out


def sweep_q4km_bytes() -> int:
    return sum(g.weight_bytes() for _, g in sweep_q4km())


# The text decoder described on the "Muse-Glimmer-30B (text decoder) - Apple Core AI" card, section
# "The architecture, and what the port had to do about it": 52 layers, hidden 6656, 32 q / 2 kv heads of
# 128, a sigmoid output gate read from the same hidden state as Q/K/V (so one fused qkvg projection of
# 4096 + 256 + 256 + 4096 rows), SwiGLU intermediate 19968, an untied 202048-row head.  The type mix is
# the one above (Q4_K projections, Q6_K down and head).
HIDDEN_P4, INTER_P4, VOCAB_P4 = 6656, 19968, 202048
QKVG_P4 = Gemv("qkvg", "q4k", 8704, HIDDEN_P4, (4096, 256, 256, 4096))
O_P4 = Gemv("o", "q4k", HIDDEN_P4, 4096)
GATE_UP_P4 = Gemv("gate_up", "q4k", 2 * INTER_P4, HIDDEN_P4, (INTER_P4, INTER_P4))
DOWN_P4 = Gemv("down", "q6k", HIDDEN_P4, INTER_P4)
HEAD_P4 = Gemv("head", "q6k", VOCAB_P4, HIDDEN_P4)


def sweep_p4():
    """The same decode-step sweep for the 6656-hidden decoder."""
    out = []
    for layer in range(N_LAYERS):
        out += [(layer, QKVG_P4), (layer, O_P4), (layer, GATE_UP_P4), (layer, DOWN_P4)]
    out.append((N_LAYERS, HEAD_P4))
    return out


def sweep_p4_bytes() -> int:
    return sum(g.rows * g.cols // QK * SB_BYTES[g.qtype] for _, g in sweep_p4())


CONFIGS = {
    0: dict(name="q4k_256x1024_b1_f32", gemv=Gemv("c0", "q4k", 256, 1024), batch=(1,), xdtype="f32"),
    1: dict(name="q4k_gate_up_62464x5120_b1", gemv=GATE_UP, batch=(1,), xdtype="bf16"),
    2: dict(name="q6k_head_131072x5120_b1", gemv=HEAD, batch=(1,), xdtype="bf16"),
    3: dict(name="sweep52_q4k_q6k_b1", sweep="q4k", batch=(1, 8), xdtype="bf16"),
    4: dict(name="sweep52_q5k_gate_up_merged_b2_4_8", sweep="q5k", batch=(2, 4, 8), xdtype="bf16",
            merge_frac=0.25),
}

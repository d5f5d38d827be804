"""Seeded synthetic workloads for the sparse MQA attention step.

This module is shared by the CPU oracle and the HIP path and therefore holds no
arithmetic of the method itself: only the shapes of the five workloads, the
derived sizes both sides need (row counts, top-k length, window length), and the
seeded random draws that fill the inputs.

Shapes and value distributions follow the DeepSeek V4.1 model page
("Attention" class, "Indexer" class and the model config JSON): 64 query heads
of dim 512 sharing one KV row per position (used as key and value), a
128-slot sliding window, 32 index heads of dim 128, index_topk 512.  The five
base workloads use compress ratio 4; the `_r2` and `_r1` workloads use the
ratios the page's config gives its layers (2 on layers 2-19, 1 on layers
20-39), at the same shapes.

Draw order per workload: q, kv_win, kv_comp, qI, kI, w, sink.  Values are
N(0,1) in fp32, rounded to bf16 (round-to-nearest-even) for bf16 workloads;
w is N(0,1)/2; sink is N(0,1) fp32.  For the fp4 workload the compressed rows
are drawn as N(0,1) and encoded by `encode_fp4_e2m1_e4m3` below (the
generator's own encoder; decoding is each side's business).
"""
from __future__ import annotations

import dataclasses
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "generate",
    "encode_fp4_e2m1_e4m3",
    "encode_mxfp4_e8m0",
    "rope_freqs",
    "scaled",
    "nbytes",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str  # "prefill" (start_pos == 0, S tokens) or "decode" (S == 1)
    B: int
    S: int
    start_pos: int
    H: int
    D: int
    rope_dim: int
    W: int
    ratio: int
    H_I: int
    D_I: int
    index_topk: int
    dtype: str  # "f32" or "bf16": q, kv, index q/k, head weights, output
    comp_fmt: str = "same"  # "same" (as dtype) or "fp4" (e2m1 + E4M3 scale per 16)
    index_fmt: str = "same"  # "same" (as dtype) or "mxfp4" (index q/k as e2m1 + E8M0 scale per 32)

    # ---- derived sizes (no arithmetic of the method, only bookkeeping) ----
    @property
    def end_pos(self) -> int:
        return self.start_pos + self.S

    @property
    def T(self) -> int:
        """Compressed rows that exist after this call (end_pos // ratio)."""
        return self.end_pos // self.ratio

    @property
    def K(self) -> int:
        """Top-k row length: min(index_topk, T)."""
        return min(self.index_topk, self.T)

    @property
    def n_win(self) -> int:
        """Window-KV rows: the chunk's own S rows in prefill, the W-slot ring in decode."""
        return self.S if self.start_pos == 0 else self.W

    @property
    def Wc(self) -> int:
        """Window columns of an index row."""
        return min(self.S, self.W) if self.start_pos == 0 else self.W

    @property
    def L(self) -> int:
        """Index row length: window columns followed by the top-k columns."""
        return self.Wc + self.K

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def check(self) -> None:
        if self.mode == "decode":
            assert self.S == 1 and self.start_pos > 0, self
        else:
            assert self.start_pos == 0, self
        if self.comp_fmt == "fp4":
            assert self.dtype == "bf16" and self.D % 16 == 0
        if self.index_fmt == "mxfp4":
            assert self.dtype == "bf16" and self.D_I % 32 == 0


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_prefill_f32", "prefill", B=1, S=64, start_pos=0, H=4, D=64, rope_dim=16,
                 W=16, ratio=4, H_I=4, D_I=32, index_topk=8, dtype="f32"),
        Workload("decode_b32_ctx8k", "decode", B=32, S=1, start_pos=8191, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("prefill_s8k", "prefill", B=1, S=8192, start_pos=0, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("decode_b16_ctx64k", "decode", B=16, S=1, start_pos=65535, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("prefill_s32k_fp4", "prefill", B=1, S=32768, start_pos=0, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16", comp_fmt="fp4"),
        # the page config's own ratios: 2 on layers 2-19, 1 on layers 20-39 (compress_ratios)
        Workload("decode_b16_ctx64k_r2", "decode", B=16, S=1, start_pos=65535, H=64, D=512, rope_dim=64,
                 W=128, ratio=2, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("decode_b16_ctx64k_r1", "decode", B=16, S=1, start_pos=65535, H=64, D=512, rope_dim=64,
                 W=128, ratio=1, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("prefill_s8k_r2", "prefill", B=1, S=8192, start_pos=0, H=64, D=512, rope_dim=64,
                 W=128, ratio=2, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        Workload("prefill_s8k_r1", "prefill", B=1, S=8192, start_pos=0, H=64, D=512, rope_dim=64,
                 W=128, ratio=1, H_I=32, D_I=128, index_topk=512, dtype="bf16"),
        # the indexer in the precision the pages give it: index queries and keys fp4 with E8M0 scales
        # per 32 elements (the same shapes as the bf16-indexer workloads)
        Workload("decode_b32_ctx8k_mxfp4", "decode", B=32, S=1, start_pos=8191, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16", index_fmt="mxfp4"),
        Workload("decode_b16_ctx64k_mxfp4", "decode", B=16, S=1, start_pos=65535, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16", index_fmt="mxfp4"),
        Workload("decode_b16_ctx64k_r1_mxfp4", "decode", B=16, S=1, start_pos=65535, H=64, D=512, rope_dim=64,
                 W=128, ratio=1, H_I=32, D_I=128, index_topk=512, dtype="bf16", index_fmt="mxfp4"),
        Workload("prefill_s8k_mxfp4", "prefill", B=1, S=8192, start_pos=0, H=64, D=512, rope_dim=64,
                 W=128, ratio=4, H_I=32, D_I=128, index_topk=512, dtype="bf16", index_fmt="mxfp4"),
    ]
}
# the order in which the workloads are listed for the method (tiny case first)
ORDER = list(WORKLOADS)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some sizes changed (smaller parity cases)."""
    out = dataclasses.replace(w, **changes)
    out.check()
    return out


# ---------------------------------------------------------------- draws
_CHUNK = 1 << 26  # elements per draw call: bounds the fp32 staging buffer


def _randn(shape, gen: torch.Generator, device, out_dtype) -> torch.Tensor:
    """N(0,1) fp32 draws in fixed-size chunks along dim 0, cast to out_dtype (RNE)."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=out_dtype, device=device)
    if out.numel() == 0:
        return out
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(out_dtype)
    return out


# e2m1 magnitudes by code 0..7 (OCP Microscaling Formats spec, FP4 E2M1)
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def encode_fp4_e2m1_e4m3(x: torch.Tensor, group: int = 16):
    """Encode rows [..., D] as packed e2m1 nibbles plus one E4M3 scale per `group`.

    This is the generator's encoder (the pages name the format but not the
    quantiser): scale = E4M3 round-to-nearest-even of amax/6 over each group
    (0 when the group is all zero); each element is x/scale rounded to the
    nearest e2m1 value, ties to the even code, saturating at 6.  Byte k of a
    row holds element 2k in its low nibble and element 2k+1 in its high
    nibble; the nibble's bit 3 is the sign.

    Returns (packed uint8 [..., D/2], scales uint8 [..., D/group]).
    """
    assert x.shape[-1] % group == 0
    xs = x.float().reshape(*x.shape[:-1], x.shape[-1] // group, group)
    amax = xs.abs().amax(dim=-1)
    s8 = (amax / 6.0).to(torch.float8_e4m3fn)
    sf = s8.to(torch.float32)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    y = torch.where(sf.unsqueeze(-1) > 0, xs / safe.unsqueeze(-1), torch.zeros_like(xs))
    m = y.abs()
    code = torch.zeros_like(m, dtype=torch.int32)
    for i in range(7):
        mid = 0.5 * (_E2M1_GRID[i] + _E2M1_GRID[i + 1])
        take_upper_on_tie = (i + 1) % 2 == 0
        code += (m > mid).int()
        if take_upper_on_tie:
            code += (m == mid).int()
    code = code.clamp(max=7) | torch.where(y < 0, 8, 0).int()
    code = code.reshape(*x.shape[:-1], x.shape[-1]).to(torch.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), s8.view(torch.uint8).reshape(*x.shape[:-1], x.shape[-1] // group).contiguous()


def encode_mxfp4_e8m0(x: torch.Tensor, block: int = 32):
    """Encode rows [..., D] as packed e2m1 nibbles plus one E8M0 scale per `block`.

    The generator's encoder for the indexer's fp4 (the pages name the format,
    fp4 with E8M0 scales per 32, but not the quantiser): the scale is the
    smallest power of two 2**e with amax / 2**e <= 6 (so nothing clips; e is
    clamped to [-127, 127], and an all-zero block takes e = -127); each element
    is x / 2**e rounded to the nearest e2m1 value, ties to the even code.  Byte
    k of a row holds element 2k in its low nibble; the scale byte is e + 127.

    Returns (packed uint8 [..., D/2], scales uint8 [..., D/block]).
    """
    assert x.shape[-1] % block == 0
    xs = x.float().reshape(*x.shape[:-1], x.shape[-1] // block, block)
    amax = xs.abs().amax(dim=-1)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    e = torch.ceil(torch.log2(safe / 6.0))
    # log2 can land a hair off an exact power of two: step e until 6 * 2**e is the first bound >= amax
    e = torch.where(6.0 * torch.exp2(e - 1) >= safe, e - 1, e)
    e = torch.where(6.0 * torch.exp2(e) < safe, e + 1, e)
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127, 127)
    y = xs / torch.exp2(e).unsqueeze(-1)
    m = y.abs()
    code = torch.zeros_like(m, dtype=torch.int32)
    for i in range(7):
        mid = 0.5 * (_E2M1_GRID[i] + _E2M1_GRID[i + 1])
        code += (m > mid).int()
        if (i + 1) % 2 == 0:
            code += (m == mid).int()
    code = code.clamp(max=7) | torch.where(y < 0, 8, 0).int()
    code = code.reshape(*x.shape[:-1], x.shape[-1]).to(torch.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    scales = (e + 127).to(torch.uint8).reshape(*x.shape[:-1], x.shape[-1] // block)
    return packed.contiguous(), scales.contiguous()


def rope_freqs(positions, rope_dim: int, theta: float = 160000.0, device="cpu") -> torch.Tensor:
    """A rotary table float32 [n, rope_dim/2, 2] of (cos, sin) for the given positions.

    The pages build theirs with `precompute_freqs_cis` (YaRN; body not shown) from the config's
    compress_rope_theta = 160000; this generator uses the plain angles position * theta**(-2i/rope_dim).
    The table is an input of the epilogue and cache-write kernels, so parity does not depend on it.
    """
    pos = torch.as_tensor(positions, dtype=torch.float64, device=device)
    inv = theta ** (-torch.arange(0, rope_dim, 2, dtype=torch.float64, device=device) / rope_dim)
    ang = pos[:, None] * inv[None, :]
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32).contiguous()


def generate(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Seeded inputs of a workload, all on `device`.

    Keys: q [B,S,H,D], kv_win [B,n_win,D], kv_comp [B,T,D] (or, for the fp4
    workload, kv_comp_fp4 [B,T,D/2] uint8 and kv_comp_scale [B,T,D/16] uint8),
    qI [B,S,H_I,D_I], kI [B,T,D_I] (or, for the MXFP4 indexer, qI_fp4
    [B,S,H_I,D_I/2], qI_scale [B,S,H_I,D_I/32], kI_fp4 [B,T,D_I/2], kI_scale
    [B,T,D_I/32], all uint8), w [B,S,H_I], sink [H] fp32.
    The draws are made on `device` with its own generator, so CPU and GPU
    draws of one seed differ; each is deterministic.
    """
    w.check()
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = w.torch_dtype
    out = {}
    out["q"] = _randn((w.B, w.S, w.H, w.D), gen, dev, dt)
    out["kv_win"] = _randn((w.B, w.n_win, w.D), gen, dev, dt)
    if w.comp_fmt == "fp4":
        raw = _randn((w.B, w.T, w.D), gen, dev, torch.float32)
        out["kv_comp_fp4"], out["kv_comp_scale"] = encode_fp4_e2m1_e4m3(raw, 16)
        del raw
    else:
        out["kv_comp"] = _randn((w.B, w.T, w.D), gen, dev, dt)
    if w.index_fmt == "mxfp4":
        raw = _randn((w.B, w.S, w.H_I, w.D_I), gen, dev, torch.float32)
        out["qI_fp4"], out["qI_scale"] = encode_mxfp4_e8m0(raw, 32)
        raw = _randn((w.B, w.T, w.D_I), gen, dev, torch.float32)
        out["kI_fp4"], out["kI_scale"] = encode_mxfp4_e8m0(raw, 32)
        del raw
    else:
        out["qI"] = _randn((w.B, w.S, w.H_I, w.D_I), gen, dev, dt)
        out["kI"] = _randn((w.B, w.T, w.D_I), gen, dev, dt)
    out["w"] = (_randn((w.B, w.S, w.H_I), gen, dev, torch.float32) * 0.5).to(dt)
    out["sink"] = _randn((w.H,), gen, dev, torch.float32)
    return out


def nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()

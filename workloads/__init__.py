"""Seeded synthetic workloads for the hybrid Muon + AdamW optimizer step.

This module is shared by the oracle-side tests and by the GPU side. It holds
*data only*: parameter tables (names, shapes, storage dtypes, roles, views),
hyper-parameter constants, a bf16 storage codec and seeded random generators.
It contains none of the optimizer's arithmetic, so that neither side can
borrow the other's implementation through it.

Inputs are drawn with numpy's PCG64 seeded from
``SeedSequence([config_seed, step, tensor_index])``; step 0 draws the initial
weights and steps 1, 2, ... draw the gradients of that step.  Every draw is
made in fp32 and rounded to the storage dtype with round-to-nearest-even, and
the same bytes are handed to both implementations.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# bf16 storage codec (a storage format, not part of the method)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits.

    NaN maps to a quiet NaN; infinities and overflow to +-inf follow IEEE RNE.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32)
    # finite values stay below 0xff800000 + 0x8000, so 32-bit sums cannot wrap
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out.reshape(a.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bits (uint16) to fp32 exactly."""
    u = np.ascontiguousarray(np.asarray(b, dtype=np.uint16)).astype(np.uint32) << 16
    return u.view(np.float32)


def to_storage(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> storage array: float32 for 'f32', uint16 bf16 bits for 'bf16'."""
    if dtype == "f32":
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x_f32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact float32 values."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Hyper-parameter constants (values stated on the pages; see the docstrings)
# ---------------------------------------------------------------------------

#: Muon momentum coefficient (OMN "dual-manifold" page, Muon-path paragraph;
#: NorMuon paper eq. (1); Qwen3.8 optimizer notes section 2).
MUON_MU = 0.95
#: Peak learning rates of the OMN-1 recipe (OMN page, learning-rate paragraph).
MUON_LR = 0.01
ADAMW_LR = 3e-4
#: AdamW betas / eps / clip (OMN page, recipe summary paragraph).
ADAMW_BETA1 = 0.90
ADAMW_BETA2 = 0.95
ADAMW_EPS = 1e-8
CLIP_MAX_NORM = 1.0
#: NorMuon second-moment decay and epsilon used by the NorMuon workload.
NORMUON_BETA2 = 0.95
NORMUON_EPS = 1e-8

#: Cubic Newton-Schulz coefficients (a, b, c): X <- 1.5 X - 0.5 (X X^T) X
#: (MuonClip page, "Newton-Schulz Orthogonalization").
CUBIC = (1.5, -0.5, 0.0)
#: Second-order Newton-Schulz polar iteration: the binomial series of
#: (X^T X)^(-1/2) truncated after the quadratic term (Bjorck & Bowie 1971).
#: Fits the (a, b, c) form of the NorMuon paper's eq. (5).
QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


def coeff_table(kind: str, steps: int = 5) -> np.ndarray:
    """[steps, 3] float64 table of per-iteration (a, b, c)."""
    base = {"cubic": CUBIC, "quintic": QUINTIC}[kind]
    return np.tile(np.asarray(base, dtype=np.float64), (steps, 1))


# ---------------------------------------------------------------------------
# Parameter tables
# ---------------------------------------------------------------------------

ROLE_MATRIX = "matrix"      # hidden projection matrix
ROLE_EMBEDDING = "embedding"  # vocabulary embedding (tied to the head)
ROLE_HEAD = "head"          # explicit output classifier
ROLE_NORM = "norm"          # normalisation gain


@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]
    dtype: str                      # storage dtype of W and G: "f32" | "bf16"
    role: str = ROLE_MATRIX
    view: Optional[Tuple[int, ...]] = None
    split: Optional[Tuple[int, ...]] = None
    requires_grad: bool = True
    no_decay: bool = False          # explicit no-decay membership
    exclude: Optional[Tuple[int, ...]] = None   # split positions stepped by AdamW

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n


@dataclass(frozen=True)
class Workload:
    key: str
    seed: int
    params: Tuple[ParamSpec, ...]
    steps: int = 1
    grad_std: float = 1e-3
    init_std: float = 0.02
    coeffs: str = "cubic"
    ns_steps: int = 5
    normuon: bool = False
    description: str = ""
    extra: dict = field(default_factory=dict)

    def by_name(self, name: str) -> ParamSpec:
        for p in self.params:
            if p.name == name:
                return p
        raise KeyError(name)

    def index(self, name: str) -> int:
        for i, p in enumerate(self.params):
            if p.name == name:
                return i
        raise KeyError(name)


def _norm(name: str, n: int, dtype: str) -> ParamSpec:
    return ParamSpec(name, (n,), dtype, ROLE_NORM, no_decay=True)


def tiny_routing() -> Workload:
    """Tiny routing check: the pages' three view examples plus two AdamW params.

    Shapes from the kimi-k3 parameter-groups page ("The layout declarations
    are literal"): gate_up (32,8) viewed (2,16,8); KDA QKV (24,8) viewed
    (3,2,4,8); MLA W_UKV (20,8) viewed (2,10,8) with split (4,6).
    """
    f = "f32"
    params = (
        ParamSpec("embed_tokens.weight", (64, 8), f, ROLE_EMBEDDING, no_decay=True),
        ParamSpec("mlp.gate_up_proj.weight", (32, 8), f, view=(2, 16, 8)),
        ParamSpec("attn.QKV.weight", (24, 8), f, view=(3, 2, 4, 8)),
        ParamSpec("attn.W_UKV.weight", (20, 8), f, view=(2, 10, 8), split=(4, 6)),
        _norm("norm.weight", 8, f),
    )
    return Workload("tiny_routing_fp32", 1, params, steps=3, grad_std=1.0,
                    description="tiny routing check, fp32, 3 steps")


def fused_exclude(dtype: str = "bf16", heads: int = 4) -> Workload:
    """Mixed routing inside fused weights (Qwen3.8 optimizer notes, section 4):
    a gated-delta-net input projection fused per head as q, k, v and two
    one-row gate vectors, with the gate pieces excluded to AdamW; a fused
    gate/up projection split in halves; an embedding and a norm gain."""
    dk, dv, c = 64, 128, 256
    params = (
        ParamSpec("embed_tokens.weight", (512, c), dtype, ROLE_EMBEDDING, no_decay=True),
        ParamSpec("gdn.in_proj.weight", (heads * (2 * dk + dv + 2), c), dtype,
                  view=(heads, 2 * dk + dv + 2, c), split=(dk, dk, dv, 1, 1), exclude=(3, 4)),
        ParamSpec("mlp.gate_up_proj.weight", (1024, c), dtype, view=(2, 512, c)),
        _norm("norm.weight", c, dtype),
    )
    return Workload(f"fused_exclude_{dtype}", 6, params, steps=3, grad_std=1e-2,
                    description="fused weights with excluded gate pieces, 3 steps")


def ns_sweep(rows: int, cols: int, coeffs: str) -> Workload:
    """Single-matrix Newton-Schulz sweep item (bf16 momentum matrix)."""
    p = (ParamSpec(f"w{rows}x{cols}", (rows, cols), "bf16"),)
    return Workload(f"ns_sweep_{rows}x{cols}_{coeffs}", 2, p, steps=1,
                    grad_std=1e-3, coeffs=coeffs,
                    description=f"single {rows}x{cols} bf16 matrix, {coeffs}")


DENSE_D = 2048
DENSE_LAYERS = 24
DENSE_FFN = 5632
DENSE_VOCAB = 128256


def dense_decoder(fused_gate_up: bool = False, normuon: bool = False,
                  layers: int = DENSE_LAYERS) -> Workload:
    """Dense decoder parameter set: d=2048, 24 layers, SwiGLU FFN I=5632.

    Muon: Q, K, V, O (2048x2048), gate/up (5632x2048), down (2048x5632) per
    layer.  AdamW: tied embedding (128256x2048) and 2 * layers + 1 RMSNorm
    gains.  With ``fused_gate_up`` gate and up are stored as one
    (11264, 2048) weight viewed (2, 5632, 2048).
    """
    d, ffn, b = DENSE_D, DENSE_FFN, "bf16"
    ps = [ParamSpec("embed_tokens.weight", (DENSE_VOCAB, d), b, ROLE_EMBEDDING,
                    no_decay=True)]
    for i in range(layers):
        pre = f"layers.{i}."
        ps.append(_norm(pre + "input_norm.weight", d, b))
        for nm in ("q_proj", "k_proj", "v_proj", "o_proj"):
            ps.append(ParamSpec(pre + f"attn.{nm}.weight", (d, d), b))
        ps.append(_norm(pre + "post_attn_norm.weight", d, b))
        if fused_gate_up:
            ps.append(ParamSpec(pre + "mlp.gate_up_proj.weight", (2 * ffn, d), b,
                                view=(2, ffn, d)))
        else:
            ps.append(ParamSpec(pre + "mlp.gate_proj.weight", (ffn, d), b))
            ps.append(ParamSpec(pre + "mlp.up_proj.weight", (ffn, d), b))
        ps.append(ParamSpec(pre + "mlp.down_proj.weight", (d, ffn), b))
    ps.append(_norm("final_norm.weight", d, b))
    key = "dense_decoder_1p2b" + ("_fused_normuon" if normuon else "")
    if layers != DENSE_LAYERS:
        key += f"_{layers}l"
    return Workload(key, 4 if normuon else 3, tuple(ps), steps=1, grad_std=1e-3,
                    normuon=normuon,
                    description=f"dense decoder d=2048 L={layers} I=5632"
                                + (" (fused gate_up, NorMuon)" if normuon else ""))


def head_batched(layers: int = 16) -> Workload:
    """Head-batched MLA/KDA views: H=32, R_q=1536, R_kv=512, d=4096.

    Per layer: W_UQ (32*192, 1536) viewed (32, 192, 1536); W_UKV
    (32*256, 512) viewed (32, 256, 512) split (128, 128); QKV (3*32*128, 4096)
    viewed (3, 32, 128, 4096).  Muon only.
    """
    b = "bf16"
    ps = []
    for i in range(layers):
        pre = f"layers.{i}.attn."
        ps.append(ParamSpec(pre + "W_UQ.weight", (32 * 192, 1536), b, view=(32, 192, 1536)))
        ps.append(ParamSpec(pre + "W_UKV.weight", (32 * 256, 512), b, view=(32, 256, 512),
                            split=(128, 128)))
        ps.append(ParamSpec(pre + "QKV.weight", (3 * 32 * 128, 4096), b,
                            view=(3, 32, 128, 4096)))
    key = "head_batched_mla_kda" + ("" if layers == 16 else f"_{layers}l")
    return Workload(key, 5, tuple(ps), steps=1, grad_std=1e-3,
                    description=f"head-batched MLA/KDA views, {layers} layers")


def omn1_shapes() -> Tuple[ParamSpec, ...]:
    """Shape-only descriptor set shaped like the OMN-1 model (no data).

    28 blocks; Q and O 2048x2048; K and V 512x2048; gate/up 5504x2048; down
    2048x5504; tied embedding 128256x2048; a shared input RMSNorm per block,
    per-head q/k norms of width 128 and a final norm (OMN page, routing and
    per-block paragraphs).
    """
    b = "bf16"
    ps = [ParamSpec("embed_tokens.weight", (128256, 2048), b, ROLE_EMBEDDING, no_decay=True)]
    for i in range(28):
        pre = f"blocks.{i}."
        ps.append(_norm(pre + "input_norm.weight", 2048, b))
        ps.append(ParamSpec(pre + "attn.q_proj.weight", (2048, 2048), b))
        ps.append(ParamSpec(pre + "attn.k_proj.weight", (512, 2048), b))
        ps.append(ParamSpec(pre + "attn.v_proj.weight", (512, 2048), b))
        ps.append(ParamSpec(pre + "attn.o_proj.weight", (2048, 2048), b))
        ps.append(_norm(pre + "attn.q_norm.weight", 128, b))
        ps.append(_norm(pre + "attn.k_norm.weight", 128, b))
        ps.append(ParamSpec(pre + "mlp.gate_proj.weight", (5504, 2048), b))
        ps.append(ParamSpec(pre + "mlp.up_proj.weight", (5504, 2048), b))
        ps.append(ParamSpec(pre + "mlp.down_proj.weight", (2048, 5504), b))
    ps.append(_norm("final_norm.weight", 2048, b))
    return tuple(ps)


def all_workloads() -> Tuple[Workload, ...]:
    return (
        tiny_routing(),
        ns_sweep(1024, 1024, "cubic"),
        ns_sweep(1024, 1024, "quintic"),
        ns_sweep(4096, 1024, "cubic"),
        ns_sweep(4096, 1024, "quintic"),
        dense_decoder(),
        dense_decoder(fused_gate_up=True, normuon=True),
        head_batched(),
    )


# ---------------------------------------------------------------------------
# Seeded generators
# ---------------------------------------------------------------------------


def rng(config_seed: int, step: int, tensor_index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(config_seed), int(step), int(tensor_index)])))


def draw_f32(config_seed: int, step: int, tensor_index: int, shape: Sequence[int],
             std: float) -> np.ndarray:
    g = rng(config_seed, step, tensor_index)
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def device_seed(config_seed: int, step: int, tensor_index: int) -> int:
    """64-bit seed of the on-device stream for (config, step, tensor)."""
    ss = np.random.SeedSequence([int(config_seed), int(step), int(tensor_index), 0xD5])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def draw_device(config_seed: int, step: int, tensor_index: int, shape: Sequence[int],
                std: float, dtype: str, device="cuda"):
    """Seeded draw made on the GPU with torch's Philox generator (full-size
    workloads, where host generation would take minutes).  Drawn in fp32,
    scaled, then rounded to the storage dtype by torch (round to nearest even).
    Read the tensor back to give the oracle exactly the same bytes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(config_seed, step, tensor_index))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x if dtype == "f32" else x.to(torch.bfloat16)


def init_weight(w: Workload, index: int) -> np.ndarray:
    """Initial weight of param ``index`` in its storage dtype (step 0 stream)."""
    p = w.params[index]
    return to_storage(draw_f32(w.seed, 0, index, p.shape, w.init_std), p.dtype)


def grad(w: Workload, index: int, step: int) -> np.ndarray:
    """Gradient of param ``index`` at optimizer step ``step`` >= 1 (storage dtype)."""
    if step < 1:
        raise ValueError("gradient steps start at 1")
    p = w.params[index]
    return to_storage(draw_f32(w.seed, step, index, p.shape, w.grad_std), p.dtype)


def spiked_grad(w: Workload, index: int, step: int, rank: int = 8,
                amplitude: float = 100.0) -> np.ndarray:
    """Gradient plus a seeded rank-``rank`` spike of ``amplitude`` x grad_std.

    Imitates ill-conditioned momentum (a few dominant singular directions).
    """
    p = w.params[index]
    if len(p.shape) != 2:
        raise ValueError("spike needs a 2-D parameter")
    base = draw_f32(w.seed, step, index, p.shape, w.grad_std)
    g = rng(w.seed, step, 10_000 + index)
    r, c = p.shape
    u = g.standard_normal((r, rank), dtype=np.float32)
    v = g.standard_normal((rank, c), dtype=np.float32)
    spike = (u @ v) * np.float32(amplitude * w.grad_std / np.sqrt(rank))
    return to_storage(base + spike, p.dtype)


def prescribed_spectrum(config_seed: int, index: int, rows: int, cols: int,
                        sigma_hi: float = 1.0, sigma_lo: float = 1e-4,
                        dtype: str = "bf16") -> np.ndarray:
    """Matrix U diag(sigma) V^T with orthonormal U, V from the QR factors of
    seeded Gaussians and sigma spaced geometrically from ``sigma_hi`` down to
    ``sigma_lo`` (condition number sigma_hi / sigma_lo), built in float64,
    rounded to fp32 and then to the storage dtype.  A stand-in for the badly
    conditioned momentum matrices the NorMuon paper describes."""
    g = rng(config_seed, 0, 20_000 + index)
    s = min(rows, cols)
    U, _ = np.linalg.qr(g.standard_normal((rows, s)))
    V, _ = np.linalg.qr(g.standard_normal((cols, s)))
    sig = np.geomspace(sigma_hi, sigma_lo, s)
    return to_storage(((U * sig) @ V.T).astype(np.float32), dtype)

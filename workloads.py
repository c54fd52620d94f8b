"""Seeded synthetic inputs for the DiG GLA token mixer and SREM step.

This module holds no arithmetic of the method itself: it only draws random tensors,
applies the input projections that produce the mixer's operands (plain matmuls that sit
outside the layer's hot path), and quantises them once to the I/O element type.  Both the
oracle (fp64) and the HIP library receive exactly the same quantised values.

Shapes follow the DiG model table (DiG study-group slides, Table 1: S = 12 layers,
D = 384, 6 heads; XL = 28 layers, D = 1152, 16 heads) at patch size 2, where a res-px image
gives a (res/16) x (res/16) token grid (Fig. 1 caption: 12 544 tokens at 1792 x 1792).
ImageNet latents and trained weights are not available; random values of the stated
distributions stand in for them:
  x ~ N(0, 1); every projection weight ~ N(0, 1/D); DWConv weights ~ N(0, 1/9);
  gate bias 0, Swish-branch bias 0, norm weight 1; upstream gradients ~ N(0, 1).
The gate logits come through a rank-16 factorisation z = (x W_a1) W_a2 + b_alpha.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROW, ROW_REV, COL, COL_REV = 0, 1, 2, 3
SCAN_NAMES = {ROW: "row", ROW_REV: "row_rev", COL: "col", COL_REV: "col_rev"}
# Layer-wise schedule of scan directions: flip the flattened sequence after every block,
# transpose the token matrix after every second block (period 4).
SCHEDULE = (ROW, ROW_REV, COL, COL_REV)


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    grid_h: int
    grid_w: int
    d_model: int
    heads: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str            # "f32" or "bf16": element type at the library boundary
    rank: int = 16
    tau: float = 16.0
    blocks: int = 1
    index: int = 0
    note: str = ""

    @property
    def seq_len(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def seed(self) -> int:
        return 1000 + self.index


CONFIGS = {
    "tiny_f32": Config("tiny_f32", 1, 8, 8, 64, 2, 16, 32, 16, "f32", index=0,
                       note="tiny GLA layer, fp32, all four scan directions + 3x3 DWConv"),
    "dig_s2_256": Config("dig_s2_256", 8, 16, 16, 384, 6, 32, 64, 64, "bf16", blocks=12, index=1,
                         note="DiG-S/2 at 256 px, 12 blocks cycling the four scan directions"),
    "dig_s2_1792": Config("dig_s2_1792", 1, 112, 112, 384, 6, 32, 64, 64, "bf16", index=2,
                          note="DiG-S/2 at 1792 px, GLA fwd + reorient + DWConv"),
    "dig_xl2_1024": Config("dig_xl2_1024", 2, 64, 64, 1152, 16, 36, 72, 64, "bf16", index=3,
                           note="DiG-XL/2 at 1024 px, forward across the four scan directions"),
    "dig_xl2_2048": Config("dig_xl2_2048", 1, 128, 128, 1152, 16, 36, 72, 64, "bf16", index=4,
                           note="DiG-XL/2 at 2048 px, forward + backward"),
}


def cfg_replace(cfg: Config, **kw) -> Config:
    d = {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}
    d.update(kw)
    return Config(**d)


# ----------------------------------------------------------------- quantisation
def f32_round(a) -> np.ndarray:
    """float64 values rounded to the nearest float32 (numpy's cast is round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(a) -> np.ndarray:
    """uint16 bfloat16 encodings of a (via float32), rounded to nearest, ties to even."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(a) -> np.ndarray:
    return bf16_to_f64(bf16_bits(a))


def quantize(a, dtype: str) -> np.ndarray:
    """Values of a as the boundary stores them, returned as float64."""
    if dtype == "bf16":
        return bf16_round(a)
    if dtype == "f32":
        return f32_round(a)
    raise ValueError(dtype)


def storage(a, dtype: str) -> np.ndarray:
    """Raw array to upload: uint16 bf16 encodings or float32."""
    if dtype == "bf16":
        return bf16_bits(a)
    return np.asarray(a, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------- cases
@dataclass
class GLACase:
    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray
    r: np.ndarray
    gamma: np.ndarray
    dy: np.ndarray
    x: np.ndarray = field(default=None)


def _normal(rng, shape, std):
    return rng.standard_normal(shape) * std


def make_gla_case(cfg: Config, seed: int | None = None, *, batch: int | None = None,
                  seq_len: int | None = None, gate_bias: float = 0.0,
                  z_std: float | None = None, random_gamma: bool = False,
                  r_bias: float = 0.0) -> GLACase:
    """Mixer operands for one block.

    q, k, v, r are projections of x ~ N(0,1) by weights ~ N(0, 1/D); z comes through the
    rank-16 factorisation plus ``gate_bias``.  ``z_std`` replaces z by N(gate_bias, z_std^2)
    draws (stress inputs).  Returned arrays are float64 holding the quantised values.
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B = cfg.batch if batch is None else batch
    L = cfg.seq_len if seq_len is None else seq_len
    D, H, dk, dv = cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v
    s = 1.0 / np.sqrt(D)
    x = rng.standard_normal((B * L, D)).astype(np.float32)
    wq = _normal(rng, (D, H * dk), s).astype(np.float32)
    wk = _normal(rng, (D, H * dk), s).astype(np.float32)
    wv = _normal(rng, (D, H * dv), s).astype(np.float32)
    wa1 = _normal(rng, (D, cfg.rank), s).astype(np.float32)
    wa2 = _normal(rng, (cfg.rank, H * dk), s).astype(np.float32)
    wr = _normal(rng, (D, H * dv), s).astype(np.float32)
    q = (x @ wq).reshape(B, L, H, dk)
    k = (x @ wk).reshape(B, L, H, dk)
    v = (x @ wv).reshape(B, L, H, dv)
    if z_std is None:
        z = ((x @ wa1) @ wa2).reshape(B, L, H, dk).astype(np.float64) + gate_bias
    else:
        z = rng.standard_normal((B, L, H, dk)) * z_std + gate_bias
    r = (x @ wr).reshape(B, L, H, dv).astype(np.float64) + r_bias
    gamma = (1.0 + 0.5 * rng.standard_normal(dv)) if random_gamma else np.ones(dv)
    dy = rng.standard_normal((B, L, H, dv))
    qz = lambda a: quantize(a, cfg.dtype)
    return GLACase(cfg, qz(q), qz(k), qz(v), qz(z), qz(r), f32_round(gamma), qz(dy),
                   x=x.reshape(B, L, D))


@dataclass
class LowRankGate:
    factor: np.ndarray  # [B, L, rank]  x W_a1 per token
    w: np.ndarray       # [H d_k, rank]  W_a2 as a linear layer's weight (out x in)
    bias: np.ndarray    # [H d_k]        b_alpha (fp32 values)


def make_lowrank_gate(cfg: Config, seed: int, *, batch: int | None = None,
                      seq_len: int | None = None, w_std: float | None = None,
                      bias_std: float = 0.0, bias_mean: float = 0.0) -> LowRankGate:
    """Inputs of the low-rank key gate: the factor x W_a1 of unit-variance tokens (N(0, 1)
    entries, as x ~ N(0,1) times weights ~ N(0, 1/D) gives), W_a2 ~ N(0, w_std^2) (default
    1/D^(1/2), the projections' initialisation), b_alpha ~ N(bias_mean, bias_std^2).  A larger
    w_std and a spread bias stress the gate (strong decays, saturated sigmoids)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = cfg.batch if batch is None else batch
    L = cfg.seq_len if seq_len is None else seq_len
    hk = cfg.heads * cfg.d_k
    std = 1.0 / np.sqrt(cfg.d_model) if w_std is None else w_std
    factor = quantize(rng.standard_normal((B, L, cfg.rank)), "bf16")
    w = quantize(rng.standard_normal((hk, cfg.rank)) * std, "bf16")
    bias = f32_round(bias_mean + bias_std * rng.standard_normal(hk))
    return LowRankGate(factor, w, bias)


def make_value_gate_logits(cfg: Config, seed: int, *, batch: int | None = None,
                           seq_len: int | None = None, std: float = 1.0,
                           mean: float = 0.0) -> np.ndarray:
    """Value-side gate logits w [B, L, H, d_v] ~ N(mean, std^2), quantised to bf16 (a
    projection x W_beta + b_beta of unit-variance tokens has unit-scale entries; a large std
    or a very negative mean stresses the gate)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    B = cfg.batch if batch is None else batch
    L = cfg.seq_len if seq_len is None else seq_len
    return quantize(mean + std * rng.standard_normal((B, L, cfg.heads, cfg.d_v)), "bf16")


@dataclass
class SREMCase:
    cfg: Config
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray | None
    dy: np.ndarray


def make_srem_case(cfg: Config, seed: int | None = None, *, batch: int | None = None,
                   with_bias: bool = False, identity: bool = False) -> SREMCase:
    """SREM input x ~ N(0,1) [B, L, D], DWConv weights ~ N(0, 1/9) [D, 3, 3] (fp32)."""
    rng = np.random.Generator(np.random.PCG64((cfg.seed if seed is None else seed) + 7919))
    B = cfg.batch if batch is None else batch
    L, D = cfg.seq_len, cfg.d_model
    x = rng.standard_normal((B, L, D))
    w = rng.standard_normal((D, 3, 3)) / 3.0
    if identity:
        w = np.zeros((D, 3, 3))
        w[:, 1, 1] = 1.0
    bias = rng.standard_normal(D) * 0.1 if with_bias else None
    dy = rng.standard_normal((B, L, D))
    qz = lambda a: quantize(a, cfg.dtype)
    return SREMCase(cfg, qz(x), f32_round(w), None if bias is None else f32_round(bias), qz(dy))


def crop_config(cfg: Config, grid: int = 16) -> Config:
    """The same layer shapes on a grid x grid crop of the token grid (one image)."""
    return cfg_replace(cfg, name=cfg.name + "_crop%d" % grid, batch=1, grid_h=grid, grid_w=grid)


# ------------------------------------------------------------- multi-block chain
@dataclass
class BlockWeights:
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wa1: np.ndarray
    wa2: np.ndarray
    wr: np.ndarray
    wo: np.ndarray      # [H * d_v, D]: the mixer's output projection
    conv_w: np.ndarray  # [D, 3, 3]


def make_block_weights(cfg: Config, rng) -> BlockWeights:
    """One block's projection weights ~ N(0, 1/D) and DWConv weights ~ N(0, 1/9) (fp32)."""
    D, H, dk, dv = cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v
    s = 1.0 / np.sqrt(D)
    f = lambda shape, std: (rng.standard_normal(shape) * std).astype(np.float32).astype(np.float64)
    return BlockWeights(f((D, H * dk), s), f((D, H * dk), s), f((D, H * dv), s),
                        f((D, cfg.rank), s), f((cfg.rank, H * dk), s), f((D, H * dv), s),
                        f((H * dv, D), s), f((D, 3, 3), 1.0 / 3.0))


def project(cfg: Config, x: np.ndarray, wts: BlockWeights):
    """The mixer's operands from block input x [B, L, D] (fp64 matmuls, quantised once):
    q, k, z = (x W_a1) W_a2, v, r, each [B, L, H, d]."""
    B, L, _ = x.shape
    H, dk, dv = cfg.heads, cfg.d_k, cfg.d_v
    x2 = x.reshape(B * L, -1)
    qz = lambda a, d: quantize(a.reshape(B, L, H, d), cfg.dtype)
    return (qz(x2 @ wts.wq, dk), qz(x2 @ wts.wk, dk), qz(x2 @ wts.wv, dv),
            qz((x2 @ wts.wa1) @ wts.wa2, dk), qz(x2 @ wts.wr, dv))


# ----------------------------------------------------------------- DiG block stack
# The full block stack forward (slides Figure 4 and Table 1: S = 12 blocks, XL = 28) on the
# same image sizes; the feedforward is D -> 4 D -> D.
STACKS = {
    "dig_s2_256_stack": (CONFIGS["dig_s2_256"], 12),
    "dig_xl2_256_stack": (Config("dig_xl2_256", 8, 16, 16, 1152, 16, 36, 72, 64, "bf16",
                                 blocks=28, index=5,
                                 note="DiG-XL/2 at 256 px, block stack forward"), 28),
}

BLOCK_WEIGHT_FIELDS = ("w_in", "b_in", "w_gate", "b_gate", "gla_norm_w", "w_out", "b_out",
                       "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "conv_w", "conv_b")


def make_dig_block_weights(cfg: Config, rng, ffn_mult: int = 4) -> dict:
    """One DiG block's weights, bf16-representable matrices and fp32 vectors (as float64):
    projections ~ N(0, 1/fan_in); biases ~ N(0, 0.1^2); head-wise norm weight 1 + N(0, 0.1^2);
    DWConv kernel = identity (centre tap 1, the initialisation the write-up describes) plus
    N(0, 1/36); rows of w_in are q | k | v | u (gate factor, rank cfg.rank) | r."""
    D, H, dk, dv, R = cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v, cfg.rank
    F = ffn_mult * D
    nin = 2 * H * dk + 2 * H * dv + R
    mat = lambda shape, fan: bf16_round(rng.standard_normal(shape) / np.sqrt(fan))
    vec = lambda n, std=0.1: f32_round(rng.standard_normal(n) * std)
    conv = rng.standard_normal((D, 3, 3)) / 6.0
    conv[:, 1, 1] += 1.0
    return dict(w_in=mat((nin, D), D), b_in=vec(nin), w_gate=mat((H * dk, R), R),
                b_gate=vec(H * dk, 1.0), gla_norm_w=f32_round(1.0 + rng.standard_normal(dv) * 0.1),
                w_out=mat((D, H * dv), H * dv), b_out=vec(D), w_ffn1=mat((F, D), D),
                b_ffn1=vec(F), w_ffn2=mat((D, F), F), b_ffn2=vec(D), conv_w=f32_round(conv),
                conv_b=vec(D))


def make_block_cond(cfg: Config, n_blocks: int, rng) -> dict:
    """The conditioning vector c [B, D] ~ N(0, 1) (standing in for the summed timestep and
    label embeddings) and the adaLN regression W_ada [n_blocks * 6 D, D] ~ N(0, 0.1^2 / D),
    b_ada = (1, 0, 0.5, 1, 0, 0.5) per D-wide part (gamma_1, beta_1, alpha_1, gamma_2, beta_2,
    alpha_2), so gamma ~ 1, beta ~ 0, alpha ~ 0.5 with a per-image spread."""
    D = cfg.d_model
    part = np.concatenate([np.full(D, v) for v in (1.0, 0.0, 0.5, 1.0, 0.0, 0.5)])
    return dict(c=bf16_round(rng.standard_normal((cfg.batch, D))),
                w_ada=bf16_round(rng.standard_normal((n_blocks * 6 * D, D)) * (0.1 / np.sqrt(D))),
                b_ada=f32_round(np.tile(part, n_blocks)))

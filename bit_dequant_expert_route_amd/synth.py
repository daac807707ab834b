"""Seeded synthetic inputs for the MoE expert hot path.

This module holds no arithmetic of the method itself (no matvec, no softmax,
no routing, no normalisation).  It only draws numbers and lays them out in the
resident expert format, so that the fp64 oracle and the HIP library can be fed
the very same bytes.

Sources of the shapes (the pages give no weights, so every value here is a
synthetic stand-in):
  * openclawradar.com (ja) "Flash-MoE: running the 397B-parameter Qwen model on
    a MacBook Pro in pure C/Metal", section "Technical implementation": hidden
    size 4096, 512 experts per layer, K=4 routed plus one shared expert, 60
    layers.
  * same page, section "SSD expert streaming": one record of about 6.75 MB per
    expert at 4 bits.
  * a2a-mcp.org (fr) "What is Flash-MoE?", section "FMA-optimised dequantisation
    kernels": weights are nibble codes with a scale and a bias per group.

Counter-based generator
-----------------------
Expert codes and (scale, bias) words come from SplitMix64 (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): output
number i of a generator whose state is k is mix(k + (i+1)*GAMMA).  Keys are
derived by the same rule, one level per id: key(seed, layer, expert, section) =
sm(sm(sm(sm(ROOT, seed), layer), expert), section).  The HIP library carries its
own implementation of this definition (a device fill kernel for the 217 GB
stack); the two are checked against each other byte for byte.

Normal draws (router, shared gate vector, x, residual, inter-layer updates) are
host-only: numpy's PCG64 seeded by a tuple of ids.
"""
from __future__ import annotations

import dataclasses
import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
ROOT = 0x6D6F652D67656E31  # fixed root state of the key tree

# expert id used by the generator for a layer's shared expert
SHARED_GEN_ID = 1 << 20

# section ids inside a record (generator streams)
SEC_GATE_CODES, SEC_UP_CODES, SEC_DOWN_CODES = 0, 1, 2
SEC_GATE_SB, SEC_UP_SB, SEC_DOWN_SB = 3, 4, 5

# normal-draw stream ids
STREAM_ROUTER, STREAM_GATEVEC, STREAM_X, STREAM_HRES, STREAM_UPDATE, STREAM_H0 = 1, 2, 3, 4, 5, 6
STREAM_TOKEN_BASE, STREAM_TOKEN = 7, 8
STREAM_GDN = 9
STREAM_GDN_STATE = 10

# generator ids of a layer's linear-attention projections: two records of the
# expert format with hidden = H and inter = D = heads * head width
#   qko: gate = W_q [D][H], up = W_k [D][H], down = W_o [H][D]
#   vab: gate = W_v [D][H], up rows 0..2 heads-1 = W_alpha, W_beta
GDN_QKO_GEN_ID = (1 << 20) + 1
GDN_VAB_GEN_ID = (1 << 20) + 2

GROUP = 64


# ----------------------------------------------------------------------------
# SplitMix64
# ----------------------------------------------------------------------------
def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def sm(key: int, i: int) -> int:
    """Output number i (0-based) of a SplitMix64 generator with state `key`."""
    return _mix_int((key + ((i + 1) * GAMMA)) & MASK64)


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(MIX1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(MIX2)
        z ^= z >> np.uint64(31)
    return z


def sm_stream(key: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of the generator with state `key` (uint64)."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GAMMA)
    return _mix_np(z)


def section_key(seed: int, layer: int, expert: int, section: int) -> int:
    k = sm(ROOT, seed)
    k = sm(k, layer)
    k = sm(k, expert)
    return sm(k, section)


# ----------------------------------------------------------------------------
# bf16 helpers (bit-level, round to nearest even)
# ----------------------------------------------------------------------------
def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns, ties to even, straight from the
    53-bit significand (no detour through fp32, so there is one rounding).
    Zero maps to (signed) zero; values must lie in bf16's normal range."""
    v = np.asarray(v, dtype=np.float64)
    b = v.view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint32)
    e = ((b >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    m = (b & np.uint64((1 << 52) - 1)) | np.uint64(1 << 52)
    keep = (m >> np.uint64(45)).astype(np.int64)
    rem = (m & np.uint64((1 << 45) - 1)).astype(np.uint64)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & 1) == 1))
    keep = keep + up.astype(np.int64)
    exp = e - 1023 + 127
    carry = keep == 256
    keep = np.where(carry, 128, keep)
    exp = np.where(carry, exp + 1, exp)
    zero = (b & np.uint64(MASK64 >> 1)) == 0
    if np.any(~zero & ((exp < 1) | (exp > 254))):
        raise ValueError("value outside bf16 normal range")
    out = (sign << 15) | (np.clip(exp, 0, 255).astype(np.uint32) << 7) | (keep & 0x7F).astype(np.uint32)
    out = np.where(zero, sign << 15, out)
    return out.astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """bf16 bits of fp32 values, ties to even (used for staging normals)."""
    return f64_to_bf16_rne(np.asarray(v, dtype=np.float32).astype(np.float64))


# ----------------------------------------------------------------------------
# resident expert record (format only)
# ----------------------------------------------------------------------------
def _round256(n: int) -> int:
    return (n + 255) // 256 * 256


@dataclasses.dataclass(frozen=True)
class RecordLayout:
    hidden: int
    inter: int
    bits: int
    gate_codes: int
    up_codes: int
    down_codes: int
    gate_sb: int
    up_sb: int
    down_sb: int
    total: int

    @property
    def words_per_gate_row(self) -> int:
        return self.hidden * self.bits // 32

    @property
    def words_per_down_row(self) -> int:
        return self.inter * self.bits // 32


def record_layout(hidden: int, inter: int, bits: int) -> RecordLayout:
    """Section offsets (bytes) of one expert record: codes of gate [I][H],
    up [I][H], down [H][I], then (scale, bias) words of gate [I][H/64],
    up [I][H/64], down [H][I/64]; each section starts on a 256-byte boundary."""
    assert hidden % GROUP == 0 and inter % GROUP == 0 and bits in (2, 4)
    cg = inter * hidden * bits // 8
    cd = hidden * inter * bits // 8
    sg = inter * (hidden // GROUP) * 4
    sd = hidden * (inter // GROUP) * 4
    off = 0
    offs = []
    for n in (cg, cg, cd, sg, sg, sd):
        offs.append(off)
        off += _round256(n)
    return RecordLayout(hidden, inter, bits, *offs, off)


@dataclasses.dataclass(frozen=True)
class QuantDist:
    """Uniform ranges of the bf16 scale and bias of each group."""
    scale_lo: float
    scale_hi: float
    bias_lo: float
    bias_hi: float


Q4_DIST = QuantDist(0.001, 0.01, -0.08, 0.0)
Q2_DIST = QuantDist(0.005, 0.04, -0.06, 0.0)


def dist_for_bits(bits: int) -> QuantDist:
    return Q4_DIST if bits == 4 else Q2_DIST


def _uniform_bf16(u24: np.ndarray, lo: float, hi: float) -> np.ndarray:
    # v = lo + (hi - lo) * ((u + 0.5) / 2^24), each operation rounded in fp64,
    # no contraction; then one rounding to bf16.
    t = (u24.astype(np.float64) + 0.5) * (1.0 / 16777216.0)
    d = np.float64(hi) - np.float64(lo)
    prod = d * t
    v = np.float64(lo) + prod
    return f64_to_bf16_rne(v)


def gen_codes(key: int, nwords: int) -> np.ndarray:
    """nwords uint32 code words: 64-bit output j fills words 2j (low half) and
    2j+1 (high half)."""
    r = sm_stream(key, (nwords + 1) // 2)
    w = np.empty(2 * r.size, dtype=np.uint32)
    w[0::2] = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    w[1::2] = (r >> np.uint64(32)).astype(np.uint32)
    return w[:nwords]


def gen_sb(key: int, n: int, dist: QuantDist) -> np.ndarray:
    """n (scale, bias) words: scale from output bits 40..63, bias from bits
    16..39; scale in the low 16 bits of the word, bias in the high 16 bits."""
    r = sm_stream(key, n)
    us = (r >> np.uint64(40)).astype(np.uint32)
    ub = ((r >> np.uint64(16)) & np.uint64(0xFFFFFF)).astype(np.uint32)
    s = _uniform_bf16(us, dist.scale_lo, dist.scale_hi).astype(np.uint32)
    b = _uniform_bf16(ub, dist.bias_lo, dist.bias_hi).astype(np.uint32)
    return (s | (b << np.uint32(16))).astype(np.uint32)


def make_record(seed: int, layer: int, expert: int, hidden: int, inter: int,
                bits: int, dist: QuantDist | None = None) -> np.ndarray:
    """One expert record as uint8 bytes (padding bytes are zero)."""
    dist = dist or dist_for_bits(bits)
    lay = record_layout(hidden, inter, bits)
    rec = np.zeros(lay.total, dtype=np.uint8)

    def put(off, arr):
        b = arr.view(np.uint8)
        rec[off:off + b.size] = b

    nw_g = inter * hidden * bits // 32
    nw_d = hidden * inter * bits // 32
    put(lay.gate_codes, gen_codes(section_key(seed, layer, expert, SEC_GATE_CODES), nw_g))
    put(lay.up_codes, gen_codes(section_key(seed, layer, expert, SEC_UP_CODES), nw_g))
    put(lay.down_codes, gen_codes(section_key(seed, layer, expert, SEC_DOWN_CODES), nw_d))
    put(lay.gate_sb, gen_sb(section_key(seed, layer, expert, SEC_GATE_SB), inter * hidden // GROUP, dist))
    put(lay.up_sb, gen_sb(section_key(seed, layer, expert, SEC_UP_SB), inter * hidden // GROUP, dist))
    put(lay.down_sb, gen_sb(section_key(seed, layer, expert, SEC_DOWN_SB), hidden * inter // GROUP, dist))
    return rec


# ----------------------------------------------------------------------------
# normal draws (host only)
# ----------------------------------------------------------------------------
def normals(shape, std: float, *ids: int) -> np.ndarray:
    """fp64 N(0, std^2) draws from PCG64 seeded by the id tuple."""
    rng = np.random.Generator(np.random.PCG64(list(ids)))
    return rng.standard_normal(shape) * std


# ----------------------------------------------------------------------------
# workload presets
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    bits_routed: int
    bits_shared: int
    router_dtype: str      # "f32" | "bf16"
    gate_dtype: str        # "f32" | "bf16"
    x_dtype: str           # "f32" | "bf16"
    n_layers: int = 1
    n_tokens: int = 1
    gdn_heads: int = 0     # linear-attention heads of a stack (0: none)
    gdn_head_dim: int = 0
    gdn_bits: int = 4

    @property
    def record_bytes(self) -> int:
        return record_layout(self.hidden, self.inter, self.bits_routed).total

    @property
    def shared_record_bytes(self) -> int:
        return record_layout(self.hidden, self.inter, self.bits_shared).total

    def weight_bytes_per_token_layer(self) -> int:
        """Router + shared-gate vector + (K+1) expert records."""
        rb = 4 if self.router_dtype == "f32" else 2
        gb = 4 if self.gate_dtype == "f32" else 2
        return (self.n_experts * self.hidden * rb + self.hidden * gb
                + self.top_k * self.record_bytes + self.shared_record_bytes)


CONFIGS = {
    # tiny parity case: H 256, I 128, 16 experts, top-2 + shared, fp32 router and x
    "tiny": LayerConfig("tiny", 256, 128, 16, 2, 4, 4, "f32", "f32", "f32"),
    # Qwen-shaped layer at 4 bits, batch 1
    "q4_layer": LayerConfig("q4_layer", 4096, 1024, 512, 4, 4, 4, "bf16", "bf16", "bf16"),
    # the same layer with 2-bit experts (shared expert at 2 bits too)
    "q2_layer": LayerConfig("q2_layer", 4096, 1024, 512, 4, 2, 2, "bf16", "bf16", "bf16"),
    # 60-layer resident stack, fp32 activations between layers
    "q4_stack": LayerConfig("q4_stack", 4096, 1024, 512, 4, 4, 4, "bf16", "bf16", "f32", n_layers=60),
    # 16-token micro-batch on the Qwen-shaped layer
    "q4_batch16": LayerConfig("q4_batch16", 4096, 1024, 512, 4, 4, 4, "bf16", "bf16", "bf16", n_tokens=16),
    # the same stack with the linear-attention block of the pages in 45 of its
    # layers (64 heads, a 128 x 128 state each, 4-bit projections); the other
    # 15 keep the random update standing in for full attention
    "q4_stack_gdn": LayerConfig("q4_stack_gdn", 4096, 1024, 512, 4, 4, 4, "bf16", "bf16", "f32",
                                n_layers=60, gdn_heads=64, gdn_head_dim=128),
    # small parity cases of the stack and batch paths
    "tiny_stack": LayerConfig("tiny_stack", 256, 128, 16, 2, 4, 4, "bf16", "bf16", "f32", n_layers=8),
    "tiny_batch": LayerConfig("tiny_batch", 256, 128, 16, 2, 4, 4, "bf16", "bf16", "bf16", n_tokens=7),
    "tiny_stack_gdn": LayerConfig("tiny_stack_gdn", 256, 128, 16, 2, 4, 4, "bf16", "bf16", "f32",
                                  n_layers=8, gdn_heads=4, gdn_head_dim=32),
}

ROUTER_STD = 0.02
GATEVEC_STD = 0.02


def router_weights(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    """Router [E][H] as fp32 values or bf16 bit patterns (per cfg)."""
    w = normals((cfg.n_experts, cfg.hidden), ROUTER_STD, seed, STREAM_ROUTER, layer)
    if cfg.router_dtype == "f32":
        return w.astype(np.float32)
    return f64_to_bf16_rne(w)


def shared_gate_vector(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    g = normals((cfg.hidden,), GATEVEC_STD, seed, STREAM_GATEVEC, layer)
    if cfg.gate_dtype == "f32":
        return g.astype(np.float32)
    return f64_to_bf16_rne(g)


def residual(cfg: LayerConfig, seed: int, attempt: int = 0, token: int = 0) -> np.ndarray:
    """fp32 residual stream h_res ~ N(0,1)."""
    return normals((cfg.hidden,), 1.0, seed, STREAM_HRES, attempt, token).astype(np.float32)


def raw_x(cfg: LayerConfig, seed: int, attempt: int = 0) -> np.ndarray:
    """fp32 N(0,1) activation drawn independently of the residual."""
    return normals((cfg.hidden,), 1.0, seed, STREAM_X, attempt).astype(np.float32)


def layer_update(cfg: LayerConfig, seed: int, layer: int, attempt: int = 0) -> np.ndarray:
    """bf16 N(0,1) inter-layer update (stands in for attention / DeltaNet)."""
    return f64_to_bf16_rne(normals((cfg.hidden,), 1.0, seed, STREAM_UPDATE, layer, attempt))


def stack_h0(cfg: LayerConfig, seed: int, token: int = 0) -> np.ndarray:
    return normals((cfg.hidden,), 1.0, seed, STREAM_H0, token).astype(np.float32)


def token_residual(cfg: LayerConfig, seed: int, rho: float, token: int, attempt: int = 0) -> np.ndarray:
    """fp32 residual of one token of a correlated batch: sqrt(rho) z0 +
    sqrt(1 - rho) z_t, with z_t redrawn per token (attempt) on its own."""
    z0 = normals((cfg.hidden,), 1.0, seed, STREAM_TOKEN_BASE)
    zt = normals((cfg.hidden,), 1.0, seed, STREAM_TOKEN, token, attempt)
    return (np.sqrt(rho) * z0 + np.sqrt(1.0 - rho) * zt).astype(np.float32)


def batch_residuals(cfg: LayerConfig, seed: int, rho: float, attempt: int = 0) -> np.ndarray:
    """[T][H] fp32 residuals h_t = sqrt(rho) z0 + sqrt(1-rho) z_t (correlated
    tokens, so that a 16-token batch touches fewer distinct experts)."""
    z0 = normals((cfg.hidden,), 1.0, seed, STREAM_TOKEN_BASE, attempt)
    zt = normals((cfg.n_tokens, cfg.hidden), 1.0, seed, STREAM_TOKEN, attempt)
    return (np.sqrt(rho) * z0[None, :] + np.sqrt(1.0 - rho) * zt).astype(np.float32)


# ----------------------------------------------------------------------------
# linear-attention decode step inputs
# ----------------------------------------------------------------------------
def gdn_inputs(seed: int, n_seq: int, n_heads: int, d_k: int, d_v: int, step: int = 0):
    """fp32 inputs of one gated delta-rule step: q and k of unit length (the
    model normalises them before the recurrence), v ~ N(0,1), decay alpha in
    [0.9, 1), write strength beta in [0, 1), state ~ N(0, 0.1^2) (step 0
    only; later steps carry the state)."""
    shape = (n_seq, n_heads)
    q = normals(shape + (d_k,), 1.0, seed, STREAM_GDN, 0, step)
    k = normals(shape + (d_k,), 1.0, seed, STREAM_GDN, 1, step)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = normals(shape + (d_v,), 1.0, seed, STREAM_GDN, 2, step)
    u = np.random.Generator(np.random.PCG64([seed, STREAM_GDN, 3, step])).random((2,) + shape)
    alpha = 0.9 + 0.1 * u[0]
    beta = u[1]
    state = normals(shape + (d_v, d_k), 0.1, seed, STREAM_GDN, 4)
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)  # noqa: E731
    return f(q), f(k), f(v), f(alpha), f(beta), f(state)


# ----------------------------------------------------------------------------
# linear-attention layers of a stack
# ----------------------------------------------------------------------------
def is_attention_layer(layer: int) -> bool:
    """Every fourth layer is a full-attention layer (15 of 60) and the others
    are linear-attention layers (45 of 60), the mix the pages give."""
    return layer % 4 == 3


def gdn_records(seed: int, layer: int, hidden: int, n_heads: int, d_head: int, bits: int):
    """The (qko, vab) projection records of one linear-attention layer."""
    D = n_heads * d_head
    return (make_record(seed, layer, GDN_QKO_GEN_ID, hidden, D, bits),
            make_record(seed, layer, GDN_VAB_GEN_ID, hidden, D, bits))


def gdn_state0(seed: int, layer: int, n_heads: int, d_head: int, attempt: int = 0) -> np.ndarray:
    """fp32 N(0, 0.1^2) state [heads][d][d] carried in from earlier tokens."""
    return normals((n_heads, d_head, d_head), 0.1, seed, STREAM_GDN_STATE, layer, attempt).astype(np.float32)

"""Seeded synthetic inputs for the sparse-MoE expert FFN layer.

This module is shared by the GPU library's tests/benchmark and by the CPU
oracle's tests.  It only *draws data*: hidden states, router matrices, router
biases, block-quantised expert weights and the expert-residency profile.  It
contains none of the layer's arithmetic (no routing, no dequantisation, no FFN,
no combine) -- both the oracle and the HIP path decode the bytes produced here
on their own.

Workload shapes follow the Strata pages: a 125B MoE model built from 24,576
small experts, 512 per layer over 48 layers, each token routed to 10 of them
(wpnews/nxbn "How Strata works", section on the three storage tiers), a
resident router and shared expert (same section), prompts processed in chunks
of up to 8,192 tokens (same page, chunked prefill section) and an MTP draft of
up to 3 tokens verified in one 4-token pass (same page, speculative decoding
section).  The page "single RTX 5090 runs a 125B model" describes the router as
a light gating network that picks the top-K experts while the rest stay idle.

Weight generation (values drawn from N(0, 0.02), then quantised per block of
32 consecutive elements along each row, one fp16 scale per block):
    s = fp16(amax / qmax)      qmax = 7 (int4) or 127 (int8)
    q = clamp(rint(w / float(s)), qmin, qmax)     (q = 0 when s == 0)
    qmin = -8 (int4) or -127 (int8)
This defines the data only; both sides consume the same bytes.

Canonical expert blob (wfmt = I4B32 or I8B32), all row-major:
    [qg : f x d] [qu : f x d] [qd : d x f] [sg : f x d/32] [su : f x d/32] [sd : d x f/32]
int4 quants are offset-binary nibbles u = q + 8, two per byte, element 2i in
the low nibble; int8 quants are plain two's-complement bytes; scales are IEEE
binary16, little endian.
"""
from __future__ import annotations

import os
import concurrent.futures as _cf
from dataclasses import dataclass, field

import numpy as np

WFMT_I4B32 = 4
WFMT_I8B32 = 8

# Tensor ids for seed streams (spawn keys are (cfg_id, layer, tensor, index)).
_T_X, _T_WR, _T_BIAS, _T_EXPERT, _T_SHARED, _T_PROFILE, _T_BLOBMAP, _T_POOL = range(8)


def expert_bytes(wfmt: int, d: int, f: int) -> int:
    """Size in bytes of one canonical expert blob."""
    n = 3 * d * f
    qbytes = n // 2 if wfmt == WFMT_I4B32 else n
    return qbytes + (n // 32) * 2


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_rows_b32(w: np.ndarray, wfmt: int):
    """Block-32 quantisation of a [R, K] fp32 matrix along its rows (data generation)."""
    R, K = w.shape
    assert K % 32 == 0
    qmax, qmin = (7, -8) if wfmt == WFMT_I4B32 else (127, -127)
    blk = w.reshape(R, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    s16 = (amax / np.float32(qmax)).astype(np.float16)
    s32 = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(blk / s32[:, :, None])
    q = np.where(s32[:, :, None] == 0, 0, q)
    q = np.clip(q, qmin, qmax).astype(np.int8).reshape(R, K)
    return q, s16


def pack_quants(q: np.ndarray, wfmt: int) -> np.ndarray:
    """Serialise quants row-major: int4 as offset-binary nibbles (even element low)."""
    flat = q.reshape(-1)
    if wfmt == WFMT_I8B32:
        return flat.view(np.uint8).copy()
    u = (flat.astype(np.int16) + 8).astype(np.uint8)
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def build_blob(qg, sg, qu, su, qd, sd, wfmt: int) -> np.ndarray:
    parts = [pack_quants(qg, wfmt), pack_quants(qu, wfmt), pack_quants(qd, wfmt),
             sg.reshape(-1).view(np.uint8), su.reshape(-1).view(np.uint8), sd.reshape(-1).view(np.uint8)]
    return np.concatenate(parts)


def gen_expert_blob(rng: np.random.Generator, d: int, f: int, wfmt: int, std: float = 0.02) -> np.ndarray:
    wg = rng.standard_normal((f, d), dtype=np.float32) * np.float32(std)
    wu = rng.standard_normal((f, d), dtype=np.float32) * np.float32(std)
    wd = rng.standard_normal((d, f), dtype=np.float32) * np.float32(std)
    qg, sg = quantize_rows_b32(wg, wfmt)
    qu, su = quantize_rows_b32(wu, wfmt)
    qd, sd = quantize_rows_b32(wd, wfmt)
    return build_blob(qg, sg, qu, su, qd, sd, wfmt)


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_expert_blobs(seed: int, cfg_id: int, layer: int, tensor: int, n: int, d: int, f: int,
                     wfmt: int, out: np.ndarray | None = None) -> np.ndarray:
    """n independent expert blobs, [n, expert_bytes] uint8, one seed stream each."""
    nb = expert_bytes(wfmt, d, f)
    if out is None:
        out = np.empty((n, nb), dtype=np.uint8)
    assert out.shape == (n, nb)

    def one(i):
        out[i] = gen_expert_blob(_rng(seed, cfg_id, layer, tensor, i), d, f, wfmt)

    if n * nb < (1 << 22):
        for i in range(n):
            one(i)
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(n)))
    return out


def zipf_bias(rng: np.random.Generator, E: int, s: float = 1.1) -> np.ndarray:
    """Per-expert router bias 2*ln(Zipf(s) rank weight), normalisation dropped.

    bias[e] = -2 s ln(pi(e) + 1) for a seeded permutation pi of 0..E-1.
    """
    perm = rng.permutation(E)
    return (-2.0 * s * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)


@dataclass
class LayerConfig:
    name: str
    cfg_id: int
    T: int
    d: int
    E: int
    k: int
    f: int
    wfmt: int
    x_dtype: str            # "f32" or "bf16"
    has_shared: bool
    act_mode: str           # "float" or "q8"
    zipf_bias: bool = False
    n_layers: int = 1
    n_resident: int = 0     # slot-pool size for the layer stack
    n_pool_blobs: int = 0   # distinct expert blobs backing the layer stack
    profile_bias: float = 0.0  # stack routers biased by alpha * ln(profile weight); alpha
    notes: str = ""


CONFIGS = {
    # Tiny layer: T=32, d=256, 64 experts, top-4, f=128, fp32 x, int8 block-32 weights, no shared.
    "tiny": LayerConfig("tiny", 1, 32, 256, 64, 4, 128, WFMT_I8B32, "f32", False, "float"),
    # Decode layer: T=1 or T=4 (MTP verify batch), int4 weights, shared expert, bf16 x.
    "decode_t1": LayerConfig("decode_t1", 2, 1, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "float"),
    "decode_t4": LayerConfig("decode_t4", 2, 4, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "float"),
    # Prefill chunk: T=8192, same layer, int8-MFMA path with per-32 int8 activations.
    "prefill": LayerConfig("prefill", 3, 8192, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "q8"),
    # Skewed routing: T=64, int8 weights, Zipf(1.1) router bias.
    "skew": LayerConfig("skew", 4, 64, 2048, 512, 10, 768, WFMT_I8B32, "bf16", True, "float", zipf_bias=True),
    # 48-layer stack, 8192-token chunk, 4,500-slot resident pool.
    "stack": LayerConfig("stack", 5, 8192, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "q8",
                         n_layers=48, n_resident=4500, n_pool_blobs=1024),
    # 48-layer decode stack (T=4 verify batch, or T=1) over the same 4,500-slot
    # pool, with every layer's router biased toward the residency profile so
    # that about 72% of the selected experts are resident ("How Strata works",
    # adaptive expert cache section: 72% of expert reads hit GPU memory with
    # ~4,500 cached experts).  alpha = 0.38 gives that rate for logits of
    # standard deviation 0.02 * sqrt(2048).
    "decode_stack": LayerConfig("decode_stack", 6, 4, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "float",
                                n_layers=48, n_resident=4500, n_pool_blobs=1024, profile_bias=0.38),
    "decode_stack_t1": LayerConfig("decode_stack_t1", 6, 1, 2048, 512, 10, 768, WFMT_I4B32, "bf16", True, "float",
                                   n_layers=48, n_resident=4500, n_pool_blobs=1024, profile_bias=0.38),
}


@dataclass
class Layer:
    cfg: LayerConfig
    x: np.ndarray            # [T, d] float32 (tiny) or uint16 bf16 bits
    Wr: np.ndarray           # [E, d] float32
    bias: np.ndarray | None  # [E] float32
    experts: np.ndarray      # [E, expert_bytes] uint8
    shared: np.ndarray | None  # [expert_bytes] uint8
    extra: dict = field(default_factory=dict)

    def x_f32(self) -> np.ndarray:
        if self.cfg.x_dtype == "bf16":
            return bf16_bits_to_f32(self.x)
        return self.x


def gen_x(seed: int, cfg: LayerConfig, T: int | None = None, layer: int = 0, draw: int = 0) -> np.ndarray:
    T = cfg.T if T is None else T
    x = _rng(seed, cfg.cfg_id, layer, _T_X, draw).standard_normal((T, cfg.d), dtype=np.float32)
    return f32_to_bf16_bits(x) if cfg.x_dtype == "bf16" else x


def gen_router(seed: int, cfg: LayerConfig, layer: int = 0):
    Wr = _rng(seed, cfg.cfg_id, layer, _T_WR, 0).standard_normal((cfg.E, cfg.d), dtype=np.float32) * np.float32(0.02)
    bias = zipf_bias(_rng(seed, cfg.cfg_id, layer, _T_BIAS, 0), cfg.E) if cfg.zipf_bias else None
    return Wr, bias


def make_layer(name: str, seed: int = 0, layer: int = 0, T: int | None = None,
               overrides: dict | None = None) -> Layer:
    """One seeded MoE layer of the named workload (optionally with field overrides)."""
    cfg = CONFIGS[name]
    if overrides:
        cfg = LayerConfig(**{**cfg.__dict__, **overrides})
    if T is not None:
        cfg = LayerConfig(**{**cfg.__dict__, "T": T})
    x = gen_x(seed, cfg, layer=layer)
    Wr, bias = gen_router(seed, cfg, layer)
    experts = gen_expert_blobs(seed, cfg.cfg_id, layer, _T_EXPERT, cfg.E, cfg.d, cfg.f, cfg.wfmt)
    shared = None
    if cfg.has_shared:
        shared = gen_expert_blobs(seed, cfg.cfg_id, layer, _T_SHARED, 1, cfg.d, cfg.f, cfg.wfmt)[0]
    return Layer(cfg, x, Wr, bias, experts, shared)


# ---------------------------------------------------------------------------
# 48-layer stack: residency profile and the expert-blob pool that backs it.
# ---------------------------------------------------------------------------

def stack_profile(seed: int, n_layers: int = 48, E: int = 512) -> np.ndarray:
    """Seeded Zipf(1.1) usage ranking over the n_layers*E global expert ids.

    Returns rank[g] (0 = most used) for global id g = layer*E + e; the
    frequency weight of rank r is (r+1)^-1.1, so residency of the top-N set
    depends only on the ranks.
    """
    rank = np.empty(n_layers * E, dtype=np.int64)
    rank[_rng(seed, 5, 0, _T_PROFILE, 0).permutation(n_layers * E)] = np.arange(n_layers * E)
    return rank


def stack_blob_map(seed: int, n_layers: int, E: int, n_blobs: int):
    """Seeded map (layer, expert) -> pool blob index, plus one blob per layer for the shared expert."""
    r = _rng(seed, 5, 0, _T_BLOBMAP, 0)
    routed = r.integers(0, n_blobs, size=(n_layers, E), dtype=np.int64)
    shared = r.integers(0, n_blobs, size=(n_layers,), dtype=np.int64)
    return routed, shared


def stack_pool(seed: int, cfg: LayerConfig, out: np.ndarray | None = None) -> np.ndarray:
    """The distinct expert blobs backing the layer stack, [n_pool_blobs, expert_bytes]."""
    return gen_expert_blobs(seed, cfg.cfg_id, 0, _T_POOL, cfg.n_pool_blobs, cfg.d, cfg.f, cfg.wfmt, out=out)


@dataclass
class Stack:
    cfg: LayerConfig
    x: np.ndarray            # [T, d] layer-0 input (bf16 bits)
    routers: list            # L arrays [E, d] fp32
    pool: np.ndarray         # [n_pool_blobs, expert_bytes] canonical blobs
    index: np.ndarray        # [L, E] pool row of routed expert (l, e)
    shared_index: np.ndarray  # [L] pool row of layer l's shared expert
    resident: np.ndarray     # global ids (l * E + e) kept resident, best rank first
    biases: list | None = None  # L arrays [E] fp32 router biases (profile-biased routing) or None

    def expert_blob(self, layer: int, e: int) -> np.ndarray:
        return self.pool[self.index[layer, e]]

    def layer_experts(self, layer: int) -> np.ndarray:
        return self.pool[self.index[layer]]

    def shared_blobs(self) -> np.ndarray:
        return self.pool[self.shared_index]


def make_stack(seed: int = 0, name: str = "stack", overrides: dict | None = None, T: int | None = None) -> Stack:
    """The layer stack: per-layer routers, a pool of distinct expert blobs that
    back every (layer, expert) through a seeded map, and the resident set =
    the n_resident best ranks of a seeded Zipf(1.1) usage profile."""
    cfg = CONFIGS[name]
    if overrides:
        cfg = LayerConfig(**{**cfg.__dict__, **overrides})
    if T is not None:
        cfg = LayerConfig(**{**cfg.__dict__, "T": T})
    x = gen_x(seed, cfg)
    routers = [gen_router(seed, cfg, layer=l)[0] for l in range(cfg.n_layers)]
    pool = gen_expert_blobs(seed, cfg.cfg_id, 0, _T_POOL, cfg.n_pool_blobs, cfg.d, cfg.f, cfg.wfmt)
    index, shared_index = stack_blob_map(seed, cfg.n_layers, cfg.E, cfg.n_pool_blobs)
    rank = stack_profile(seed, cfg.n_layers, cfg.E)
    resident = np.argsort(rank, kind="stable")[:cfg.n_resident]
    biases = None
    if cfg.profile_bias:
        biases = [profile_router_bias(rank, l, cfg.E, cfg.profile_bias) for l in range(cfg.n_layers)]
    return Stack(cfg, x, routers, pool, index, shared_index, resident, biases)


def profile_router_bias(rank: np.ndarray, layer: int, E: int, alpha: float, s: float = 1.1) -> np.ndarray:
    """Router bias of one layer from the residency profile: alpha * ln w(rank)
    with w(r) = (r + 1)^-s, the profile's frequency weight of global id layer*E + e."""
    r = rank[layer * E:(layer + 1) * E].astype(np.float64)
    return (-alpha * s * np.log(r + 1.0)).astype(np.float32)

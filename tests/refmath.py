"""Independent reference arithmetic used to pin the oracle (tests only).

Nothing here is shared with the oracle or the HIP library:
  * exact router logits by integer arithmetic on the dyadic fp32 inputs;
  * a numpy decoder of the canonical expert blob;
  * a dense, masked float64 brute force of the whole layer (every expert is
    evaluated for every token and masked by the exact top-k);
  * the int8-activation ("Q8") expert in numpy: its own per-32 quantiser
    (fp32 amax / 127, ties-to-even, clamp +-127), exact int64 block sums
    scaled by both block scales in float64, h rounded to fp32 and requantised
    the same way before the int8 down projection.  The pages' prefill step
    multiplies int8 activations by the quantised weights without
    dequantising them ("Strata benchmarks", bottleneck analysis (1), the
    MMQ int8 tensor-core row of the prefill optimisation table).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_SHIFT = 149  # every finite fp32 value is an integer multiple of 2^-149


def f32_to_int(v: np.ndarray) -> list:
    """fp32 values -> exact Python ints v * 2^149."""
    out = []
    for a in np.asarray(v, dtype=np.float32).reshape(-1).tolist():
        fr = Fraction(a) * (1 << _SHIFT)
        assert fr.denominator == 1
        out.append(int(fr))
    return out


def exact_logits(x: np.ndarray, Wr: np.ndarray, bias=None) -> list:
    """z[t][e] * 2^298 as exact integers (x: [T,d] fp32, Wr: [E,d] fp32)."""
    T, d = x.shape
    E = Wr.shape[0]
    xi = [f32_to_int(x[t]) for t in range(T)]
    wi = [f32_to_int(Wr[e]) for e in range(E)]
    bi = None if bias is None else [b << _SHIFT for b in f32_to_int(bias)]
    z = []
    for t in range(T):
        row = []
        for e in range(E):
            acc = sum(a * b for a, b in zip(xi[t], wi[e]))
            if bi is not None:
                acc += bi[e]
            row.append(acc)
        z.append(row)
    return z


def exact_topk(zrow: list, k: int) -> list:
    """Top-k ids by (logit descending, index ascending) -- Python's sort."""
    return sorted(range(len(zrow)), key=lambda e: (-zrow[e], e))[:k]


def logits_to_float(zrow: list) -> np.ndarray:
    return np.array([float(Fraction(v, 1 << (2 * _SHIFT))) for v in zrow], dtype=np.float64)


def blob_parts(blob: np.ndarray, wfmt: int, d: int, f: int):
    """numpy decoder of the canonical blob -> signed quants (int64) and block
    scales (float64) of the three matrices: ((qg, sg), (qu, su), (qd, sd)),
    qg/qu [f,d], qd [d,f], scales [rows, K/32]."""
    n = d * f
    qb = n // 2 if wfmt == 4 else n
    sb = (n // 32) * 2
    blob = np.asarray(blob, dtype=np.uint8)

    def quants(off, R, K):
        raw = blob[off:off + qb]
        if wfmt == 8:
            q = raw.view(np.int8).astype(np.int64)
        else:
            q = np.empty(n, dtype=np.int64)
            q[0::2] = (raw & 0xF).astype(np.int64) - 8
            q[1::2] = (raw >> 4).astype(np.int64) - 8
        return q.reshape(R, K)

    def scales(off, R, K):
        return blob[off:off + sb].view(np.float16).astype(np.float64).reshape(R, K // 32)

    return ((quants(0, f, d), scales(3 * qb, f, d)), (quants(qb, f, d), scales(3 * qb + sb, f, d)),
            (quants(2 * qb, d, f), scales(3 * qb + 2 * sb, d, f)))


def decode_blob(blob: np.ndarray, wfmt: int, d: int, f: int):
    """numpy decoder of the canonical blob -> (Wg [f,d], Wu [f,d], Wd [d,f]) float64."""
    return tuple(q * np.repeat(s, 32, axis=1) for q, s in blob_parts(blob, wfmt, d, f))


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_ffn(X: np.ndarray, W) -> np.ndarray:
    wg, wu, wd = W
    X = X.astype(np.float64)
    return (silu(X @ wg.T) * (X @ wu.T)) @ wd.T


def brute_force_layer(x, Wr, bias, experts, shared, wfmt, d, f, k, residual=None):
    """Dense masked evaluation: all experts on all tokens, masked by the exact top-k."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    E = Wr.shape[0]
    z = exact_logits(x, Wr, bias)
    mask = np.zeros((T, E))
    ids = []
    for t in range(T):
        top = exact_topk(z[t], k)
        ids.append(top)
        zf = logits_to_float([z[t][e] for e in top])
        p = np.exp(zf - zf[0])
        g = (p / p.sum()).astype(np.float32).astype(np.float64)
        mask[t, top] = g
    out = np.zeros((T, d)) if residual is None else residual.astype(np.float64).copy()
    for e in range(E):
        if not mask[:, e].any():
            continue
        out += mask[:, e:e + 1] * dense_ffn(x, decode_blob(experts[e], wfmt, d, f))
    if shared is not None:
        out += dense_ffn(x, decode_blob(shared, wfmt, d, f))
    return np.array(ids, dtype=np.int32), out


def quant8_blocks(a: np.ndarray):
    """Per-32 int8 quantisation of the rows of a float32 matrix [R, K]:
    s = amax / 127 as an IEEE float32 quotient, q = rint(a / s) in float32
    (ties to even) clamped to +-127, and s = 0, q = 0 for an all-zero block.
    Returns (q int64 [R, K], s float32 [R, K/32])."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    R, K = a.shape
    blk = a.reshape(R, K // 32, 32)
    s = (np.abs(blk).max(axis=2) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(blk / s[:, :, None])
    q = np.where(s[:, :, None] == 0, 0.0, np.clip(r, -127.0, 127.0)).astype(np.int64)
    return q.reshape(R, K), s


def block_scaled_products(qa, sa, qw, sw) -> np.ndarray:
    """out[m, n] = sum over 32-blocks b of sa[m, b] * sw[n, b] * (exact integer
    sum over the block of qa[m, .] * qw[n, .]); float64, [M, N]."""
    M, K = qa.shape
    N = qw.shape[0]
    nb = K // 32
    blk = np.einsum("mbi,nbi->mnb", qa.reshape(M, nb, 32), qw.reshape(N, nb, 32))  # int64, exact
    terms = np.asarray(sa, np.float64)[:, None, :] * np.asarray(sw, np.float64)[None, :, :] * blk
    return terms.sum(axis=2)


def q8_ffn(X: np.ndarray, blob: np.ndarray, wfmt: int, d: int, f: int):
    """One expert in int8-activation mode on the rows of X [M, d] (fp32).
    Returns (y [M, d], g [M, f], u [M, f]) in float64."""
    (qg, sg), (qu, su), (qd, sd) = blob_parts(blob, wfmt, d, f)
    xq, xs = quant8_blocks(X)
    g = block_scaled_products(xq, xs, qg, sg)
    u = block_scaled_products(xq, xs, qu, su)
    h = (silu(g) * u).astype(np.float32)
    hq, hs = quant8_blocks(h)
    return block_scaled_products(hq, hs, qd, sd), g, u


def brute_force_layer_q8(x, Wr, bias, experts, shared, wfmt, d, f, k, residual=None):
    """The dense masked brute force of the layer with int8-activation experts."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    E = Wr.shape[0]
    z = exact_logits(x, Wr, bias)
    mask = np.zeros((T, E))
    ids = []
    for t in range(T):
        top = exact_topk(z[t], k)
        ids.append(top)
        zf = logits_to_float([z[t][e] for e in top])
        p = np.exp(zf - zf[0])
        mask[t, top] = (p / p.sum()).astype(np.float32).astype(np.float64)
    out = np.zeros((T, d)) if residual is None else residual.astype(np.float64).copy()
    for e in range(E):
        if mask[:, e].any():
            out += mask[:, e:e + 1] * q8_ffn(x, experts[e], wfmt, d, f)[0]
    if shared is not None:
        out += q8_ffn(x, shared, wfmt, d, f)[0]
    return np.array(ids, dtype=np.int32), out


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def within_tolerance(got, ref, rel=2e-3, maxabs_frac=1e-2):
    """Float parity bar: rel-L2 <= 2e-3 and max-abs <= 1e-2 * RMS(ref); exact if ref == 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if rms == 0.0:
        return bool(np.all(got == 0.0)), 0.0, float(np.max(np.abs(got))) if got.size else 0.0
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref)))
    return (r <= rel and m <= maxabs_frac * rms), r, m / rms

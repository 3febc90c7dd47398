"""Quality diagnostics of the quantized cache formats -- TEST INFRASTRUCTURE ONLY.

Built on the CPU oracle: for synthetic caches of four kinds it compares attention over the
decoded cache with exact fp64 attention over the unquantized inputs and reports

  * KL(p_ref || p_q) of the softmax distributions, mean and worst case over query heads;
  * top-5 routing recall: the share of the 5 highest-weight reference positions that are
    also among the 5 highest quantized ones;
  * scale and direction errors of keys, values and the attention output (the "6D" card):
    SNR = 10 log10(||x||^2 / ||x - x^||^2) in dB and eps_dir = 1 - cos(x, x^), averaged.

(Statistical Inference and Quality Measures of KV Cache Quantisations Inspired by
TurboQuant: the KL and top-5 recall proxies, worst-case KL as the reliability measure, the
6D scale/direction card for K, V and output, and the Gaussian, heavy-tailed, low-rank and
"focused" test distributions.)  Readings: SNR in dB of the energy ratio, direction error as
one minus the cosine, a low-rank cache as keys and values in a random rank-r subspace plus
1 % isotropic noise, a focused cache as Gaussian keys with the query aligned to one key
scaled up so that it dominates the softmax.

Run ``python -m oracle.quality`` for the report over the library's formats.
"""
from __future__ import annotations

import numpy as np

from . import K_ASYM2, K_ASYM4, K_LLOYD4, V_ASYM4_G32, V_KQV, Geometry, OracleCache


# ------------------------------------------------------------------ metrics
def softmax(lg: np.ndarray) -> np.ndarray:
    e = np.exp(lg - lg.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def kl(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """KL(p || q) along the last axis (terms with p = 0 contribute 0)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * (np.log(p) - np.log(q)), 0.0)
    return t.sum(-1)


def topk_recall(p: np.ndarray, q: np.ndarray, k: int = 5) -> np.ndarray:
    """|topk(p) & topk(q)| / k along the last axis."""
    a = np.argsort(-p, axis=-1)[..., :k]
    b = np.argsort(-q, axis=-1)[..., :k]
    return np.array([len(set(x) & set(y)) / k for x, y in zip(a.reshape(-1, k), b.reshape(-1, k))]).reshape(
        p.shape[:-1])


def snr_db(x: np.ndarray, xh: np.ndarray) -> float:
    """Mean over vectors (last axis) of 10 log10(||x||^2 / ||x - x^||^2)."""
    num = (x ** 2).sum(-1)
    den = np.maximum(((x - xh) ** 2).sum(-1), 1e-300)
    return float(np.mean(10.0 * np.log10(num / den)))


def dir_err(x: np.ndarray, xh: np.ndarray) -> float:
    """Mean over vectors of 1 - cos(x, x^)."""
    c = (x * xh).sum(-1) / np.maximum(np.linalg.norm(x, axis=-1) * np.linalg.norm(xh, axis=-1), 1e-300)
    return float(np.mean(1.0 - c))


# ------------------------------------------------------------------ synthetic caches
def draw(kind: str, T: int, d: int, G: int, rng: np.random.Generator, nu: float = 3.0, rank: int = 4):
    """Keys, values [T, d] and queries [G, d] (fp32) of one kind: "gaussian", "t" (Student-t
    with nu degrees of freedom), "lowrank" (rank-r subspace + 1 % noise), "focused"."""
    if kind == "gaussian":
        k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
        q = rng.standard_normal((G, d))
    elif kind == "t":
        k, v = rng.standard_t(nu, (T, d)), rng.standard_t(nu, (T, d))
        q = rng.standard_normal((G, d))
    elif kind == "lowrank":
        B = np.linalg.qr(rng.standard_normal((d, rank)))[0] * np.sqrt(d / rank)
        k = rng.standard_normal((T, rank)) @ B.T + 0.01 * rng.standard_normal((T, d))
        v = rng.standard_normal((T, rank)) @ B.T + 0.01 * rng.standard_normal((T, d))
        q = rng.standard_normal((G, rank)) @ B.T
    elif kind == "focused":
        k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
        hot = rng.integers(0, T, G)
        q = k[hot] / np.linalg.norm(k[hot], axis=1, keepdims=True) * 3.0 * np.sqrt(d) ** 0.5
    else:
        raise ValueError(kind)
    return k.astype(np.float32), v.astype(np.float32), q.astype(np.float32)


# ------------------------------------------------------------------ one measurement
def measure(kind: str, *, k_format=K_ASYM2, k_hadamard=0, k_ch0_bf16=0, v_format=V_ASYM4_G32, d=128, T=2048,
            G=4, seed=0, keep=0, qjl_signs=None, **draw_kw) -> dict:
    """Quality of one format on one synthetic cache (one KV head, G query heads)."""
    rng = np.random.default_rng(seed)
    k, v, q = draw(kind, T, d, G, rng, **draw_kw)
    cap = (T + 255) // 256 * 256
    geo = Geometry(batch=1, n_kv_heads=1, head_dim=d, capacity=cap, k_format=k_format, k_hadamard=k_hadamard,
                   k_ch0_bf16=k_ch0_bf16, v_format=v_format)
    if v_format == V_KQV and qjl_signs is None:
        qjl_signs = rng.integers(0, 2 ** 32, d // 32, dtype=np.uint64).astype(np.uint32)
    oc = OracleCache(geo, qjl_signs=qjl_signs)
    oc.append(k[None], v[None])
    sm = 1.0 / np.sqrt(d)
    out, _, lg = oc.decode(q[None], sm, keep, want_logits=True)
    kh, vh = oc.dequant(0)
    if k_hadamard:  # decoded keys are in rotated coordinates: back to the inputs' ones
        import scipy.linalg
        kh = kh @ scipy.linalg.hadamard(d).astype(np.float64) / d
    k64, v64, q64 = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    p_ref = softmax(sm * q64 @ k64.T)
    p_q = softmax(lg[0])
    o_ref = p_ref @ v64
    kls = kl(p_ref, p_q)
    return {"kl_mean": float(kls.mean()), "kl_max": float(kls.max()),
            "top5_recall": float(topk_recall(p_ref, p_q).mean()),
            "k_snr_db": snr_db(k64, kh), "k_dir": dir_err(k64, kh),
            "v_snr_db": snr_db(v64, vh), "v_dir": dir_err(v64, vh),
            "o_snr_db": snr_db(o_ref, out[0]), "o_dir": dir_err(o_ref, out[0])}


FORMATS = {
    "INT2 keys + INT4 values": dict(k_format=K_ASYM2),
    "INT2+ch0 keys + INT4 values": dict(k_format=K_ASYM2, k_ch0_bf16=1),
    "INT4 keys + INT4 values": dict(k_format=K_ASYM4),
    "WHT+Lloyd-Max keys + INT4 values": dict(k_format=K_LLOYD4, k_hadamard=1),
    "KQV (WHT+Lloyd-Max keys, WHT+3-bit+QJL values)": dict(k_format=K_LLOYD4, k_hadamard=1, v_format=V_KQV),
}
KINDS = ("gaussian", "t", "lowrank", "focused")


def report(T: int = 2048, seeds=(0, 1, 2)) -> str:
    """Markdown table of the quality metrics, averaged over seeds (kl_max: worst over seeds)."""
    cols = ["kl_mean", "kl_max", "top5_recall", "k_snr_db", "k_dir", "v_snr_db", "v_dir", "o_snr_db", "o_dir"]
    lines = ["| format | cache | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for fname, fkw in FORMATS.items():
        for kind in KINDS:
            ms = [measure(kind, T=T, seed=s, **fkw) for s in seeds]
            row = [max(m[c] for m in ms) if c == "kl_max" else float(np.mean([m[c] for m in ms])) for c in cols]
            lines.append(f"| {fname} | {kind} | " + " | ".join(f"{x:.4g}" for x in row) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    print(report())

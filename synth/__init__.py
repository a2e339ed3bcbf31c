"""Seeded synthetic inputs for the local MoE expert layer.

This module only draws inputs; it holds none of the layer's arithmetic. Both
the CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so the two sides see the same values.

Shapes and value distributions follow the workloads the pages describe:
 - x ~ N(0,1) rounded to bf16 (Hysen Labs page, usage example draws x with randn);
 - W_up [E,H,2I], W_down [E,I,H] ~ N(0, 0.02) bf16 (same page: weight init std 0.02,
   no bias);
 - topk_idx [N,K] int32 with -1 for slots that are not valid on this rank
   (GitHub issue #68, non-expand outputs of DeepEP dispatch);
 - topk_weights [N,K] fp32 = softmax of N(0,1) logits over the valid slots of a
   row, 0 at -1 slots;
 - dout ~ N(0,1) bf16 (the upstream gradient; the pages are silent).

Named workloads (sizes of one expert-parallel rank's share):
 - ``tiny``: N=64, H=128, I=256, E=8, K=2; distinct uniform experts, 10% of slots -1.
 - ``qwen3_rank``: 256 global experts top-8 over 8 ranks, this rank owns globals
   [0,32); rows that hit the rank at least once (DeepEP only sends those), N=16384,
   H=2048, I=512 (Qwen3.6 commit notes: 256 experts x top-8, 16384 tokens).
 - ``dsv3_rank``: N=8192, H=7168, I=2048, E=32 of 256 globals, K=8; expert
   popularity Zipf(1.1) with a seeded rank permutation; the rank's two least
   popular local experts get zero popularity, so some experts receive 0 rows and
   some more than 4x the mean (checked; the next seed is taken otherwise).
 - ``decode``: N=8, H=7168, I=2048, E=32, K=8, each slot -1 with probability 0.5,
   rows left with no valid slot redrawn.
 - ``long_prefill``: N=65536, H=4096, I=1536, E=64, K=6, uniform, 20% of slots -1.
"""
from __future__ import annotations

import os

import numpy as np

CONFIGS = {
    "tiny": dict(N=64, H=128, I=256, E=8, K=2, routing="uniform", p_invalid=0.1,
                 min_valid=0, backward=False),
    "qwen3_rank": dict(N=16384, H=2048, I=512, E=32, K=8, routing="ep_share",
                       global_experts=256, zipf_s=None, backward=True),
    "dsv3_rank": dict(N=8192, H=7168, I=2048, E=32, K=8, routing="ep_share",
                      global_experts=256, zipf_s=1.1, zero_tail=2, backward=True),
    "decode": dict(N=8, H=7168, I=2048, E=32, K=8, routing="uniform", p_invalid=0.5,
                   min_valid=1, backward=False),
    "long_prefill": dict(N=65536, H=4096, I=1536, E=64, K=6, routing="uniform",
                         p_invalid=0.2, min_valid=0, backward=True),
}

# independent streams per drawn quantity, so changing one draw leaves the others fixed
_S_ROUTE, _S_LOGIT, _S_X, _S_WUP, _S_WDOWN, _S_DOUT, _S_LOGITS = range(7)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_normal(seed: int, stream: int, shape, std: float, chunk: int = 1 << 22) -> np.ndarray:
    """N(0, std) rounded to bf16, as uint16 bits. Chunk i is drawn from its own
    generator (seed, stream, i), so the values do not depend on how many threads
    fill the chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)

    def fill(i):
        m = min(chunk, n - i)
        v = np.random.default_rng([int(seed), int(stream), i // chunk]).standard_normal(
            m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[i:i + m] = f32_to_bf16_bits(v)

    starts = range(0, n, chunk)
    if n > 4 * chunk:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    else:
        for i in starts:
            fill(i)
    return out.reshape(shape)


# ---- routing structures --------------------------------------------------------

def _distinct_topk(keys: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest keys per row, largest first (a top-k selection)."""
    part = np.argpartition(-keys, K - 1, axis=1)[:, :K]
    kv = np.take_along_axis(keys, part, axis=1)
    order = np.argsort(-kv, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def routing_uniform(N: int, E: int, K: int, p_invalid: float, min_valid: int, seed: int):
    """K distinct uniform experts per row; each slot independently -1 with p_invalid."""
    assert K <= E
    rng = _rng(seed, _S_ROUTE)
    idx = _distinct_topk(rng.random((N, E)), K).astype(np.int32)
    drop = rng.random((N, K)) < p_invalid
    idx[drop] = -1
    if min_valid > 0:
        for _ in range(1000):
            bad = (idx >= 0).sum(axis=1) < min_valid
            if not bad.any():
                break
            nb = int(bad.sum())
            re = _distinct_topk(rng.random((nb, E)), K).astype(np.int32)
            re[rng.random((nb, K)) < p_invalid] = -1
            idx[bad] = re
        else:
            raise RuntimeError("could not draw rows with enough valid slots")
    return idx


def _zipf_log_popularity(G: int, s: float, rng: np.random.Generator, zero_tail_local: int, E: int):
    ranks = rng.permutation(G) + 1  # popularity rank of each global expert
    logp = -s * np.log(ranks.astype(np.float64))
    if zero_tail_local:
        local = np.arange(E)
        least = local[np.argsort(ranks[local])[::-1][:zero_tail_local]]
        logp[least] = -np.inf
    return logp


def routing_ep_share(N: int, E: int, K: int, G: int, seed: int, zipf_s=None, zero_tail: int = 0):
    """One EP rank's received rows: each token picks K distinct of G global experts
    (uniform, or Gumbel-top-k on Zipf log-popularity); this rank owns globals [0,E)
    as local 0..E-1, other slots are -1; only rows with >= 1 local slot are kept."""
    rng = _rng(seed, _S_ROUTE)
    logp = None
    if zipf_s is not None:
        logp = _zipf_log_popularity(G, zipf_s, rng, zero_tail, E)
    rows = []
    have = 0
    while have < N:
        B = max(1024, int((N - have) * 2))
        if logp is None:
            keys = rng.random((B, G))
        else:
            keys = logp[None, :] + rng.gumbel(size=(B, G))
        g = _distinct_topk(keys, K)
        loc = np.where(g < E, g, -1).astype(np.int32)
        keep = loc[(loc >= 0).any(axis=1)]
        rows.append(keep)
        have += keep.shape[0]
    return np.concatenate(rows, axis=0)[:N]


def make_routing(name_or_cfg, seed: int = 0):
    """(topk_idx, seed actually used) for a named workload or a config dict."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    N, E, K = cfg["N"], cfg["E"], cfg["K"]
    if cfg["routing"] == "uniform":
        return routing_uniform(N, E, K, cfg["p_invalid"], cfg.get("min_valid", 0), seed), seed
    if cfg["routing"] == "ep_share":
        s = seed
        for _ in range(64):
            idx = routing_ep_share(N, E, K, cfg["global_experts"], s, cfg.get("zipf_s"),
                                   cfg.get("zero_tail", 0))
            if cfg.get("zipf_s") is None:
                return idx, s
            freq = np.bincount(idx[idx >= 0], minlength=E)
            if (freq == 0).any() and freq.max() > 4 * freq.mean():
                return idx, s
            s += 1
        raise RuntimeError("no seed gave the required skew")
    raise ValueError(cfg["routing"])


def make_topk_weights(topk_idx: np.ndarray, seed: int) -> np.ndarray:
    """softmax of N(0,1) logits over each row's valid slots (fp32); 0 at -1 slots."""
    rng = _rng(seed, _S_LOGIT)
    logits = rng.standard_normal(topk_idx.shape)
    valid = topk_idx >= 0
    logits = np.where(valid, logits, -np.inf)
    m = np.max(logits, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    ex = np.where(valid, np.exp(logits - m), 0.0)
    den = ex.sum(axis=1, keepdims=True)
    w = np.divide(ex, den, out=np.zeros_like(ex), where=den > 0)
    return w.astype(np.float32)


def make_inputs(name_or_cfg, seed: int = 0, dout: bool = True, topk_idx=None,
                w_std: float = 0.02) -> dict:
    """All inputs of one workload as numpy arrays; float tensors as bf16 bits (uint16)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    N, H, I, E, K = cfg["N"], cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    used = seed
    if topk_idx is None:
        topk_idx, used = make_routing(cfg, seed)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    d = dict(cfg=cfg, seed=used, N=N, H=H, I=I, E=E, K=K, topk_idx=topk_idx,
             topk_weights=make_topk_weights(topk_idx, used),
             x=bf16_normal(used, _S_X, (N, H), 1.0),
             w_up=bf16_normal(used, _S_WUP, (E, H, 2 * I), w_std),
             w_down=bf16_normal(used, _S_WDOWN, (E, I, H), w_std))
    if dout:
        d["dout"] = bf16_normal(used, _S_DOUT, (N, H), 1.0)
    return d


def router_logits(N: int, E: int, seed: int, ties: bool = False) -> np.ndarray:
    """Router logits [N,E] fp32 ~ N(0,1); with ties=True they are rounded to multiples
    of 0.25 in [-1, 1], so most rows hold many equal values."""
    rng = _rng(seed, _S_LOGITS)
    lg = rng.standard_normal((N, E)).astype(np.float32)
    if ties:
        lg = np.clip(np.round(lg * 4.0) / 4.0, -1.0, 1.0).astype(np.float32)
    return lg


def case(N, H, I, E, K, seed=0, p_invalid=0.1, min_valid=0, topk_idx=None, dout=True,
         w_std=0.02) -> dict:
    """A uniform-routing case of any shape (tests)."""
    cfg = dict(N=N, H=H, I=I, E=E, K=K, routing="uniform", p_invalid=p_invalid,
               min_valid=min_valid)
    return make_inputs(cfg, seed=seed, dout=dout, topk_idx=topk_idx, w_std=w_std)

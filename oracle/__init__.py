"""CPU oracle for the local MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Python bindings (ctypes) for ``moe_oracle.c``: a plain fp64 CPU implementation
of the routing metadata, the forward (grouped up-projection with SwiGLU, down
projection, weighted combine) and the backward, plus a brute-force forward and
sampled entry points for large shapes.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never loads it; it
shares no code with the HIP path. The C source cites the web pages it follows
(GitHub issue #68 on Dao-AILab/sonic-moe and the pages listed in
``moe_oracle.h``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "libmoe_oracle.so")

BF16, F32, F64 = 0, 1, 2
FLAG_BAD_EXPERT = 1

_lib = None


def build() -> str:
    """Compile the oracle with gcc (C11, -O2, OpenMP). Returns the .so path."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = ctypes.CDLL(_SO)
        _declare(_lib)
    return _lib


_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p


def _declare(L):
    L.oracle_build_metadata.restype = _i64
    L.oracle_build_metadata.argtypes = [_i64, _i64, _i64] + [_vp] * 13
    L.oracle_forward.restype = None
    L.oracle_forward.argtypes = [_i64] * 4 + [_vp] * 12
    L.oracle_backward.restype = None
    L.oracle_backward.argtypes = [_i64] * 5 + [_vp] * 19
    L.oracle_bruteforce_forward.restype = None
    L.oracle_bruteforce_forward.argtypes = [_i64] * 5 + [_vp] * 6
    L.oracle_sample_tokens.restype = None
    L.oracle_sample_tokens.argtypes = [_i64] * 5 + [_vp, _int, _vp, _int, _vp, _vp, _int,
                                                     _vp, _vp, _i64, _vp, _vp, _vp, _vp]
    L.oracle_sample_h_rows.restype = None
    L.oracle_sample_h_rows.argtypes = [_i64] * 3 + [_vp, _int, _vp, _int, _vp, _vp, _i64, _vp, _vp]
    L.oracle_sample_dw_down_rows.restype = None
    L.oracle_sample_dw_down_rows.argtypes = [_i64] * 3 + [_vp, _int, _vp, _int, _vp, _int,
                                                          _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]
    L.oracle_sample_dw_up_cols.restype = None
    L.oracle_sample_dw_up_cols.argtypes = [_i64] * 3 + [_vp, _int, _vp, _int, _vp, _vp, _int,
                                                        _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]
    L.oracle_route.restype = None
    L.oracle_route.argtypes = [_i64] * 3 + [_vp, _int, _int, _int, _vp, _vp, _vp]
    L.oracle_num_threads.restype = _int
    L.oracle_num_threads.argtypes = []


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _typed(a: np.ndarray):
    """(array, dtype code) for a tensor given as bf16 bits (uint16), fp32 or fp64."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    raise TypeError(f"unsupported oracle tensor dtype {a.dtype}")


def route(logits, K: int, mode: int, renormalize: bool = False) -> dict:
    """Router top-K, weights and the load-balancing aux loss (see oracle_route).
    logits [N,E] as bf16 bits (uint16), fp32 or fp64."""
    lg, dt = _typed(logits)
    N, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError(f"route needs 1 <= K <= E (K={K}, E={E})")
    idx = np.zeros((N, K), np.int32)
    w = np.zeros((N, K), np.float64)
    aux = np.zeros(1, np.float64)
    lib().oracle_route(N, E, K, _p(lg), dt, int(mode), int(bool(renormalize)), _p(idx), _p(w),
                       _p(aux))
    return dict(topk_idx=idx, topk_weights=w, aux=float(aux[0]))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def build_metadata(topk_idx: np.ndarray, topk_weights: np.ndarray, E: int) -> dict:
    """Routing metadata of the non-expand layout. Arrays are sized to P."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    N, K = idx.shape
    cap = max(N * K, 1)
    freq = np.zeros(E, np.int32)
    foff = np.zeros(E + 1, np.int32)
    xg = np.zeros(cap, np.int32)
    ss = np.zeros(cap, np.int32)
    sr = np.zeros(cap, np.int32)
    toff = np.zeros(N + 1, np.int32)
    rs = np.zeros(cap, np.float32)
    pt = np.zeros(cap, np.int32)
    pk = np.zeros(cap, np.int32)
    pe = np.zeros(cap, np.int32)
    flags = np.zeros(1, np.uint32)
    P = lib().oracle_build_metadata(N, K, E, _p(idx), _p(w), _p(freq), _p(foff), _p(xg), _p(ss),
                                    _p(sr), _p(toff), _p(rs), _p(pt), _p(pk), _p(pe), _p(flags))
    P = int(P)
    return dict(
        P=P, N=N, K=K, E=E,
        expert_frequency=freq, expert_frequency_offset=foff,
        x_gather_idx=xg[:P].copy(), s_scatter_idx=ss[:P].copy(),
        s_reverse_scatter_idx=sr[:P].copy(),
        num_activated_expert_per_token_offset=toff, router_scores=rs[:P].copy(),
        pair_token=pt[:P].copy(), pair_slot=pk[:P].copy(), pair_expert=pe[:P].copy(),
        flags=int(flags[0]),
    )


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def forward(x, w_up, w_down, meta) -> dict:
    """Full forward in fp64. x [N,H], w_up [E,H,2I], w_down [E,I,H] (fp64)."""
    x, w_up, w_down = _f64(x), _f64(w_up), _f64(w_down)
    N, H = x.shape
    E, _, I2 = w_up.shape
    I = I2 // 2
    P = meta["P"]
    h = np.zeros((P, I2))
    a = np.zeros((P, I))
    y = np.zeros((P, H))
    out = np.zeros((N, H))
    lib().oracle_forward(N, H, I, E, _p(x), _p(w_up), _p(w_down),
                         _p(meta["expert_frequency_offset"]), _p(meta["x_gather_idx"]),
                         _p(meta["s_reverse_scatter_idx"]),
                         _p(meta["num_activated_expert_per_token_offset"]),
                         _p(meta["router_scores"]), _p(h), _p(a), _p(y), _p(out))
    return dict(h=h, a=a, y=y, out=out)


def backward(x, w_up, w_down, dout, meta, fwd) -> dict:
    """Full backward in fp64; ``fwd`` is the dict returned by :func:`forward`."""
    x, w_up, w_down, dout = _f64(x), _f64(w_up), _f64(w_down), _f64(dout)
    N, H = x.shape
    E, _, I2 = w_up.shape
    I = I2 // 2
    K = meta["K"]
    dx = np.zeros((N, H))
    dw_up = np.zeros((E, H, I2))
    dw_down = np.zeros((E, I, H))
    dtw = np.zeros((N, K))
    lib().oracle_backward(N, K, H, I, E, _p(x), _p(w_up), _p(w_down), _p(dout),
                          _p(meta["expert_frequency_offset"]), _p(meta["x_gather_idx"]),
                          _p(meta["s_scatter_idx"]), _p(meta["s_reverse_scatter_idx"]),
                          _p(meta["num_activated_expert_per_token_offset"]),
                          _p(meta["router_scores"]), _p(meta["pair_token"]),
                          _p(meta["pair_slot"]), _p(fwd["h"]), _p(fwd["a"]), _p(fwd["y"]),
                          _p(dx), _p(dw_up), _p(dw_down), _p(dtw))
    return dict(dx=dx, dw_up=dw_up, dw_down=dw_down, d_topk_weights=dtw)


def bruteforce_forward(x, topk_idx, topk_weights, w_up, w_down) -> np.ndarray:
    x, w_up, w_down = _f64(x), _f64(w_up), _f64(w_down)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    N, H = x.shape
    E, _, I2 = w_up.shape
    K = idx.shape[1]
    out = np.zeros((N, H))
    lib().oracle_bruteforce_forward(N, K, H, I2 // 2, E, _p(x), _p(idx), _p(w),
                                    _p(w_up), _p(w_down), _p(out))
    return out


def sample_tokens(x, w_up, w_down, topk_idx, topk_weights, tokens, dout=None) -> dict:
    """out / dx / d_topk_weights rows of the listed tokens (any size)."""
    x, xd = _typed(x)
    w_up, wd = _typed(w_up)
    w_down, wd2 = _typed(w_down)
    assert wd == wd2, "w_up and w_down must share a dtype"
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    N, H = x.shape
    E, _, I2 = w_up.shape
    K = idx.shape[1]
    n = tok.shape[0]
    out = np.zeros((n, H))
    dx = dtw = None
    dd_ptr, dd_dt = None, F64
    if dout is not None:
        dout, dd_dt = _typed(dout)
        dd_ptr = _p(dout)
        dx = np.zeros((n, H))
        dtw = np.zeros((n, K))
    lib().oracle_sample_tokens(N, K, H, I2 // 2, E, _p(x), xd, _p(w_up), wd, _p(w_down),
                               dd_ptr, dd_dt, _p(idx), _p(w), n, _p(tok), _p(out), _p(dx), _p(dtw))
    return dict(out=out, dx=dx, d_topk_weights=dtw)


def sample_h_rows(x, w_up, meta, rows) -> np.ndarray:
    x, xd = _typed(x)
    w_up, wd = _typed(w_up)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    H = x.shape[1]
    E, _, I2 = w_up.shape
    out = np.zeros((rows.shape[0], I2))
    lib().oracle_sample_h_rows(H, I2 // 2, E, _p(x), xd, _p(w_up), wd,
                               _p(meta["expert_frequency_offset"]), _p(meta["x_gather_idx"]),
                               rows.shape[0], _p(rows), _p(out))
    return out


def sample_dw_down_rows(x, w_up, dout, meta, e_list, j_list) -> np.ndarray:
    x, xd = _typed(x)
    w_up, wd = _typed(w_up)
    dout, dd = _typed(dout)
    el = np.ascontiguousarray(e_list, dtype=np.int64)
    jl = np.ascontiguousarray(j_list, dtype=np.int64)
    H = x.shape[1]
    E, _, I2 = w_up.shape
    out = np.zeros((el.shape[0], H))
    lib().oracle_sample_dw_down_rows(H, I2 // 2, E, _p(x), xd, _p(w_up), wd, _p(dout), dd,
                                     _p(meta["expert_frequency_offset"]),
                                     _p(meta["x_gather_idx"]), _p(meta["s_scatter_idx"]),
                                     _p(meta["router_scores"]), el.shape[0], _p(el), _p(jl),
                                     _p(out))
    return out


def sample_dw_up_cols(x, w_up, w_down, dout, meta, e_list, jj_list) -> np.ndarray:
    """Returns [n, 2, H]: columns 2jj (gate) and 2jj+1 (up) of dW_up[e]."""
    x, xd = _typed(x)
    w_up, wd = _typed(w_up)
    w_down, wd2 = _typed(w_down)
    assert wd == wd2
    dout, dd = _typed(dout)
    el = np.ascontiguousarray(e_list, dtype=np.int64)
    jl = np.ascontiguousarray(jj_list, dtype=np.int64)
    H = x.shape[1]
    E, _, I2 = w_up.shape
    out = np.zeros((el.shape[0], 2, H))
    lib().oracle_sample_dw_up_cols(H, I2 // 2, E, _p(x), xd, _p(w_up), wd, _p(w_down), _p(dout),
                                   dd, _p(meta["expert_frequency_offset"]),
                                   _p(meta["x_gather_idx"]), _p(meta["s_scatter_idx"]),
                                   _p(meta["router_scores"]), el.shape[0], _p(el), _p(jl),
                                   _p(out))
    return out

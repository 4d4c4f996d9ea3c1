"""CPU oracle for the TokenGate gate-layer path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product: the two share no code.

The arithmetic lives in ``tg_oracle.c`` (plain fp64 loops, OpenMP over
independent rows).  This module builds it with gcc and wraps it with ctypes;
it only converts inputs to float64 (an exact widening of bf16 / fp32 values)
and allocates outputs.  Every function cites the passage it follows on the
pages:

  DeepDive = "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient LLM
             Prefill" (agientry.com paper deep dive)
  Summary  = "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill with
             Learned Token Pruning" (thelatestinai.com)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tg_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile tg_oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.tgo_gate_score.argtypes = [_D, _D, _D, _U8, _i64, _i64, _i64, _D, _D]
    lib.tgo_gate_score.restype = None
    lib.tgo_select_topk.argtypes = [_F, _U8, _i64, _i64, _i64, _I32]
    lib.tgo_select_topk.restype = _i64
    lib.tgo_compact.argtypes = [_U8, _I32, _F, _I32, _i64, _i64, _i64, _U8, _I32, _F]
    lib.tgo_compact.restype = None
    lib.tgo_attn_fwd.argtypes = [_D, _D, _D, _D, _D, _I32, ctypes.c_double, ctypes.c_double, _D,
                                 _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _I64, _i64, ctypes.c_int, _D, _D]
    lib.tgo_attn_fwd.restype = ctypes.c_int
    lib.tgo_attn_bwd.argtypes = [_D, _D, _D, _D, _D, _I32, ctypes.c_double, ctypes.c_double, _D,
                                 _D, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                 _D, _D, _D, _D, _D, _D]
    lib.tgo_attn_bwd.restype = ctypes.c_int
    lib.tgo_round_bf16.argtypes = [ctypes.c_double]
    lib.tgo_gate_score_heads.argtypes = [_D, _D, _D, _i64, _i64, _i64, _i64, _D]
    lib.tgo_gate_score_clone.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64, _i64, _D]
    lib.tgo_rms_norm.argtypes = [_D, _D, ctypes.c_double, _i64, _i64, _D]
    lib.tgo_gate_score_ln.argtypes = [_D, _D, ctypes.c_double, _D, _D, _U8, _i64, _i64, _i64, _D, _D]
    lib.tgo_score_normalize.argtypes = [_D, _U8, _i64, _i64, ctypes.c_double, _D]
    lib.tgo_gate_softmax.argtypes = [_D, _I32, _i64, _i64, _D]
    lib.tgo_gate_softmax_bwd.argtypes = [_D, _D, _i64, _i64, _D]
    lib.tgo_round_bf16.restype = ctypes.c_double
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (accepts NumPy or CPU torch)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use (OMP_NUM_THREADS, else the CPUs this process may run on)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


def gate_score(hidden, w1, w2, forced=None):
    """Scores and gates (DeepDive section 3.1, Eq. 3 first part; gate g = sigmoid(s), g = 1 if forced).

    hidden [T, d]; w1 [d_ff, d]; w2 [d_ff]; forced [T] (nonzero = non-prunable) or None.
    Returns (scores float64 [T], gates float64 [T]).
    """
    lib = _load()
    h = _f64(hidden)
    W1 = _f64(w1)
    W2 = _f64(w2).reshape(-1)
    T, d = h.shape
    d_ff = W1.shape[0]
    assert W1.shape == (d_ff, d) and W2.shape == (d_ff,)
    f = None if forced is None else np.ascontiguousarray(np.asarray(forced, dtype=np.uint8).reshape(T))
    s = np.empty(T, np.float64)
    g = np.empty(T, np.float64)
    lib.tgo_gate_score(_ptr(h, _D), _ptr(W1, _D), _ptr(W2, _D), _ptr(f, _U8), T, d, d_ff,
                       _ptr(s, _D), _ptr(g, _D))
    return s, g


def gate_score_ln(hidden, ln_w, eps, w1, w2, forced=None):
    """Scores and gates of the LN2-normalised residual (DeepDive section 2 Eq. 1, section 3.1 Eq. 3).

    hidden [T, d] raw residual; ln_w [d] RMSNorm weight or None (= 1); eps >= 0.
    Returns (scores float64 [T], gates float64 [T]) as gate_score on the normalised rows.
    """
    lib = _load()
    h = _f64(hidden)
    W1 = _f64(w1)
    W2 = _f64(w2).reshape(-1)
    T, d = h.shape
    d_ff = W1.shape[0]
    lw = None if ln_w is None else _f64(ln_w).reshape(d)
    f = None if forced is None else np.ascontiguousarray(np.asarray(forced, dtype=np.uint8).reshape(T))
    s = np.empty(T, np.float64)
    g = np.empty(T, np.float64)
    lib.tgo_gate_score_ln(_ptr(h, _D), _ptr(lw, _D), float(eps), _ptr(W1, _D), _ptr(W2, _D), _ptr(f, _U8), T, d,
                          d_ff, _ptr(s, _D), _ptr(g, _D))
    return s, g


def rms_norm(hidden, ln_w, eps):
    """LN2 as RMSNorm (DeepDive section 2 Eq. 1): rows divided by their root mean square (+eps), times w."""
    lib = _load()
    h = _f64(hidden)
    T, d = h.shape
    lw = None if ln_w is None else _f64(ln_w).reshape(d)
    out = np.empty((T, d), np.float64)
    lib.tgo_rms_norm(_ptr(h, _D), _ptr(lw, _D), float(eps), T, d, _ptr(out, _D))
    return out


def gate_score_heads(hidden, w1, w2):
    """Per-head scores (DeepDive section 3.4: per-head bias, uniform head aggregation for selection).

    hidden [T, d] (already normalised); w1 [d_ff, d]; w2 [H, d_ff].  Returns float64 [H, T].
    """
    lib = _load()
    h = _f64(hidden)
    W1 = _f64(w1)
    W2 = np.ascontiguousarray(_f64(w2).reshape(-1, W1.shape[0]))
    T, d = h.shape
    d_ff = W1.shape[0]
    H = W2.shape[0]
    out = np.empty((H, T), np.float64)
    lib.tgo_gate_score_heads(_ptr(h, _D), _ptr(W1, _D), _ptr(W2, _D), T, d, d_ff, H, _ptr(out, _D))
    return out


def gate_score_clone(hidden, w_gate, w_up, w_down, w_head):
    """Raw scores of the scoring branch cloned from the gate layer's MLP (DeepDive section 3.4 and the
    section 3 pipeline figure), read as the gated (SwiGLU) MLP followed by a head projection:
    b~^h = w_head[h] . (w_down (SiLU(w_gate a~) * (w_up a~))).

    hidden [T, d] (already normalised); w_gate, w_up [d_i, d]; w_down [d, d_i]; w_head [H, d] (or [d]
    for one head).  Returns float64 [H, T].
    """
    lib = _load()
    h = _f64(hidden)
    Wg, Wu, Wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    T, d = h.shape
    d_i = Wg.shape[0]
    if Wg.shape != (d_i, d) or Wu.shape != (d_i, d) or Wd.shape != (d, d_i):
        raise ValueError("w_gate, w_up must be [d_i, d] and w_down [d, d_i]")
    P = np.ascontiguousarray(_f64(w_head).reshape(-1, d))
    H = P.shape[0]
    out = np.empty((H, T), np.float64)
    lib.tgo_gate_score_clone(_ptr(h, _D), _ptr(Wg, _D), _ptr(Wu, _D), _ptr(Wd, _D), _ptr(P, _D), T, d, d_i, H,
                             _ptr(out, _D))
    return out


def aggregate_heads(b):
    """Uniform aggregation over heads for selection (DeepDive section 3.4): the mean over axis -2 of
    [..., H, N] normalised per-head scores."""
    x = _f64(b)
    return x.sum(axis=-2) / x.shape[-2]


def score_normalize(scores, forced, eps):
    """Sequence RMS normalisation over the prunable positions, 0 on forced ones (DeepDive section 3.1 Eq. 3).

    scores [B, N] or [N]; forced of the same shape (nonzero = non-prunable) or None.  Returns float64, same shape.
    """
    lib = _load()
    s = _f64(scores)
    shp = s.shape
    s2 = s.reshape(-1, shp[-1])
    B, N = s2.shape
    f = None if forced is None else np.ascontiguousarray(np.asarray(forced, dtype=np.uint8).reshape(B, N))
    out = np.empty((B, N), np.float64)
    lib.tgo_score_normalize(_ptr(np.ascontiguousarray(s2), _D), _ptr(f, _U8), B, N, float(eps), _ptr(out, _D))
    return out.reshape(shp)


def gate_softmax(bsc, kept=None):
    """Gate values as the softmax of the normalised scores over the kept set (DeepDive section 3.2 Eq. 5).

    bsc [B, M] or [M]; kept int32 of the same shape or None (negative index = padding, g = 0).
    """
    lib = _load()
    x = _f64(bsc)
    shp = x.shape
    x2 = np.ascontiguousarray(x.reshape(-1, shp[-1]))
    B, M = x2.shape
    k = None if kept is None else np.ascontiguousarray(np.asarray(kept, dtype=np.int32).reshape(B, M))
    g = np.empty((B, M), np.float64)
    lib.tgo_gate_softmax(_ptr(x2, _D), _ptr(k, _I32), B, M, _ptr(g, _D))
    return g.reshape(shp)


def gate_softmax_bwd(g, dg):
    """db = g (dg - sum g dg) per row: the backward of gate_softmax."""
    lib = _load()
    G = _f64(g)
    shp = G.shape
    G2 = np.ascontiguousarray(G.reshape(-1, shp[-1]))
    dG = np.ascontiguousarray(_f64(dg).reshape(G2.shape))
    B, M = G2.shape
    out = np.empty((B, M), np.float64)
    lib.tgo_gate_softmax_bwd(_ptr(G2, _D), _ptr(dG, _D), B, M, _ptr(out, _D))
    return out.reshape(shp)


def select_topk(scores, forced, K, M=None):
    """Kept indices, ascending (DeepDive section 3.1 Eq. 4 and section 3.4).

    scores float32 [B, N] or [N]; forced uint8 of the same shape or None; K >= 0.
    M: row length to write (defaults to each row's true count, which must then be
    equal across rows).  Returns (kept int32 [B, M] padded with -1, counts int64 [B]).
    """
    lib = _load()
    sc = np.asarray(scores, dtype=np.float32)
    squeeze = sc.ndim == 1
    sc = np.ascontiguousarray(sc.reshape(1, -1) if squeeze else sc)
    B, N = sc.shape
    fo = None
    if forced is not None:
        fo = np.ascontiguousarray(np.asarray(forced, dtype=np.uint8).reshape(B, N))
    if M is None:
        nF = 0 if fo is None else (fo != 0).sum(axis=1)
        counts = np.asarray(nF + np.minimum(K, N - np.asarray(nF)), dtype=np.int64).reshape(-1)
        if counts.size > 1:
            assert np.all(counts == counts[0]), "rows differ in kept count; pass M"
        M = int(counts[0]) if counts.size else 0
    kept = np.empty((B, max(M, 0)), np.int32)
    counts = np.empty(B, np.int64)
    for b in range(B):
        row = np.ascontiguousarray(sc[b])
        fr = None if fo is None else np.ascontiguousarray(fo[b])
        out = np.empty(max(M, 1), np.int32)
        counts[b] = lib.tgo_select_topk(_ptr(row, _F), _ptr(fr, _U8), N, int(K), M, _ptr(out, _I32))
        kept[b] = out[:M]
    if squeeze:
        return kept[0], counts[0]
    return kept, counts


def compact(hidden, pos, gates, kept):
    """Gather of kept rows, positions and gates (DeepDive section 3.4).

    hidden: NumPy array [B, N, ...] of any dtype (raw bytes are copied); pos int32
    [B, N] or None (= index); gates float32 [B, N] or None; kept int32 [B, M].
    Returns (hidden_out [B, M, ...], pos_out int32 [B, M], gates_out float32 [B, M] or None).
    """
    lib = _load()
    h = np.ascontiguousarray(hidden)
    B, N = h.shape[0], h.shape[1]
    kp = np.ascontiguousarray(np.asarray(kept, dtype=np.int32))
    M = kp.shape[1]
    row_bytes = int(np.prod(h.shape[2:], dtype=np.int64)) * h.itemsize
    out = np.empty((B, M) + h.shape[2:], h.dtype)
    pos_out = np.empty((B, M), np.int32)
    g_out = None if gates is None else np.empty((B, M), np.float32)
    for b in range(B):
        src = np.ascontiguousarray(h[b]).view(np.uint8).reshape(-1)
        dst = np.empty(M * row_bytes, np.uint8)
        p = None if pos is None else np.ascontiguousarray(np.asarray(pos, dtype=np.int32)[b])
        g = None if gates is None else np.ascontiguousarray(np.asarray(gates, dtype=np.float32)[b])
        po = np.empty(M, np.int32)
        go = None if gates is None else np.empty(M, np.float32)
        lib.tgo_compact(_ptr(src, _U8), _ptr(p, _I32), _ptr(g, _F), _ptr(np.ascontiguousarray(kp[b]), _I32),
                        N, M, row_bytes, _ptr(dst, _U8), _ptr(po, _I32), _ptr(go, _F))
        out[b] = dst.view(h.dtype).reshape((M,) + h.shape[2:])
        pos_out[b] = po
        if g_out is not None:
            g_out[b] = go
    return out, pos_out, g_out


def attn_fwd(q, k, v, g, gamma, pos=None, theta=1e6, tau=1.0, round_bf16=False, rows=None, sigma=None):
    """Token-gated causal attention forward (DeepDive section 2 Eq. 2, section 3.2 Eqs. 5-6;
    Summary Figure 1(c)).  With sigma [Hq] the operative rule of section 3.2 Eq. 8: the whole
    logit scaled by tau_ih = softplus(sigma_h) ln(i+1) / ln max(2, pos_i+1) (Eq. 7).

    q [B, M, Hq, D]; k, v [B, M, Hkv, D]; g [B, M] (one gate per key) or [B, Hq, M] (per-head gates,
    the per-head bias of section 3.4's released-code walkthrough); gamma [Hq]; pos int32 [B, M] or None.
    round_bf16: round the rotated q, k to bf16 before the product (as the tensor cores see them).
    rows: optional flattened query rows (b*M + i) to compute; the others come back NaN.
    Returns (o float64 [B, M, Hq, D], lse float64 [B, Hq, M]).
    """
    lib = _load()
    Q, Kt, V = _f64(q), _f64(k), _f64(v)
    B, M, Hq, D = Q.shape
    Hkv = Kt.shape[2]
    G = _f64(g)
    per_head = G.ndim == 3
    G = np.ascontiguousarray(G.reshape((B, Hq, M) if per_head else (B, M)))
    gm = _f64(gamma).reshape(Hq)
    p = None if pos is None else np.ascontiguousarray(np.asarray(pos, dtype=np.int32).reshape(B, M))
    o = np.full((B, M, Hq, D), np.nan)
    lse = np.full((B, Hq, M), np.nan)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    sg = None if sigma is None else _f64(sigma).reshape(Hq)
    rc = lib.tgo_attn_fwd(_ptr(Q, _D), _ptr(Kt, _D), _ptr(V, _D), _ptr(G, _D), _ptr(gm, _D), _ptr(p, _I32),
                          float(theta), float(tau), _ptr(sg, _D), B, M, Hq, Hkv, D, int(bool(round_bf16)),
                          _ptr(r, _I64), 0 if r is None else r.size, int(per_head), _ptr(o, _D), _ptr(lse, _D))
    if rc != 0:
        raise ValueError("oracle attn_fwd: bad arguments")
    return o, lse


def attn_bwd(q, k, v, g, gamma, dout, pos=None, theta=1e6, tau=1.0, round_bf16=False, sigma=None):
    """Gradients of the token-gated attention (DeepDive section 3.1 last paragraph and section 3.2:
    the task gradient reaches the scores through the attention bias).

    Returns (dq [B,M,Hq,D], dk [B,M,Hkv,D], dv [B,M,Hkv,D], dg (the shape of g: [B,M] or per-head
    [B,Hq,M]), dgamma [Hq]), all float64, followed by dsigma [Hq] when sigma is given (Eq. 7/8).
    """
    lib = _load()
    Q, Kt, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, M, Hq, D = Q.shape
    Hkv = Kt.shape[2]
    G = _f64(g)
    per_head = G.ndim == 3
    G = np.ascontiguousarray(G.reshape((B, Hq, M) if per_head else (B, M)))
    gm = _f64(gamma).reshape(Hq)
    p = None if pos is None else np.ascontiguousarray(np.asarray(pos, dtype=np.int32).reshape(B, M))
    dq = np.empty((B, M, Hq, D))
    dk = np.empty((B, M, Hkv, D))
    dv = np.empty((B, M, Hkv, D))
    dg = np.empty(G.shape)
    dgamma = np.empty(Hq)
    sg = None if sigma is None else _f64(sigma).reshape(Hq)
    dsigma = None if sigma is None else np.empty(Hq)
    rc = lib.tgo_attn_bwd(_ptr(Q, _D), _ptr(Kt, _D), _ptr(V, _D), _ptr(G, _D), _ptr(gm, _D), _ptr(p, _I32),
                          float(theta), float(tau), _ptr(sg, _D), _ptr(dO, _D), B, M, Hq, Hkv, D,
                          int(bool(round_bf16)), int(per_head), _ptr(dq, _D), _ptr(dk, _D), _ptr(dv, _D),
                          _ptr(dg, _D),
                          _ptr(dgamma, _D), _ptr(dsigma, _D))
    if rc != 0:
        raise ValueError("oracle attn_bwd: bad arguments")
    if sigma is None:
        return dq, dk, dv, dg, dgamma
    return dq, dk, dv, dg, dgamma, dsigma


def _runs(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0)
    return cu


def attn_fwd_varlen(q, k, v, g, gamma, cu_seqlens, pos=None, theta=1e6, tau=1.0, round_bf16=False, sigma=None):
    """Token-gated attention over packed sequences (the training path packs both budgets in one call:
    DeepDive section 3.3): sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends
    causally within itself only, exactly as attn_fwd on that sequence alone (row index i and the
    temperature's m_i = i + 1 count from the sequence start).

    q [T, Hq, D]; k, v [T, Hkv, D]; g [T]; pos int32 [T] or None.  Returns (o [T, Hq, D], lse [Hq * T]),
    lse holding sequence s's [Hq, M_s] block at offset Hq * cu_seqlens[s].
    """
    cu = _runs(cu_seqlens)
    Q, K, V = _f64(q), _f64(k), _f64(v)
    T, Hq, D = Q.shape
    o = np.full((T, Hq, D), np.nan)
    lse = np.full(Hq * T, np.nan)
    G = _f64(g).reshape(T)
    P = None if pos is None else np.asarray(pos, dtype=np.int32).reshape(T)
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        os_, ls = attn_fwd(Q[None, a:e], K[None, a:e], V[None, a:e], G[None, a:e], gamma,
                           pos=None if P is None else P[None, a:e], theta=theta, tau=tau, round_bf16=round_bf16,
                           sigma=sigma)
        o[a:e] = os_[0]
        lse[Hq * a:Hq * e] = ls.reshape(-1)
    return o, lse


def attn_bwd_varlen(q, k, v, g, gamma, dout, cu_seqlens, pos=None, theta=1e6, tau=1.0, round_bf16=False,
                    sigma=None):
    """Gradients of attn_fwd_varlen: dq, dk, dv, dg per token; dgamma (and dsigma) summed over sequences."""
    cu = _runs(cu_seqlens)
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    T, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = _f64(g).reshape(T)
    P = None if pos is None else np.asarray(pos, dtype=np.int32).reshape(T)
    dq, dk, dv, dg = np.zeros((T, Hq, D)), np.zeros((T, Hkv, D)), np.zeros((T, Hkv, D)), np.zeros(T)
    dgamma, dsigma = np.zeros(Hq), np.zeros(Hq)
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        r = attn_bwd(Q[None, a:e], K[None, a:e], V[None, a:e], G[None, a:e], gamma, dO[None, a:e],
                     pos=None if P is None else P[None, a:e], theta=theta, tau=tau, round_bf16=round_bf16,
                     sigma=sigma)
        dq[a:e], dk[a:e], dv[a:e], dg[a:e] = r[0][0], r[1][0], r[2][0], r[3][0]
        dgamma += r[4]
        if sigma is not None:
            dsigma += r[5]
    if sigma is None:
        return dq, dk, dv, dg, dgamma
    return dq, dk, dv, dg, dgamma, dsigma


def round_bf16(x: float) -> float:
    """The oracle's fp64 -> bf16 round-to-nearest-even (exposed for its pin tests)."""
    return _load().tgo_round_bf16(float(x))

"""libtokengate: the TokenGate gate-layer hot path on AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/tokengate.h``.  Each ``tg_*``
function here has the name of the C entry point it calls; it only marshals
torch device tensors into pointers and sizes, passes the current HIP stream and
raises on a non-OK status.  Every step of the computation runs in the HIP
kernels of libtokengate.so; there is no fallback: if the library is not built
the calls raise.

Stages (TokenGate deep dive, "TokenGate: Learnable Token Pruning for Fast,
Memory-Efficient LLM Prefill", sections 3.1-3.4):
  tg_gate_score      scoring MLP -> raw scores and gate values
                     (tg_gate_pack_w1 + tg_gate_score_packed: the same with W1
                     rewritten once in matrix-core fragment order)
  tg_select_topk     top-K prunable tokens plus every forced token, ascending
  tg_compact         gather of kept hidden states, positions and gates
  tg_gated_attn_fwd  causal attention with the per-key bias gamma_h * ln g_j and,
                     optionally, the pruning-ratio temperature (section 3.2, Eq. 7/8)
  tg_gated_attn_bwd  its gradients (dq, dk, dv, dg, dgamma, and dsigma)
The rest of the scoring definition (section 2 Eq. 1, section 3.1 Eq. 3, section 3.2 Eq. 5):
  tg_gate_score_ln     the scorer on the raw residual with the RMSNorm (LN2) in front
  tg_score_normalize   sequence RMS normalisation over the prunable positions, 0 on forced ones
  tg_gate_softmax      gate values as the softmax of the normalised scores over the kept set
  tg_gate_softmax_bwd  its backward
Per-head scores, uniform head aggregation, per-head gates (section 3.4):
  tg_gate_score_heads, tg_score_normalize_heads, tg_aggregate_heads, tg_gather_heads,
  tg_gate_softmax_heads, tg_gated_attn_fwd_headgates / tg_gated_attn_bwd_headgates
The scoring branch cloned from the gate layer's MLP (section 3.4):
  tg_gate_score_clone
Packed variable-length sequences (section 3.3: both budgets in one call):
  tg_gated_attn_fwd_varlen / tg_gated_attn_bwd_varlen
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "TokenGateError", "library_path", "load", "tg_version", "tg_kept_count", "tg_gate_score",
    "tg_gate_score_workspace_size", "tg_gate_pack_w1", "tg_gate_score_packed", "gate_workspace",
    "tg_select_topk", "tg_compact", "tg_gated_attn_fwd", "tg_gated_attn_bwd",
    "tg_select_topk_workspace_size", "tg_gated_attn_workspace_size", "gate_layer_forward", "attn_workspace",
    "select_workspace", "tg_select_topk_noalloc",
    "tg_gate_score_ln", "tg_score_normalize", "tg_gate_softmax", "tg_gate_softmax_bwd",
    "tg_gated_attn_varlen_workspace_size", "tg_gated_attn_fwd_varlen", "tg_gated_attn_bwd_varlen",
    "attn_varlen_workspace", "tg_gate_score_heads", "tg_score_normalize_heads", "tg_aggregate_heads",
    "tg_gather_heads", "tg_gate_softmax_heads", "tg_gated_attn_fwd_headgates", "tg_gated_attn_bwd_headgates",
    "tg_gate_score_clone", "tg_gate_score_clone_workspace_size",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtokengate.so"
_lib = None

TG_OK, TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_HIP = range(5)
TG_F32, TG_BF16 = 0, 1


class TokenGateError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load libtokengate.so (built in-tree by learned_token_pruning_gatescore_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m learned_token_pruning_gatescore_amd.build`")
    lib = ctypes.CDLL(path)
    P, i64, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    c_int = ctypes.c_int
    lib.tg_version.restype = c_int
    lib.tg_version.argtypes = []
    lib.tg_status_string.restype = ctypes.c_char_p
    lib.tg_status_string.argtypes = [c_int]
    lib.tg_last_error.restype = ctypes.c_char_p
    lib.tg_last_error.argtypes = []
    lib.tg_kept_count.restype = i64
    lib.tg_kept_count.argtypes = [i64, i64, i64]
    lib.tg_gate_score.restype = c_int
    lib.tg_gate_score.argtypes = [P, P, P, P, i64, i64, i64, i64, c_int, P, P, P, sz, P]
    lib.tg_gate_score_workspace_size.restype = sz
    lib.tg_gate_score_workspace_size.argtypes = [i64, i64, c_int]
    lib.tg_gate_pack_w1.restype = c_int
    lib.tg_gate_pack_w1.argtypes = [P, i64, i64, c_int, P, sz, P]
    lib.tg_gate_score_packed.restype = c_int
    lib.tg_gate_score_packed.argtypes = [P, P, P, P, i64, i64, i64, i64, c_int, P, P, P]
    lib.tg_select_topk_workspace_size.restype = sz
    lib.tg_select_topk_workspace_size.argtypes = [i64, i64]
    lib.tg_select_topk.restype = c_int
    lib.tg_select_topk.argtypes = [P, P, i64, i64, i64, i64, P, P, P, sz, P]
    lib.tg_select_topk_noalloc.restype = c_int
    lib.tg_select_topk_noalloc.argtypes = [P, P, i64, i64, i64, i64, P, P, P]
    lib.tg_compact.restype = c_int
    lib.tg_compact.argtypes = [P, P, P, P, i64, i64, i64, i64, c_int, P, P, P, P]
    lib.tg_gate_score_ln.restype = c_int
    lib.tg_gate_score_ln.argtypes = [P, P, f32, P, P, P, i64, i64, i64, i64, c_int, P, P, P, sz, P]
    lib.tg_score_normalize.restype = c_int
    lib.tg_score_normalize.argtypes = [P, P, i64, i64, f32, P, P]
    lib.tg_gate_softmax.restype = c_int
    lib.tg_gate_softmax.argtypes = [P, P, i64, i64, P, P]
    lib.tg_gate_softmax_bwd.restype = c_int
    lib.tg_gate_softmax_bwd.argtypes = [P, P, i64, i64, P, P]
    lib.tg_gate_score_heads.restype = c_int
    lib.tg_gate_score_heads.argtypes = [P, c_int, P, f32, P, P, i64, i64, i64, i64, i64, c_int, P, P, sz, P]
    lib.tg_gate_score_clone_workspace_size.restype = sz
    lib.tg_gate_score_clone_workspace_size.argtypes = [i64, i64, i64, c_int]
    lib.tg_gate_score_clone.restype = c_int
    lib.tg_gate_score_clone.argtypes = [P, c_int, P, f32, P, P, P, P, i64, i64, i64, i64, i64, c_int, P, P, sz, P]
    lib.tg_score_normalize_heads.restype = c_int
    lib.tg_score_normalize_heads.argtypes = [P, P, i64, i64, i64, f32, P, P]
    lib.tg_aggregate_heads.restype = c_int
    lib.tg_aggregate_heads.argtypes = [P, i64, i64, i64, P, P]
    lib.tg_gather_heads.restype = c_int
    lib.tg_gather_heads.argtypes = [P, P, i64, i64, i64, i64, P, P]
    lib.tg_gate_softmax_heads.restype = c_int
    lib.tg_gate_softmax_heads.argtypes = [P, P, i64, i64, i64, P, P]
    lib.tg_gated_attn_varlen_workspace_size.restype = sz
    lib.tg_gated_attn_varlen_workspace_size.argtypes = [P, i64, i64, i64, i64, c_int]
    lib.tg_gated_attn_fwd_varlen.restype = c_int
    lib.tg_gated_attn_fwd_varlen.argtypes = [P, P, P, P, P, P, f32, f32, P, P, i64, i64, i64, i64, c_int, P, P, P,
                                             P, sz, P]
    lib.tg_gated_attn_bwd_varlen.restype = c_int
    lib.tg_gated_attn_bwd_varlen.argtypes = [P, P, P, P, P, P, f32, f32, P, P, P, P, P, P, i64, i64, i64, i64,
                                             c_int, P, P, P, P, P, P, P, sz, P]
    lib.tg_gated_attn_workspace_size.restype = sz
    lib.tg_gated_attn_workspace_size.argtypes = [i64, i64, i64, i64, i64, c_int]
    lib.tg_gated_attn_fwd.restype = c_int
    lib.tg_gated_attn_fwd.argtypes = [P, P, P, P, P, P, f32, f32, P, i64, i64, i64, i64, i64, c_int, P, P, P, P,
                                      sz, P]
    lib.tg_gated_attn_bwd.restype = c_int
    lib.tg_gated_attn_bwd.argtypes = [P, P, P, P, P, P, f32, f32, P, P, P, P, P, i64, i64, i64, i64, i64, c_int,
                                      P, P, P, P, P, P, P, sz, P]
    lib.tg_gated_attn_fwd_headgates.restype = c_int
    lib.tg_gated_attn_fwd_headgates.argtypes = lib.tg_gated_attn_fwd.argtypes
    lib.tg_gated_attn_bwd_headgates.restype = c_int
    lib.tg_gated_attn_bwd_headgates.argtypes = lib.tg_gated_attn_bwd.argtypes
    _lib = lib
    return lib


def _check(status: int):
    if status != TG_OK:
        lib = load()
        raise TokenGateError(status, f"{lib.tg_status_string(status).decode()}: {lib.tg_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    """The HIP stream handle: a torch Stream, a raw handle, or None for torch's current stream."""
    if stream is not None:
        return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return TG_BF16
    if t.dtype == torch.float32:
        return TG_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def tg_version() -> int:
    return load().tg_version()


def tg_kept_count(N: int, n_forced: int, K: int) -> int:
    return load().tg_kept_count(N, n_forced, K)


def tg_select_topk_workspace_size(B: int, N: int) -> int:
    return load().tg_select_topk_workspace_size(B, N)


def tg_gated_attn_workspace_size(B: int, M: int, Hq: int, Hkv: int, D: int, bwd: bool) -> int:
    return load().tg_gated_attn_workspace_size(B, M, Hq, Hkv, D, int(bool(bwd)))


def tg_gate_score_workspace_size(d: int, d_ff: int, bf16: bool) -> int:
    return load().tg_gate_score_workspace_size(d, d_ff, TG_BF16 if bf16 else TG_F32)


def gate_workspace(d, d_ff, dtype, device):
    """A workspace tensor of the size tg_gate_score needs (also the packed-W1 buffer)."""
    import torch

    n = tg_gate_score_workspace_size(d, d_ff, dtype == torch.bfloat16)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def tg_gate_score(hidden, w1, w2, forced_keep, scores, gates=None, ws=None, stream=None):
    """hidden [B, N, d], w1 [d_ff, d], w2 [d_ff] (bf16 or fp32); forced_keep u8 [B, N] or None;
    writes scores (and gates) f32 [B, N].  ws: workspace (allocated here when None)."""
    _contig(hidden, w1, w2, forced_keep, scores, gates, ws)
    B, N, d = hidden.shape
    d_ff = w1.shape[0]
    if ws is None:
        ws = gate_workspace(d, d_ff, hidden.dtype, hidden.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().tg_gate_score(_ptr(hidden), _ptr(w1), _ptr(w2), _ptr(forced_keep), B, N, d, d_ff, _dt(hidden),
                                _ptr(scores), _ptr(gates), _ptr(ws), ws_bytes, _stream(stream)))


def tg_gate_pack_w1(w1, w1_packed, stream=None):
    """w1 [d_ff, d] bf16 -> w1_packed (uint8 tensor of tg_gate_score_workspace_size bytes)."""
    _contig(w1, w1_packed)
    d_ff, d = w1.shape
    nbytes = w1_packed.numel() * w1_packed.element_size()
    _check(load().tg_gate_pack_w1(_ptr(w1), d, d_ff, _dt(w1), _ptr(w1_packed), nbytes, _stream(stream)))


def tg_gate_score_packed(hidden, w1_packed, d_ff, w2, forced_keep, scores, gates=None, stream=None):
    """tg_gate_score from a W1 copy made by tg_gate_pack_w1 (bf16 only)."""
    _contig(hidden, w1_packed, w2, forced_keep, scores, gates)
    B, N, d = hidden.shape
    _check(load().tg_gate_score_packed(_ptr(hidden), _ptr(w1_packed), _ptr(w2), _ptr(forced_keep), B, N, d,
                                       int(d_ff), _dt(hidden), _ptr(scores), _ptr(gates), _stream(stream)))


def tg_gate_score_ln(hidden, ln_w, ln_eps, w1, w2, forced_keep, scores, gates=None, ws=None, stream=None):
    """tg_gate_score on the raw residual [B, N, d] with the RMSNorm (weight ln_w [d] or None, eps) in front."""
    _contig(hidden, ln_w, w1, w2, forced_keep, scores, gates, ws)
    B, N, d = hidden.shape
    d_ff = w1.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().tg_gate_score_ln(_ptr(hidden), _ptr(ln_w), float(ln_eps), _ptr(w1), _ptr(w2), _ptr(forced_keep),
                                   B, N, d, d_ff, _dt(hidden), _ptr(scores), _ptr(gates), _ptr(ws), ws_bytes,
                                   _stream(stream)))


def tg_score_normalize(scores, forced_keep, eps, out, stream=None):
    """out [B, N] = scores / their RMS over the prunable positions (+eps), 0 on forced ones (out may be scores)."""
    _contig(scores, forced_keep, out)
    B, N = scores.shape
    _check(load().tg_score_normalize(_ptr(scores), _ptr(forced_keep), B, N, float(eps), _ptr(out), _stream(stream)))


def tg_gate_softmax(b, kept_idx, g, stream=None):
    """g [B, M] = softmax of b [B, M] over each row's kept entries (kept_idx < 0: padding, g = 0)."""
    _contig(b, kept_idx, g)
    B, M = b.shape
    _check(load().tg_gate_softmax(_ptr(b), _ptr(kept_idx), B, M, _ptr(g), _stream(stream)))


def tg_gate_softmax_bwd(g, dg, db, stream=None):
    """db = g (dg - sum g dg) per row."""
    _contig(g, dg, db)
    B, M = g.shape
    _check(load().tg_gate_softmax_bwd(_ptr(g), _ptr(dg), B, M, _ptr(db), _stream(stream)))


def select_workspace(B, N, device):
    """A workspace tensor of the size tg_select_topk needs (256-byte aligned by the allocator)."""
    import torch

    return torch.empty(max(tg_select_topk_workspace_size(B, N), 1), dtype=torch.uint8, device=device)


def tg_select_topk(scores, forced_keep, K, n_forced, kept_idx, kept_count=None, ws=None, stream=None):
    """scores f32 [B, N]; forced_keep u8 [B, N] or None; writes kept_idx i32 [B, M] (M = tg_kept_count).
    ws: the workspace (select_workspace); allocated here when None."""
    _contig(scores, forced_keep, kept_idx, kept_count, ws)
    B, N = scores.shape
    if ws is None:
        ws = select_workspace(B, N, scores.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().tg_select_topk(_ptr(scores), _ptr(forced_keep), B, N, int(K), int(n_forced), _ptr(kept_idx),
                                 _ptr(kept_count), _ptr(ws), ws_bytes, _stream(stream)))


def tg_select_topk_noalloc(scores, forced_keep, K, n_forced, kept_idx, kept_count=None, stream=None):
    """tg_select_topk with the library's own device scratch (no workspace, nothing allocated)."""
    _contig(scores, forced_keep, kept_idx, kept_count)
    B, N = scores.shape
    _check(load().tg_select_topk_noalloc(_ptr(scores), _ptr(forced_keep), B, N, int(K), int(n_forced),
                                         _ptr(kept_idx), _ptr(kept_count), _stream(stream)))


def tg_compact(hidden, pos, gates, kept_idx, hidden_out=None, pos_out=None, gates_out=None, stream=None):
    """hidden [B, N, d]; pos i32 [B, N] or None; gates f32 [B, N] or None; kept_idx i32 [B, M]."""
    _contig(hidden, pos, gates, kept_idx, hidden_out, pos_out, gates_out)
    B, N, d = hidden.shape
    M = kept_idx.shape[1]
    _check(load().tg_compact(_ptr(hidden), _ptr(pos), _ptr(gates), _ptr(kept_idx), B, N, M, d, _dt(hidden),
                             _ptr(hidden_out), _ptr(pos_out), _ptr(gates_out), _stream(stream)))


def attn_workspace(B, M, Hq, Hkv, D, bwd, device):
    """A workspace tensor of the size the attention calls need (256-byte aligned by torch's allocator)."""
    import torch

    n = tg_gated_attn_workspace_size(B, M, Hq, Hkv, D, bwd)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def tg_gated_attn_fwd(q, k, v, g, gamma, pos, rope_theta, tau, o, lse=None, ws=None, stream=None, *, sigma=None,
                      o_lo=None):
    """q [B, M, Hq, D], k, v [B, M, Hkv, D] (bf16 or fp32); g f32 [B, M]; gamma f32 [Hq];
    pos i32 [B, M] or None; sigma f32 [Hq] or None (the pruning-ratio temperature);
    writes o [B, M, Hq, D], lse f32 [B, Hq, M] and (bf16, if given) o_lo [B, M, Hq, D],
    the residual of o's rounding."""
    _contig(q, k, v, g, gamma, pos, o, lse, ws, sigma, o_lo)
    B, M, Hq, D = q.shape
    Hkv = k.shape[2]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos), float(rope_theta),
                                    float(tau), _ptr(sigma), B, M, Hq, Hkv, D, _dt(q), _ptr(o), _ptr(lse),
                                    _ptr(o_lo), _ptr(ws), ws_bytes, _stream(stream)))


def tg_gated_attn_bwd(q, k, v, g, gamma, pos, rope_theta, tau, lse, dout, dq, dk, dv, dg, dgamma, ws,
                      stream=None, *, sigma=None, dsigma=None, o=None, o_lo=None):
    """Gradients of tg_gated_attn_fwd; dq, dk, dv, dg, dgamma (and dsigma f32 [Hq], given with
    sigma) are f32 outputs, fully overwritten.  o and o_lo (the forward's, bf16, together)
    give the row terms D_i without a second pass over the keys."""
    _contig(q, k, v, g, gamma, pos, lse, dout, dq, dk, dv, dg, dgamma, ws, sigma, dsigma, o, o_lo)
    B, M, Hq, D = q.shape
    Hkv = k.shape[2]
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos), float(rope_theta),
                                    float(tau), _ptr(sigma), _ptr(lse), _ptr(dout), _ptr(o), _ptr(o_lo), B, M, Hq,
                                    Hkv, D, _dt(q), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dgamma),
                                    _ptr(dsigma), _ptr(ws), ws_bytes, _stream(stream)))


def tg_gate_score_heads(hidden, w1, w2, scores, ws=None, ln_w=None, ln_eps=None, stream=None):
    """Per-head scores [B, H, N] of hidden [B, N, d] (RMSNorm in front when ln_eps is given); w2 [H, d_ff]."""
    _contig(hidden, w1, w2, scores, ws, ln_w)
    B, N, d = hidden.shape
    d_ff = w1.shape[0]
    H = w2.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    ln = ln_eps is not None
    _check(load().tg_gate_score_heads(_ptr(hidden), int(ln), _ptr(ln_w), float(ln_eps if ln else 0.0), _ptr(w1),
                                      _ptr(w2), B, N, d, d_ff, H, _dt(hidden), _ptr(scores), _ptr(ws), ws_bytes,
                                      _stream(stream)))


def tg_gate_score_clone_workspace_size(d, d_i, H, bf16=True):
    return load().tg_gate_score_clone_workspace_size(d, d_i, H, TG_BF16 if bf16 else TG_F32)


def tg_gate_score_clone(hidden, w_gate, w_up, w_down, w_head, scores, ws=None, ln_w=None, ln_eps=None, stream=None):
    """Scores [B, H, N] of the branch cloned from the gate layer's MLP: hidden [B, N, d]; w_gate, w_up
    [d_i, d]; w_down [d, d_i]; w_head [H, d] (RMSNorm in front when ln_eps is given).  ws: workspace
    (allocated here when None)."""
    import torch

    _contig(hidden, w_gate, w_up, w_down, w_head, scores, ws, ln_w)
    B, N, d = hidden.shape
    d_i = w_gate.shape[0]
    H = w_head.shape[0] if w_head.dim() == 2 else 1
    if ws is None:
        n = tg_gate_score_clone_workspace_size(d, d_i, H, hidden.dtype == torch.bfloat16)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=hidden.device)
    ws_bytes = ws.numel() * ws.element_size()
    ln = ln_eps is not None
    _check(load().tg_gate_score_clone(_ptr(hidden), int(ln), _ptr(ln_w), float(ln_eps if ln else 0.0), _ptr(w_gate),
                                      _ptr(w_up), _ptr(w_down), _ptr(w_head), B, N, d, d_i, H, _dt(hidden),
                                      _ptr(scores), _ptr(ws), ws_bytes, _stream(stream)))


def tg_score_normalize_heads(scores, forced_keep, eps, out, stream=None):
    _contig(scores, forced_keep, out)
    B, H, N = scores.shape
    _check(load().tg_score_normalize_heads(_ptr(scores), _ptr(forced_keep), B, H, N, float(eps), _ptr(out),
                                           _stream(stream)))


def tg_aggregate_heads(b, out, stream=None):
    _contig(b, out)
    B, H, N = b.shape
    _check(load().tg_aggregate_heads(_ptr(b), B, H, N, _ptr(out), _stream(stream)))


def tg_gather_heads(b, kept_idx, out, stream=None):
    _contig(b, kept_idx, out)
    B, H, N = b.shape
    M = kept_idx.shape[1]
    _check(load().tg_gather_heads(_ptr(b), _ptr(kept_idx), B, H, N, M, _ptr(out), _stream(stream)))


def tg_gate_softmax_heads(b, kept_idx, g, stream=None):
    _contig(b, kept_idx, g)
    B, H, M = b.shape
    _check(load().tg_gate_softmax_heads(_ptr(b), _ptr(kept_idx), B, H, M, _ptr(g), _stream(stream)))


def tg_gated_attn_fwd_headgates(q, k, v, g, gamma, pos, rope_theta, tau, o, lse=None, ws=None, stream=None, *,
                                sigma=None, o_lo=None):
    """tg_gated_attn_fwd with per-head gates g [B, Hq, M]."""
    _contig(q, k, v, g, gamma, pos, o, lse, ws, sigma, o_lo)
    B, M, Hq, D = q.shape
    Hkv = k.shape[2]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_fwd_headgates(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos),
                                              float(rope_theta), float(tau), _ptr(sigma), B, M, Hq, Hkv, D, _dt(q),
                                              _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(ws), ws_bytes, _stream(stream)))


def tg_gated_attn_bwd_headgates(q, k, v, g, gamma, pos, rope_theta, tau, lse, dout, dq, dk, dv, dg, dgamma, ws,
                                stream=None, *, sigma=None, dsigma=None, o=None, o_lo=None):
    """tg_gated_attn_bwd with per-head gates g [B, Hq, M]; dg [B, Hq, M]."""
    _contig(q, k, v, g, gamma, pos, lse, dout, dq, dk, dv, dg, dgamma, ws, sigma, dsigma, o, o_lo)
    B, M, Hq, D = q.shape
    Hkv = k.shape[2]
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_bwd_headgates(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos),
                                              float(rope_theta), float(tau), _ptr(sigma), _ptr(lse), _ptr(dout),
                                              _ptr(o), _ptr(o_lo), B, M, Hq, Hkv, D, _dt(q), _ptr(dq), _ptr(dk),
                                              _ptr(dv), _ptr(dg),
                                              _ptr(dgamma), _ptr(dsigma), _ptr(ws), ws_bytes, _stream(stream)))


def _cu_host(cu_seqlens):
    """cu_seqlens as a host int64 array (list, NumPy or CPU tensor) and the pointer to pass."""
    import numpy as np

    if hasattr(cu_seqlens, "detach"):
        if cu_seqlens.device.type != "cpu":
            raise TokenGateError(1, "cu_seqlens must be a host (CPU) array")
        cu_seqlens = cu_seqlens.detach().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
    return cu, cu.ctypes.data_as(ctypes.c_void_p)


def tg_gated_attn_varlen_workspace_size(cu_seqlens, Hq, Hkv, D, bwd) -> int:
    cu, p = _cu_host(cu_seqlens)
    return load().tg_gated_attn_varlen_workspace_size(p, cu.size - 1, Hq, Hkv, D, int(bool(bwd)))


def attn_varlen_workspace(cu_seqlens, Hq, Hkv, D, bwd, device):
    import torch

    n = tg_gated_attn_varlen_workspace_size(cu_seqlens, Hq, Hkv, D, bwd)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def tg_gated_attn_fwd_varlen(q, k, v, g, gamma, pos, rope_theta, tau, cu_seqlens, o, lse=None, ws=None,
                             stream=None, *, sigma=None, o_lo=None):
    """Packed sequences: q [T, Hq, D], k, v [T, Hkv, D]; g [T]; pos [T] or None; cu_seqlens host [nseq + 1].
    Writes o [T, Hq, D] and lse (Hq * T, sequence s's [Hq, M_s] block at Hq * cu_seqlens[s])."""
    _contig(q, k, v, g, gamma, pos, o, lse, ws, sigma, o_lo)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    cu, cp = _cu_host(cu_seqlens)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos),
                                           float(rope_theta), float(tau), _ptr(sigma), cp, cu.size - 1, Hq, Hkv, D,
                                           _dt(q), _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(ws), ws_bytes,
                                           _stream(stream)))


def tg_gated_attn_bwd_varlen(q, k, v, g, gamma, pos, rope_theta, tau, lse, dout, cu_seqlens, dq, dk, dv, dg, dgamma,
                             ws, stream=None, *, sigma=None, dsigma=None, o=None, o_lo=None):
    """Gradients of tg_gated_attn_fwd_varlen (per token; dgamma, dsigma summed over the sequences)."""
    _contig(q, k, v, g, gamma, pos, lse, dout, dq, dk, dv, dg, dgamma, ws, sigma, dsigma, o, o_lo)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    cu, cp = _cu_host(cu_seqlens)
    ws_bytes = ws.numel() * ws.element_size()
    _check(load().tg_gated_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gamma), _ptr(pos),
                                           float(rope_theta), float(tau), _ptr(sigma), _ptr(lse), _ptr(dout),
                                           _ptr(o), _ptr(o_lo), cp, cu.size - 1, Hq, Hkv, D, _dt(q), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                           _ptr(dgamma), _ptr(dsigma), _ptr(ws), ws_bytes, _stream(stream)))


def gate_layer_forward(hidden, w1, w2, forced_keep, n_forced, K, q, k, v, gamma, tau, rope_theta=1.0e6,
                       pos=None, select_scores=None, bufs=None, stream=None):
    """The four forward stages back to back on one stream (no host synchronisation).

    q/k/v are the kept tokens' projections [B, M, H, D].  select_scores, when given,
    replaces the computed scores as the ranking key (the computed scores and gates
    are still produced).  bufs: optional dict of preallocated outputs (reused across
    calls).  Returns the dict of outputs; "kept_count" [B] holds each row's true kept
    count, which differs from M when a row's forced count differs from n_forced (its
    kept_idx row is then truncated to M, or padded with -1).
    """
    import torch

    B, N, d = hidden.shape
    M = tg_kept_count(N, n_forced, K)
    dev = hidden.device
    if bufs is None:
        bufs = {}
    Hq, D = q.shape[2], q.shape[3]

    def buf(name, shape, dtype):
        t = bufs.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            t = torch.empty(shape, dtype=dtype, device=dev)
            bufs[name] = t
        return t

    scores = buf("scores", (B, N), torch.float32)
    gates = buf("gates", (B, N), torch.float32)
    kept = buf("kept_idx", (B, M), torch.int32)
    kept_count = buf("kept_count", (B,), torch.int32)
    h_out = buf("hidden_kept", (B, M, d), hidden.dtype)
    p_out = buf("pos_kept", (B, M), torch.int32)
    g_out = buf("g_kept", (B, M), torch.float32)
    o = buf("o", (B, M, Hq, D), q.dtype)
    lse = buf("lse", (B, Hq, M), torch.float32)
    ws = bufs.get("attn_ws")
    need = tg_gated_attn_workspace_size(B, M, Hq, k.shape[2], D, False)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        bufs["attn_ws"] = ws
    gws = bufs.get("gate_ws")
    gneed = tg_gate_score_workspace_size(d, w1.shape[0], hidden.dtype == torch.bfloat16)
    if gws is None or gws.numel() < gneed:
        gws = torch.empty(max(gneed, 1), dtype=torch.uint8, device=dev)
        bufs["gate_ws"] = gws
    tg_gate_score(hidden, w1, w2, forced_keep, scores, gates, ws=gws, stream=stream)
    key = scores if select_scores is None else select_scores
    sws = bufs.get("select_ws")
    sneed = tg_select_topk_workspace_size(B, N)
    if sws is None or sws.numel() < sneed:
        sws = select_workspace(B, N, dev)
        bufs["select_ws"] = sws
    tg_select_topk(key, forced_keep, K, n_forced, kept, kept_count, ws=sws, stream=stream)
    tg_compact(hidden, pos, gates, kept, h_out, p_out, g_out, stream=stream)
    tg_gated_attn_fwd(q, k, v, g_out, gamma, p_out, rope_theta, tau, o, lse, ws, stream=stream)
    return bufs

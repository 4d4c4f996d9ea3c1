"""Seeded synthetic inputs for the gate-layer workloads.

This module only draws random tensors (and rounds them to their storage
type).  It holds none of the method's arithmetic: no scoring, selection,
gathering or attention.  Both the HIP path's tests/benchmark and the CPU
oracle's tests take their inputs from here, so the two sides see identical
bytes.

Shapes follow a Qwen3-1.7B-sized gate layer (hidden 2048, 16 query heads,
8 KV heads, head dim 128); the pages time TokenGate on Qwen3-1.7B in bf16 at
batch 1.  The public evaluation datasets the pages use are not needed: these
synthetic tensors stand in for their hidden states.

Every tensor has its own child stream of ``numpy.random.SeedSequence(seed)``,
spawned in a fixed order, so adding a tensor never changes the others.
bf16 tensors are returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROPE_THETA = 1.0e6  # Qwen3's rotary base (a model constant, not fixed by the pages)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    N: int            # context tokens per row
    n_forced: int     # non-prunable (scaffold) tokens per row, at positions 0..n_forced-1
    d: int            # hidden size
    d_ff: int         # scorer width
    Ks: tuple         # budgets of document tokens to keep
    Hq: int
    Hkv: int
    D: int
    tau: float
    dtype: str        # "f32" or "bf16"
    rope: bool
    clustered_scores: bool = False
    M_fixed: int = 0  # attention-only workloads: kept tokens per row, drawn positions in [0, N)
    notes: str = field(default="", compare=False)

    def M(self, K: int) -> int:
        if self.M_fixed:
            return self.M_fixed
        return self.n_forced + min(K, self.N - self.n_forced)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 1, B=1, N=512, n_forced=32, d=256, d_ff=64, Ks=(64,), Hq=4, Hkv=4, D=64,
        tau=1.2, dtype="f32", rope=False,
        notes="N=512, 32 scaffold, d=256, scorer 256->64->1, K=64 -> 96 kept, 4/4 heads, D=64, tau=1.2"),
    "qwen3_8k": Workload(
        "qwen3_8k", 2, B=1, N=8192, n_forced=64, d=2048, d_ff=512, Ks=(1024,), Hq=16, Hkv=8, D=128,
        tau=1.0, dtype="bf16", rope=True,
        notes="N=8192, 64 scaffold, K=1024 -> 1088 kept, RMSNorm'd hidden, RoPE at original positions"),
    "qwen3_32k": Workload(
        "qwen3_32k", 3, B=1, N=32768, n_forced=128, d=2048, d_ff=512, Ks=(2048,), Hq=16, Hkv=8, D=128,
        tau=1.0, dtype="bf16", rope=True, clustered_scores=True,
        notes="N=32768, 128 scaffold, K=2048 -> 2176 kept; selection runs on a drawn score vector "
              "with ~5% of document tokens in high-score spans"),
    "sweep_128k": Workload(
        "sweep_128k", 4, B=1, N=131072, n_forced=256, d=2048, d_ff=512, Ks=(256, 1024, 4096, 16384),
        Hq=16, Hkv=8, D=128, tau=1.0, dtype="bf16", rope=True,
        notes="N=131072, 256 scaffold, one scorer pass, K in {256, 1024, 4096, 16384}"),
    "train_b4": Workload(
        "train_b4", 5, B=4, N=16384, n_forced=0, d=0, d_ff=0, Ks=(2048,), Hq=16, Hkv=8, D=128,
        tau=1.0, dtype="bf16", rope=True, M_fixed=2048,
        notes="attention forward + backward, B=4, 2048 kept tokens at sorted distinct positions in [0, 16384)"),
}


def _streams(seed: int, names):
    kids = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.default_rng(k) for n, k in zip(names, kids)}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def forced_mask(w: Workload) -> np.ndarray:
    """uint8 [B, N]: 1 on the scaffold tokens (the first n_forced positions of each row)."""
    f = np.zeros((w.B, w.N), np.uint8)
    f[:, : w.n_forced] = 1
    return f


def gate_inputs(w: Workload, N: int | None = None):
    """Hidden states and scorer weights.

    tiny_f32: hidden ~ N(0,1) in fp32.  bf16 workloads: N(0,1) rows scaled to unit
    root-mean-square (eps 1e-6, unit weight) and rounded to bf16, standing in for
    the normalised post-attention residual.  W1 ~ N(0, 1/d) stored [d_ff, d]
    (out x in), w2 ~ N(0, 1/d_ff).  Returns dict(hidden [B,N,d], w1, w2, forced).
    """
    N = w.N if N is None else N
    rs = _streams(w.seed, ["hidden", "w1", "w2"])
    h = rs["hidden"].standard_normal((w.B, N, w.d), dtype=np.float32)
    if w.dtype == "bf16":
        ms = np.mean(np.square(h, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
        h *= (1.0 / np.sqrt(ms + np.float32(1e-6))).astype(np.float32)
    w1 = rs["w1"].standard_normal((w.d_ff, w.d), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.d))
    w2 = rs["w2"].standard_normal((w.d_ff,), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.d_ff))
    f = np.zeros((w.B, N), np.uint8)
    f[:, : w.n_forced] = 1
    return dict(hidden=_store(h, w.dtype), w1=_store(w1, w.dtype), w2=_store(w2, w.dtype), forced=f)


def residual_inputs(w: Workload, N: int | None = None):
    """Raw post-attention residual rows and an RMSNorm weight, for the scorer with LN2 in front.

    hidden [B, N, d]: N(0,1) rows, each scaled by exp(U(ln 1/4, ln 4)) (token norms spread over
    a factor of 16, the spread the normalisation removes), stored bf16 (or fp32); ln_w [d] ~
    U(0.5, 1.5) in the same storage type.  The scorer weights are gate_inputs' (same seed).
    """
    N = w.N if N is None else N
    rs = _streams(w.seed + 2000, ["hidden", "scale", "ln_w"])
    h = rs["hidden"].standard_normal((w.B, N, w.d), dtype=np.float32)
    h *= np.exp(rs["scale"].uniform(np.log(0.25), np.log(4.0), (w.B, N, 1))).astype(np.float32)
    lw = rs["ln_w"].uniform(0.5, 1.5, w.d).astype(np.float32)
    return dict(hidden=_store(h, w.dtype), ln_w=_store(lw, w.dtype))


QWEN3_1P7B_MLP = 6144  # the Qwen3-1.7B MLP width (public model config; the pages give no width)


def clone_inputs(w: Workload, d_i: int, H: int, N: int | None = None, seed_offset: int = 0):
    """Weights of the scorer cloned from the gate layer's MLP, for w's hidden states.

    w_gate, w_up ~ N(0, 1/d) [d_i, d]; w_down ~ N(0, 1/d_i) [d, d_i]; w_head ~ N(0, 1/d) [H, d]
    (all out x in, in w's storage type).  Hidden rows and the RMSNorm weight are gate_inputs' and
    residual_inputs' (same seed).  Returns dict(w_gate, w_up, w_down, w_head).
    """
    rs = _streams(w.seed + 3000 + seed_offset, ["w_gate", "w_up", "w_down", "w_head"])
    sd, si = np.float32(1.0 / np.sqrt(w.d)), np.float32(1.0 / np.sqrt(d_i))
    wg = rs["w_gate"].standard_normal((d_i, w.d), dtype=np.float32) * sd
    wu = rs["w_up"].standard_normal((d_i, w.d), dtype=np.float32) * sd
    wd = rs["w_down"].standard_normal((w.d, d_i), dtype=np.float32) * si
    wh = rs["w_head"].standard_normal((H, w.d), dtype=np.float32) * sd
    return {k: _store(v, w.dtype) for k, v in dict(w_gate=wg, w_up=wu, w_down=wd, w_head=wh).items()}


def clustered_scores(w: Workload, N: int | None = None, frac: float = 0.05) -> np.ndarray:
    """float32 [B, N] selection scores with relevant spans.

    Background ~ N(0,1); non-overlapping, non-adjacent spans of U[8, 64] document
    tokens at random starts receive 3 + |N(0, 0.5)| until about `frac` of the
    document tokens are covered.  All values lie on the bf16 grid, so many
    tokens tie exactly near the selection threshold.
    """
    N = w.N if N is None else N
    rs = _streams(w.seed + 1000, ["background", "spans", "span_values"])
    out = np.empty((w.B, N), np.float32)
    for b in range(w.B):
        s = rs["background"].standard_normal(N, dtype=np.float32)
        covered = np.zeros(N, bool)
        target = int(round(frac * (N - w.n_forced)))
        got = 0
        tries = 0
        while got < target and tries < 100000:
            tries += 1
            L = int(rs["spans"].integers(8, 65))
            lo = w.n_forced
            if N - L < lo:
                break
            st = int(rs["spans"].integers(lo, N - L + 1))
            if covered[max(st - 1, 0): st + L + 1].any():
                continue
            covered[st: st + L] = True
            s[st: st + L] = 3.0 + np.abs(rs["span_values"].normal(0.0, 0.5, L)).astype(np.float32)
            got += L
        out[b] = bf16_to_f32(bf16_bits(s))
    return out


def attn_inputs(w: Workload, M: int, with_grad: bool = False, seed_offset: int = 0):
    """Attention operands at M kept tokens per row.

    q ~ N(0,1) [B, M, Hq, D]; k, v ~ N(0,1) [B, M, Hkv, D] (bf16 or fp32 per the
    workload); gamma ~ U(0.5, 1.5) [Hq]; g = 1/(1+exp(-z)), z ~ N(0,1), float32
    [B, M] (a distribution of gate values in (0, 1)); positions int32 [B, M]:
    sorted distinct draws from [0, max(N, M)), the shape of the original positions
    that compaction hands to attention; dout ~ N(0,1) like q when with_grad;
    sigma [Hq] float32 ~ N(ln(e - 1), 0.5^2), the raw temperature parameter
    (softplus(ln(e - 1)) = 1, the identity scale, plus a spread across heads).
    """
    rs = _streams(w.seed * 7919 + 17 + seed_offset, ["q", "k", "v", "gamma", "g", "pos", "dout", "sigma"])
    q = rs["q"].standard_normal((w.B, M, w.Hq, w.D), dtype=np.float32)
    k = rs["k"].standard_normal((w.B, M, w.Hkv, w.D), dtype=np.float32)
    v = rs["v"].standard_normal((w.B, M, w.Hkv, w.D), dtype=np.float32)
    gamma = rs["gamma"].uniform(0.5, 1.5, w.Hq).astype(np.float32)
    z = rs["g"].standard_normal((w.B, M)).astype(np.float64)
    g = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    pos = np.stack([np.sort(rs["pos"].choice(max(w.N, M), M, replace=False)) for _ in range(w.B)]).astype(np.int32)
    sigma = (np.log(np.e - 1.0) + 0.5 * rs["sigma"].standard_normal(w.Hq)).astype(np.float32)
    out = dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype), gamma=gamma, g=g, pos=pos,
               sigma=sigma)
    if with_grad:
        out["dout"] = _store(rs["dout"].standard_normal((w.B, M, w.Hq, w.D), dtype=np.float32), w.dtype)
    return out


def as_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float32 values (exact)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def to_torch(x: np.ndarray, dtype: str, device="cpu"):
    """Storage array -> torch tensor of the storage dtype (bf16 bits reinterpreted, no rounding)."""
    import torch

    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)

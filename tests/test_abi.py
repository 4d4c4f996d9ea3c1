"""The C-ABI library loads and exports what include/tokengate.h declares; host-side
argument checks return their status before any device call (CPU only, no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")


def _lib():
    import learned_token_pruning_gatescore_amd as tg

    if not os.path.exists(tg.library_path()):
        pytest.skip("libtokengate.so not built")
    return tg.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (tg_[a-z_]+)\b", out))
    assert set(names) <= exported
    # nothing but the declared C entry points leaks as tg_* symbols
    assert exported <= set(names)


def test_status_strings_and_version():
    lib = _lib()
    assert lib.tg_version() >= 100
    for s in range(5):
        assert lib.tg_status_string(s)
    assert lib.tg_kept_count(32768, 128, 2048) == 2176
    assert lib.tg_kept_count(100, 10, 1000) == 100
    assert lib.tg_kept_count(100, 10, 0) == 10
    assert lib.tg_kept_count(100, 101, 5) == -1
    assert lib.tg_kept_count(100, 10, -1) == -1


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first
MIS = ctypes.c_void_p(0x10008)    # misaligned


def test_gate_score_validation():
    lib = _lib()
    g = lambda *a, ws=None, wsb=0: lib.tg_gate_score(*a, ws, wsb, None)
    st = g(None, FAKE, FAKE, None, 1, 10, 32, 16, 1, FAKE, None)
    assert st == 1 and b"required" in lib.tg_last_error()
    assert g(FAKE, FAKE, FAKE, None, 1, 10, 0, 16, 1, FAKE, None) == 1
    assert g(FAKE, FAKE, FAKE, None, 1, 10, 48, 16, 1, FAKE, None) == 2  # bf16 d % 32
    assert g(FAKE, FAKE, FAKE, None, 1, 10, 32, 16, 7, FAKE, None) == 1  # dtype
    assert g(MIS, FAKE, FAKE, None, 1, 10, 32, 16, 1, FAKE, None) == 1  # alignment
    # bf16 needs the fragment-order workspace: d_ff rounded up to 512 units, d to 128 inputs
    need = lib.tg_gate_score_workspace_size(2048, 512, 1)
    assert need == 512 * 2048 * 2
    assert lib.tg_gate_score_workspace_size(32, 16, 1) == 512 * 128 * 2
    assert lib.tg_gate_score_workspace_size(2048, 512, 0) == 0
    assert lib.tg_gate_score_workspace_size(0, 512, 1) == 0
    assert g(FAKE, FAKE, FAKE, None, 1, 10, 2048, 512, 1, FAKE, None) == 3
    assert g(FAKE, FAKE, FAKE, None, 1, 10, 2048, 512, 1, FAKE, None, ws=FAKE, wsb=need - 1) == 3
    assert g(FAKE, FAKE, FAKE, None, 0, 10, 2048, 512, 1, FAKE, None, ws=FAKE, wsb=need) == 0  # B = 0
    # packed pair
    assert lib.tg_gate_pack_w1(FAKE, 2048, 512, 0, FAKE, need, None) == 2            # f32 not packed
    assert lib.tg_gate_pack_w1(FAKE, 2048, 512, 1, FAKE, need - 16, None) == 3       # too small
    assert lib.tg_gate_pack_w1(None, 2048, 512, 1, FAKE, need, None) == 1
    assert lib.tg_gate_score_packed(FAKE, FAKE, FAKE, None, 1, 10, 2048, 512, 0, FAKE, None, None) == 2
    assert lib.tg_gate_score_packed(FAKE, FAKE, FAKE, None, 1, 10, 48, 512, 1, FAKE, None, None) == 2


def test_select_validation():
    lib = _lib()
    assert lib.tg_select_topk(FAKE, FAKE, 1, 100, -1, 0, FAKE, None, None, 0, None) == 1   # K < 0
    assert lib.tg_select_topk(FAKE, FAKE, 1, 100, 5, 101, FAKE, None, None, 0, None) == 1  # n_forced > N
    assert lib.tg_select_topk(FAKE, None, 1, 100, 5, 3, FAKE, None, None, 0, None) == 1    # mask missing
    assert lib.tg_select_topk(None, None, 1, 100, 5, 0, FAKE, None, None, 0, None) == 1    # scores missing
    # a workspace of tg_select_topk_workspace_size bytes (256-byte aligned) is required
    need = lib.tg_select_topk_workspace_size(2, 40000)
    assert need >= 2 * 40000 * 8 and lib.tg_select_topk_workspace_size(1, 1) > 0
    assert lib.tg_select_topk_workspace_size(1, (1 << 22) + 1) == 0
    assert lib.tg_select_topk(FAKE, None, 2, 40000, 5, 0, FAKE, None, None, 0, None) == 3
    assert lib.tg_select_topk(FAKE, None, 2, 40000, 5, 0, FAKE, None, FAKE, need - 1, None) == 3
    assert lib.tg_select_topk(FAKE, None, 2, 40000, 5, 0, FAKE, None, ctypes.c_void_p(0x10010), need, None) == 1
    assert lib.tg_select_topk(FAKE, None, 1, (1 << 22) + 1, 5, 0, FAKE, None, FAKE, 1 << 40, None) == 2
    assert lib.tg_select_topk(FAKE, None, 0, 100, 5, 0, FAKE, None, None, 0, None) == 0    # B = 0: nothing to do


def test_compact_validation():
    lib = _lib()
    assert lib.tg_compact(FAKE, None, None, None, 1, 10, 4, 64, 1, FAKE, None, None, None) == 1     # kept_idx
    assert lib.tg_compact(FAKE, None, None, FAKE, 1, 10, 4, 64, 1, FAKE, None, FAKE, None) == 1     # gates_out w/o gates
    assert lib.tg_compact(FAKE, None, None, FAKE, 1, 10, 4, 4, 1, FAKE, None, None, None) == 2      # 8-byte rows
    assert lib.tg_compact(FAKE, None, None, FAKE, 1, 10, 0, 64, 1, FAKE, None, None, None) == 0     # M = 0


def test_attn_validation():
    lib = _lib()
    f = lib.tg_gated_attn_fwd
    args = lambda **kw: [kw.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, kw.get("pos", None), 1e6, kw.get("tau", 1.0),
                         kw.get("sigma", None), 1, 100, kw.get("Hq", 16), kw.get("Hkv", 8), kw.get("D", 128),
                         kw.get("dt", 1), FAKE, None, kw.get("o_lo", None), kw.get("ws", None), kw.get("wsb", 0),
                         None]
    assert f(*args(q=None)) == 1
    assert f(*args(Hq=12, Hkv=8)) == 1          # Hq % Hkv
    assert f(*args(D=96)) == 2                  # bf16 D
    assert f(*args(Hq=24, Hkv=8)) == 2          # group of 3
    assert f(*args(tau=0.0)) == 1
    assert f(*args()) == 3                      # a workspace is required
    assert f(*args(pos=FAKE)) == 3
    need = lib.tg_gated_attn_workspace_size(1, 100, 16, 8, 128, 0)
    assert need >= 100 * 64 * 8
    assert f(*args(pos=FAKE, ws=FAKE, wsb=need - 1)) == 3
    assert f(*args(q=MIS)) == 1
    assert f(*args(sigma=MIS)) == 1             # misaligned sigma
    assert f(*args(o_lo=MIS)) == 1              # misaligned o_lo
    assert f(*args(dt=0, o_lo=FAKE)) == 1       # o_lo with f32
    # the bf16 kernels' 32-bit buffer ranges: M * max(Hq, Hkv) * D * 2 must stay below 2^31
    big = lambda M: [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, None, 1, M, 16, 8, 128, 1, FAKE, None, None, FAKE,
                     1 << 40, None]
    assert f(*big(1 << 20)) == 2
    assert f(*big((1 << 19) + 1)) == 2
    assert b"2^31" in lib.tg_last_error()
    bbig = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, None, FAKE, FAKE, None, None, 1, 1 << 20, 16, 8, 128, 1,
            FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None]
    assert lib.tg_gated_attn_bwd(*bbig) == 2
    b = lib.tg_gated_attn_bwd
    bargs = lambda **kw: [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, kw.get("sigma", None), kw.get("lse", FAKE),
                          FAKE, kw.get("o", None), kw.get("o_lo", None), 1, 100, 16, 8, 128, kw.get("dt", 1), FAKE,
                          FAKE, FAKE, FAKE, FAKE, kw.get("dsigma", None), FAKE, kw.get("wsb", 1 << 20), None]
    assert b(*bargs(lse=None)) == 1              # missing lse
    assert b(*bargs(wsb=16)) == 3                # workspace too small
    assert b(*bargs(sigma=FAKE)) == 1            # sigma without dsigma
    assert b(*bargs(dsigma=FAKE)) == 1           # dsigma without sigma
    assert b(*bargs(sigma=FAKE, dsigma=MIS)) == 1
    assert b(*bargs(o=FAKE)) == 1                # o without o_lo
    assert b(*bargs(o_lo=FAKE)) == 1             # o_lo without o
    assert b(*bargs(o=MIS, o_lo=FAKE)) == 1      # misaligned o
    assert b(*bargs(o=FAKE, o_lo=FAKE, dt=0)) == 1  # o and o_lo with f32


def test_norm_gate_validation():
    lib = _lib()
    # tg_gate_score_ln: (hidden, ln_w, ln_eps, w1, w2, forced, B, N, d, d_ff, dt, scores, gates, ws, ws_bytes, stream)
    f = lib.tg_gate_score_ln
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(FAKE, None, -1.0, FAKE, FAKE, None, 1, 10, 64, 16, 1, FAKE, None, FAKE, 1 << 30, None) == 1  # eps < 0
    assert f(FAKE, None, float("nan"), FAKE, FAKE, None, 1, 10, 64, 16, 1, FAKE, None, FAKE, 1 << 30, None) == 1
    assert f(FAKE, MIS, 1e-6, FAKE, FAKE, None, 1, 10, 64, 16, 1, FAKE, None, FAKE, 1 << 30, None) == 1  # ln_w
    assert f(FAKE, None, 1e-6, FAKE, FAKE, None, 1, 10, 64, 16, 1, FAKE, None, FAKE, 16, None) == 3  # workspace
    assert f(FAKE, None, 1e-6, FAKE, FAKE, None, 1, 10, 48, 16, 1, FAKE, None, FAKE, 1 << 30, None) == 2  # d % 32
    n = lib.tg_score_normalize
    n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert n(None, None, 1, 10, 1e-6, FAKE, None) == 1
    assert n(FAKE, None, 1, 10, -1.0, FAKE, None) == 1
    assert n(FAKE, None, -1, 10, 1e-6, FAKE, None) == 1
    assert n(FAKE, None, 1, (1 << 24) + 1, 1e-6, FAKE, None) == 2
    assert n(FAKE, None, 1, 10, 1e-6, MIS, None) == 1
    assert n(FAKE, None, 0, 10, 1e-6, FAKE, None) == 0  # empty: nothing launched
    s = lib.tg_gate_softmax
    s.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert s(None, None, 1, 10, FAKE, None) == 1
    assert s(FAKE, MIS, 1, 10, FAKE, None) == 1
    assert s(FAKE, None, 1, -2, FAKE, None) == 1
    assert s(FAKE, None, 1, 0, FAKE, None) == 0
    sb = lib.tg_gate_softmax_bwd
    sb.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_void_p]
    assert sb(FAKE, None, 1, 10, FAKE, None) == 1
    assert sb(FAKE, FAKE, 1, 10, MIS, None) == 1
    assert sb(FAKE, FAKE, 0, 10, FAKE, None) == 0


def test_varlen_validation():
    lib = _lib()
    i64 = ctypes.c_int64
    ws = lib.tg_gated_attn_varlen_workspace_size
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, ctypes.c_int]
    cu_t = ctypes.c_int64 * 5
    good = cu_t(0, 100, 100, 200, 250)  # runs: (2 x 100), (1 x 50)
    bad0 = cu_t(1, 100, 100, 200, 250)
    desc = cu_t(0, 100, 90, 200, 250)
    assert ws(good, 4, 16, 8, 128, 0) > 0
    assert ws(good, 4, 16, 8, 128, 1) > ws(good, 4, 16, 8, 128, 0)
    assert ws(bad0, 4, 16, 8, 128, 0) == 0 and ws(desc, 4, 16, 8, 128, 0) == 0 and ws(None, 4, 16, 8, 128, 0) == 0
    # every run's arrays side by side: at least those of the largest run (2 sequences x 100 tokens)
    assert ws(good, 4, 16, 8, 128, 0) >= lib.tg_gated_attn_workspace_size(2, 100, 16, 8, 128, 0)
    f = lib.tg_gated_attn_fwd_varlen
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, i64, i64,
                                          i64, i64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    args = lambda cu, **kw: [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, None, cu, 4, kw.get("Hq", 16), 8,
                             kw.get("D", 128), 1, FAKE, None, kw.get("o_lo", None), kw.get("ws", FAKE),
                             kw.get("wsb", 16), None]
    assert f(*args(None)) == 1                 # cu_seqlens required
    assert f(*args(bad0)) == 1                 # cu_seqlens[0] != 0
    assert f(*args(desc)) == 1                 # decreasing
    assert f(*args(good, Hq=12)) == 1          # Hq % Hkv
    assert f(*args(good, D=96)) == 2           # bf16 D
    assert f(*args(good)) == 3                 # workspace too small
    huge = cu_t(0, 1 << 19, 1 << 20, (1 << 20) + 5, (1 << 20) + 5)
    assert f(*args(huge, wsb=1 << 40)) == 2    # the packed tokens exceed the kernels' 32-bit ranges
    b = lib.tg_gated_attn_bwd_varlen
    b.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_float, ctypes.c_float] + [ctypes.c_void_p] * 6 + [
        i64, i64, i64, i64, ctypes.c_int] + [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p]
    bargs = lambda **kw: [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, kw.get("sigma", None), kw.get("lse", FAKE),
                          FAKE, kw.get("o", None), kw.get("o_lo", None), good, 4, 16, 8, 128, 1, FAKE, FAKE, FAKE,
                          FAKE, FAKE, kw.get("dsigma", None), FAKE, kw.get("wsb", 16), None]
    assert b(*bargs(lse=None)) == 1
    assert b(*bargs(sigma=FAKE)) == 1          # sigma without dsigma
    assert b(*bargs()) == 3                    # workspace too small
    assert b(*bargs(o=FAKE)) == 1              # o without o_lo
    assert f(*args(good, o_lo=MIS)) == 1       # misaligned o_lo


def test_heads_validation():
    lib = _lib()
    i64 = ctypes.c_int64
    f = lib.tg_gate_score_heads
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    assert f(FAKE, 0, None, 0.0, FAKE, FAKE, 1, 10, 64, 16, 17, 1, FAKE, FAKE, 1 << 30, None) == 2  # H > 16
    assert f(FAKE, 0, None, 0.0, FAKE, FAKE, 1, 10, 64, 16, 0, 1, FAKE, FAKE, 1 << 30, None) == 2   # H < 1
    assert f(FAKE, 1, None, -1.0, FAKE, FAKE, 1, 10, 64, 16, 4, 1, FAKE, FAKE, 1 << 30, None) == 1  # eps
    assert f(FAKE, 0, None, 0.0, FAKE, FAKE, 1, 10, 64, 16, 4, 1, FAKE, FAKE, 16, None) == 3        # workspace
    n = lib.tg_score_normalize_heads
    n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64, i64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    assert n(FAKE, None, 1, 0, 10, 1e-6, FAKE, None) == 1
    assert n(None, None, 1, 2, 10, 1e-6, FAKE, None) == 1
    a = lib.tg_aggregate_heads
    a.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
    assert a(FAKE, 1, 0, 10, FAKE, None) == 1
    assert a(FAKE, 1, 2, 10, MIS, None) == 1
    g = lib.tg_gather_heads
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
    assert g(FAKE, None, 1, 2, 10, 5, FAKE, None) == 1
    s = lib.tg_gate_softmax_heads
    s.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
    assert s(FAKE, None, 1, 0, 10, FAKE, None) == 1
    hf = lib.tg_gated_attn_fwd_headgates
    hf.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, i64, i64, i64, i64, i64,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert hf(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, None, 1, 100, 12, 8, 128, 1, FAKE, None, None, None, 0,
              None) == 1  # Hq % Hkv
    assert hf(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e6, 1.0, None, 1, 100, 16, 8, 128, 1, FAKE, None, None, None, 0,
              None) == 3  # workspace


def test_clone_validation():
    lib = _lib()
    i64 = ctypes.c_int64
    P = ctypes.c_void_p
    f = lib.tg_gate_score_clone
    f.argtypes = [P, ctypes.c_int, P, ctypes.c_float, P, P, P, P, i64, i64, i64, i64, i64, ctypes.c_int, P, P,
                  ctypes.c_size_t, P]
    ws = lib.tg_gate_score_clone_workspace_size
    ws.argtypes = [i64, i64, i64, ctypes.c_int]
    ws.restype = ctypes.c_size_t
    # workspace: packed gate/up (bf16), then U = [H, d_i] fp32 and the fold's partial sums
    assert ws(2048, 6144, 16, 1) >= 2 * 6144 * 2048 * 2 + 2 * 16 * 6144 * 4
    assert 2 * 3 * 100 * 4 <= ws(256, 100, 3, 0) < ws(256, 100, 3, 1)
    assert ws(256, 100, 17, 1) == 0 and ws(256, 40000, 1, 1) == 0 and ws(0, 64, 1, 1) == 0
    big = 1 << 34
    c = lambda *a, **kw: f(kw.get("h", FAKE), kw.get("ln", 0), None, kw.get("eps", 0.0), FAKE, FAKE,
                           kw.get("wd", FAKE), kw.get("wh", FAKE), *a, kw.get("dt", 1), FAKE, kw.get("ws", FAKE),
                           kw.get("wsb", big), None)
    assert c(1, 10, 64, 32, 17) == 2                       # H > 16
    assert c(1, 10, 64, 32, 0) == 2                        # H < 1
    assert c(1, 10, 64, 40000, 4) == 2                     # d_i > 32768
    assert c(1, 10, 48, 32, 4) == 2                        # bf16 needs d % 32 == 0
    assert c(1, 10, 64, 16000, 4, dt=0) == 2               # f32: d + d_i too large for one row in LDS
    assert c(1, 10, 64, 32, 4, wd=None) == 1               # w_down missing
    assert c(1, 10, 64, 32, 4, wh=MIS) == 1                # misaligned
    assert c(1, 10, 64, 32, 4, ln=1, eps=-1.0) == 1        # ln_eps
    assert c(1, 10, 64, 32, 4, wsb=16) == 3                # workspace too small
    assert c(1, 10, 64, 32, 4, ws=None) == 3               # workspace missing

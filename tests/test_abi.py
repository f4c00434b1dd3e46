"""The C-ABI library loads, exports every function include/gdn.h declares, and
rejects bad arguments on the host before touching the GPU (these calls pass
fake, never-dereferenced device addresses and need no GPU)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_34_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gdn.lib_path), reason="libgdn.so not built")

FAKE = 0x7F0000000000  # 256-aligned, never dereferenced by the validation paths
NULL = None


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn\w*)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("gdn_chunk_fwd", "gdn2_chunk_fwd", "gdn_recurrent_step", "gdn2_recurrent_step", "gdn_chunk_intra",
              "gdn_chunk_bwd", "gdn_chunk_bwd_workspace", "gdn_chunk_fwd_varlen",
              "gdn_chunk_fwd_workspace", "gdn2_chunk_fwd_workspace", "gdn_status_string",
              "gdn_prologue", "gdn_gated_rmsnorm", "gdn2_chunk_bwd", "gdn2_chunk_bwd_workspace"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gdn.lib_path)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings():
    assert gdn.status_string(0) == "ok"
    for c in range(1, 5):
        assert gdn.status_string(c) not in ("ok", "unknown status")


def _p(x):
    return ctypes.c_void_p(x) if x else None


def _chunk(lib, q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), g=FAKE + (3 << 32), beta=FAKE + (4 << 32),
           h0=None, o=FAKE + (5 << 32), ht=FAKE + (6 << 32), B=2, T=100, H=3, Dk=128, Dv=128, dt=1,
           ws=FAKE + (7 << 32), ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.gdn_chunk_fwd_workspace(B, T, H, Dk, Dv, dt)
    return lib.gdn_chunk_fwd(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(o), _p(ht), B, T, H, Dk, Dv, dt,
                             0.1, _p(ws), ws_bytes, None)


def test_workspace_size():
    lib = gdn.load()
    assert lib.gdn_chunk_fwd_workspace(2, 100, 3, 128, 128, 1) == 256   # bf16: single kernel
    n = lib.gdn_chunk_fwd_workspace(2, 100, 3, 128, 128, 0)
    NT = 2
    assert n >= 2 * 3 * NT * 64 * 4 + 2 * 3 * NT * 64 * 64 * 4
    assert n % 256 == 0
    assert lib.gdn_chunk_fwd_workspace(0, 100, 3, 128, 128, 1) == 0
    assert lib.gdn_chunk_fwd_workspace(2, 100, 3, 96, 128, 1) == 0


def test_chunk_fwd_rejects_bad_arguments():
    lib = gdn.load()
    assert _chunk(lib, q=NULL) == 1
    assert _chunk(lib, o=NULL) == 1
    assert _chunk(lib, B=0) == 1
    assert _chunk(lib, T=0) == 1
    assert _chunk(lib, H=-1) == 1
    assert _chunk(lib, Dk=96, ws_bytes=1 << 30) == 2
    assert _chunk(lib, Dv=32, ws_bytes=1 << 30) == 2
    assert _chunk(lib, dt=7, ws_bytes=1 << 30) == 2
    assert _chunk(lib, ws=NULL, dt=0) == 3                           # fp32 path needs a workspace
    assert _chunk(lib, ws=FAKE + (7 << 32) + 4, dt=0) == 3           # misaligned
    assert _chunk(lib, ws_bytes=1024, dt=0) == 3                     # too small
    assert _chunk(lib, o=FAKE) == 1                                  # o overlaps q
    assert _chunk(lib, ht=FAKE + (5 << 32)) == 1                     # ht overlaps o
    assert _chunk(lib, h0=FAKE + (8 << 32), ht=FAKE + (8 << 32) + 256) == 1   # partial alias


def test_step_and_intra_reject_bad_arguments():
    lib = gdn.load()
    f = lambda *a: lib.gdn_recurrent_step(*[_p(x) for x in a[:7]], *a[7:], 0.1, None)
    base = [FAKE + (i << 32) for i in range(7)]
    assert f(*base[:6], None, 4, 2, 128, 128, 1) == 1
    assert f(*base, 0, 2, 128, 128, 1) == 1
    assert f(*base, 4, 2, 100, 128, 1) == 2
    assert f(*base[:5], base[0], base[6], 4, 2, 128, 128, 1) == 1   # S overlaps q
    assert lib.gdn_chunk_intra(None, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 1, 64, 1, 128, 1, None) == 1
    assert lib.gdn_chunk_intra(_p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 1, 64, 1, 48, 1, None) == 2


def test_gdn2_step_rejects_bad_arguments():
    lib = gdn.load()
    f = lambda *a: lib.gdn2_recurrent_step(*[_p(x) for x in a[:8]], *a[8:], 0.1, None)
    base = [FAKE + (i << 32) for i in range(8)]
    assert f(*base[:7], None, 4, 2, 128, 128, 1) == 1                  # no output
    assert f(*base, 0, 2, 128, 128, 1) == 1                            # B = 0
    assert f(*base, 4, 2, 96, 128, 1) == 2                             # unsupported head size
    assert f(*base, 4, 2, 128, 128, 5) == 2                            # unknown dtype
    assert f(*base[:6], base[3], base[7], 4, 2, 128, 128, 1) == 1      # S overlaps log_alpha
    assert f(*base[:7], base[1], 4, 2, 128, 128, 1) == 1               # o overlaps k


def test_bwd_workspace_and_validation():
    lib = gdn.load()
    B, T, H, Dk, Dv = 2, 100, 3, 128, 128
    n = lib.gdn_chunk_bwd_workspace(B, T, H, Dk, Dv, 1)
    NT = 2
    assert n >= 2 * B * H * NT * Dk * Dv * 4 + B * H * NT * 64 * 64 * 4
    assert n % 256 == 0
    assert lib.gdn_chunk_bwd_workspace(B, T, H, 96, Dv, 1) == 0
    ptrs = [FAKE + (i << 32) for i in range(14)]   # q k v g beta h0 dO dht dq dk dv dg dbeta dh0
    ws = FAKE + (20 << 32)

    def f(p=ptrs, Dk=Dk, dt=1, w=ws, nbytes=n):
        return lib.gdn_chunk_bwd(*[_p(x) for x in p], B, T, H, Dk, Dv, dt, 0.1, _p(w), nbytes, None)

    assert f(p=ptrs[:6] + [None] + ptrs[7:]) == 1                   # no dO
    assert f(p=ptrs[:8] + [None] + ptrs[9:]) == 1                   # no dq
    assert f(Dk=96) == 2
    assert f(dt=4) == 2
    assert f(w=None) == 3
    assert f(nbytes=n - 256) == 3
    assert f(w=ws + 8) == 3                                          # misaligned
    assert f(p=ptrs[:8] + [ptrs[0]] + ptrs[9:]) == 1                # dq overlaps q
    assert f(p=ptrs[:9] + [ptrs[8]] + ptrs[10:]) == 1               # dk overlaps dq
    assert f(p=ptrs[:13] + [ws]) == 1                               # dh0 overlaps the workspace


def test_varlen_rejects_bad_arguments():
    lib = gdn.load()
    p = [FAKE + (i << 32) for i in range(9)]   # q k v g beta cu h0 o ht

    def f(ptrs=p, N=3, total=300, Dk=128, dt=1):
        return lib.gdn_chunk_fwd_varlen(*[_p(x) for x in ptrs], N, total, 2, Dk, 128, dt, 0.1, None)

    assert f(ptrs=p[:5] + [None] + p[6:]) == 1      # no cu_seqlens
    assert f(N=0) == 1
    assert f(total=0) == 1
    assert f(dt=0) == 2                             # fp32: not supported on this path
    assert f(Dk=96) == 2
    assert f(ptrs=p[:7] + [p[0]] + p[8:]) == 1      # o overlaps q
    assert f(ptrs=p[:7] + [p[5]] + p[8:]) == 1      # o overlaps cu_seqlens


def test_gdn2_varlen_workspace_and_validation():
    lib = gdn.load()
    N, total, H = 3, 300, 2
    need = lib.gdn2_chunk_fwd_varlen_workspace(N, total, H, 128, 128, 1)
    # chunk numbers ceil(300 / 64) + 3 = 8 per head, one block each, plus the two tables
    blk = 66304
    assert need >= H * 8 * blk and need % 256 == 0
    assert lib.gdn2_chunk_fwd_varlen_workspace(N, total, H, 128, 128, 0) == 0   # fp32 unsupported
    assert lib.gdn2_chunk_fwd_varlen_workspace(0, total, H, 128, 128, 1) == 0
    assert lib.gdn2_chunk_fwd_varlen_workspace(N, total, H, 96, 128, 1) == 0
    p = [FAKE + (i << 36) for i in range(10)]   # q k v log_alpha b w cu h0 o ht
    ws = FAKE + (12 << 36)

    def f(ptrs=p, N=N, total=total, Dk=128, dt=1, w=ws, nbytes=need):
        return lib.gdn2_chunk_fwd_varlen(*[_p(x) for x in ptrs], N, total, H, Dk, 128, dt, 0.1, _p(w), nbytes, None)

    assert f(ptrs=p[:6] + [None] + p[7:]) == 1      # no cu_seqlens
    assert f(ptrs=p[:8] + [None] + p[9:]) == 1      # no o
    assert f(N=0) == 1
    assert f(total=0) == 1
    assert f(dt=0) == 2                             # fp32: not supported on this path
    assert f(Dk=96) == 2
    assert f(w=None) == 3
    assert f(w=ws + 8) == 3                         # misaligned workspace
    assert f(nbytes=need - 1) == 3
    assert f(ptrs=p[:8] + [p[0]] + p[9:]) == 1      # o overlaps q
    assert f(ptrs=p[:8] + [p[6]] + p[9:]) == 1      # o overlaps cu_seqlens
    assert f(ptrs=p[:9] + [p[8]]) == 1              # ht overlaps o
    assert f(w=p[3]) == 1                           # workspace overlaps log_alpha
    assert f(ptrs=[p[0] + 2] + p[1:]) == 1          # q not 16-byte aligned
    assert f(ptrs=p[:5] + [p[5] + 8] + p[6:]) == 1  # w not 16-byte aligned


def test_gdn2_bwd_workspace_and_validation():
    lib = gdn.load()
    assert lib.gdn2_chunk_bwd_workspace(2, 100, 3, 128, 128, 1) > 0
    assert lib.gdn2_chunk_bwd_workspace(2, 100, 3, 96, 128, 1) == 0
    assert lib.gdn2_chunk_bwd_workspace(0, 100, 3, 128, 128, 1) == 0
    # q k v la b w h0 dO dht | dq dk dv dla db dw dh0
    p = [FAKE + (i << 32) for i in range(16)]
    ws = FAKE + (20 << 32)
    need = lib.gdn2_chunk_bwd_workspace(2, 100, 3, 128, 128, 1)

    def f(ptrs=p, B=2, Dk=128, dt=1, w=ws, nbytes=need):
        return lib.gdn2_chunk_bwd(*[_p(x) for x in ptrs], B, 100, 3, Dk, 128, dt, 0.1, _p(w), nbytes, None)

    assert f(ptrs=[None] + p[1:]) == 1                # no q
    assert f(ptrs=p[:9] + [None] + p[10:]) == 1       # no dq
    assert f(B=0) == 1
    assert f(Dk=96) == 2
    assert f(dt=7) == 2
    assert f(w=None) == 3
    assert f(w=ws + 8) == 3                           # misaligned
    assert f(nbytes=need - 1) == 3
    assert f(ptrs=p[:9] + [p[0]] + p[10:]) == 1       # dq overlaps q
    assert f(ptrs=p[:10] + [p[9]] + p[11:]) == 1      # dk overlaps dq
    assert f(w=p[3]) == 1                             # workspace overlaps log_alpha
    assert f(ptrs=[p[0] + 2] + p[1:]) == 1            # bf16 q not 16-byte aligned
    assert f(ptrs=p[:3] + [p[3] + 4] + p[4:]) == 1    # bf16 path: log_alpha not 16-byte aligned


def test_prologue_rejects_bad_arguments():
    lib = gdn.load()
    # xq xk xv a b wq wk wv A_log dt_bias conv_in | q k v g beta conv_out
    p = [FAKE + (i << 32) for i in range(17)]

    def f(ptrs=p, B=2, T=100, H=3, Dk=128, Dv=128):
        return lib.gdn_prologue(*[_p(x) for x in ptrs], B, T, H, Dk, Dv, None)

    assert f(ptrs=[None] + p[1:]) == 1               # no xq
    assert f(ptrs=p[:14] + [None] + p[15:]) == 1     # no g
    assert f(B=0) == 1
    assert f(T=0) == 1
    assert f(Dk=96) == 2
    assert f(Dv=32) == 2
    assert f(ptrs=p[:11] + [p[0]] + p[12:]) == 1     # q overlaps xq
    assert f(ptrs=p[:12] + [p[11]] + p[13:]) == 1    # k overlaps q
    assert f(ptrs=p[:16] + [p[12]]) == 1             # conv_out overlaps k
    assert f(ptrs=p[:16] + [p[0]]) == 1              # conv_out overlaps xq
    assert f(ptrs=p[:16] + [p[10] + 4]) == 1         # conv_out partly overlaps conv_in
    assert f(ptrs=p[:5] + [p[5] + 4] + p[6:]) == 1   # taps not 16-byte aligned
    assert f(ptrs=[p[0] + 8] + p[1:]) == 1           # projection not 16-byte aligned


def test_gated_rmsnorm_rejects_bad_arguments():
    lib = gdn.load()
    p = [FAKE + (i << 32) for i in range(4)]         # o z weight y

    def f(ptrs=p, rows=1000, Dv=128, eps=1e-5):
        return lib.gdn_gated_rmsnorm(*[_p(x) for x in ptrs], rows, Dv, eps, None)

    assert f(ptrs=[None] + p[1:]) == 1
    assert f(rows=0) == 1
    assert f(eps=0.0) == 1
    assert f(Dv=96) == 2
    assert f(ptrs=p[:3] + [p[0]]) == 1               # y overlaps o
    assert f(ptrs=p[:3] + [p[1] + 64]) == 1          # y overlaps z
    assert f(ptrs=[p[0] + 8] + p[1:]) == 1           # o not 16-byte aligned


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "lib_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load()


def test_noalloc_rejects_sizes_beyond_its_array():
    """gdn2_chunk_fwd_noalloc refuses, on the host, sizes whose workspace exceeds
    the fixed device array (fake pointers: nothing is launched or touched)."""
    lib = gdn.load()
    cap = lib.gdn2_chunk_fwd_noalloc_max_bytes()
    assert cap == 144 << 20
    B, T, H = 8, 8192, 8          # 8,192 chunk-heads of ~65 KB each
    assert lib.gdn2_chunk_fwd_workspace(B, T, H, 128, 128, 1) > cap
    a = [_p(FAKE + (i << 32)) for i in range(9)]
    assert lib.gdn2_chunk_fwd_noalloc(*a, B, T, H, 128, 128, 1, 0.1, None) == 3
    assert lib.gdn2_chunk_fwd_noalloc(*a, 0, T, H, 128, 128, 1, 0.1, None) == 1
    assert lib.gdn2_chunk_fwd_noalloc(*a, 1, T, H, 96, 128, 1, 0.1, None) == 2

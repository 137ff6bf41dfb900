"""The C-ABI library on the CPU: it builds for gfx950, loads, exports every symbol that
include/kda.h declares, and rejects bad arguments on the host before any launch.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_51_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIBRARY):
        import __graft_entry__

        __graft_entry__.build()
    return kda.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_library_is_built_for_gfx950_only():
    blob = open(kda.LIBRARY, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def test_status_strings(lib):
    for code, name in kda.STATUS.items():
        assert kda.kda_status_string(code).startswith(name)
    assert "unknown" in kda.kda_status_string(99)


def test_workspace_bytes(lib):
    # floor(N/16) + nseq chunk slots, 2 KiB per slot and head
    assert kda.kda_prefill_workspace_bytes(65536, 1, 96, 128, 128) == (4096 + 1) * 96 * 2048
    assert kda.kda_prefill_workspace_bytes(0, 3, 2, 16, 16) == 3 * 2 * 2048
    assert kda.kda_prefill_workspace_bytes(64, 1, 1, 24, 16) == 0   # unsupported dk
    assert kda.kda_prefill_workspace_bytes(64, 0, 1, 16, 16) == 0   # nseq < 1
    assert kda.kda_prefill_workspace_bytes(-1, 1, 1, 16, 16) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, init=None, cu=FAKE, nseq=1, N=64, H=1, dk=16,
             dv=16, dt=kda.KDA_BF16, o=FAKE, fin=None, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.kda_prefill(a["q"], a["k"], a["v"], a["g"], a["b"], a["init"], a["cu"], a["nseq"], a["N"],
                           a["H"], a["dk"], a["dv"], a["dt"], a["o"], a["fin"], a["ws"], a["wsb"], a["stream"])


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, q=None) == 1                 # KDA_ERR_NULL
    assert _prefill(lib, o=None) == 1
    assert _prefill(lib, cu=None) == 1
    assert _prefill(lib, k=FAKE + 2) == 2             # KDA_ERR_ALIGN
    assert _prefill(lib, init=FAKE + 8) == 2
    assert _prefill(lib, nseq=0) == 3                 # KDA_ERR_SHAPE
    assert _prefill(lib, H=0) == 3
    assert _prefill(lib, N=-5) == 3
    assert _prefill(lib, N=1 << 31) == 3
    assert _prefill(lib, dk=24) == 4                  # KDA_ERR_UNSUPPORTED
    assert _prefill(lib, dv=256) == 4
    assert _prefill(lib, dt=7) == 4
    assert _prefill(lib, wsb=100) == 5                # KDA_ERR_WORKSPACE
    assert _prefill(lib, ws=None, wsb=1 << 20) == 5


def test_phase_entry_points_reject_bad_arguments(lib):
    f = lib.kda_chunk_local
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 16, 1, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 48, 1, FAKE, 1 << 20, None) == 4
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 16, 1, FAKE, 16, None) == 5
    g = lib.kda_inter_chunk
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 64, 1, 16, 16, 1, FAKE, 16, FAKE, None, None) == 5
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 64, 1, 16, 16, 1, FAKE, 1 << 20, None, None, None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 64, 0, 16, 16, 1, FAKE, 1 << 20, FAKE, None, None) == 3


def test_decode_rejects_bad_arguments(lib):
    f = lib.kda_decode_step
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 16, 16, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 1, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 16, 16, 1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 80, 1, None) == 4


def test_decode_window_rejects_bad_arguments(lib):
    f = lib.kda_decode_window
    # q k v g beta state o accept B T H dk dv dt stream
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 1, 4, 1, 16, 16, 1, None) == 1
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 1, 16, 16, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 4, 1, 16, 16, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None, 1, 4, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, None, 1, 4, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 4, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 0, 1, 16, 16, 1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 1, 16, 16, 1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1 << 16, 1 << 8, 1 << 7, 16, 16, 1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 1, 16, 24, 1, None) == 4
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 1, 16, 16, 3, None) == 4


def test_python_binding_refuses_cpu_tensors(lib):
    import torch

    x = torch.zeros((16, 1, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_prefill(x, x, x, x, torch.zeros((16, 1), dtype=torch.bfloat16))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        kda.load_library(str(tmp_path / "absent.so"))


def test_layer_passes_reject_bad_arguments(lib):
    g = lib.kda_gate  # z A_log N H dk dt out stream
    assert g(FAKE, None, 8, 2, 16, 1, FAKE, None) == 1
    assert g(None, FAKE, 8, 2, 16, 1, FAKE, None) == 1
    assert g(FAKE + 2, FAKE, 8, 2, 16, 1, FAKE, None) == 2
    assert g(FAKE, FAKE, 8, 0, 16, 1, FAKE, None) == 3
    assert g(FAKE, FAKE, -1, 2, 16, 1, FAKE, None) == 3
    assert g(FAKE, FAKE, 8, 2, 24, 1, FAKE, None) == 4
    c = lib.kda_short_conv  # x w cin cout cu nseq N H d l2 eps dt y stream
    assert c(FAKE, None, None, None, FAKE, 1, 8, 2, 16, 0, 1e-6, 1, FAKE + 64, None) == 1
    assert c(FAKE, FAKE, None, None, None, 1, 8, 2, 16, 0, 1e-6, 1, FAKE + 64, None) == 3  # no cu: nseq == N
    assert c(FAKE, FAKE + 4, None, None, FAKE, 1, 8, 2, 16, 0, 1e-6, 1, FAKE + 64, None) == 2
    assert c(FAKE, FAKE, FAKE + 2, None, FAKE, 1, 8, 2, 16, 0, 1e-6, 1, FAKE + 64, None) == 2
    assert c(FAKE, FAKE, None, None, FAKE, 0, 8, 2, 16, 0, 1e-6, 1, FAKE + 64, None) == 3
    assert c(FAKE, FAKE, None, None, FAKE, 1, 8, 2, 16, 0, -1.0, 1, FAKE + 64, None) == 3
    assert c(FAKE, FAKE, None, None, FAKE, 1, 8, 2, 16, 0, 1e-6, 1, FAKE, None) == 3   # y aliases x
    assert c(FAKE, FAKE, None, None, FAKE, 1, 8, 2, 48, 0, 1e-6, 1, FAKE + 64, None) == 4
    e = lib.kda_out_norm_gate  # o u w eps N H dv dt y stream
    assert e(None, FAKE, FAKE, 1e-6, 8, 2, 16, 1, FAKE, None) == 1
    assert e(FAKE, FAKE, None, 1e-6, 8, 2, 16, 1, FAKE, None) == 1
    assert e(FAKE + 4, FAKE, FAKE, 1e-6, 8, 2, 16, 1, FAKE, None) == 2
    assert e(FAKE, FAKE, FAKE, float("nan"), 8, 2, 16, 1, FAKE, None) == 3
    assert e(FAKE, FAKE, FAKE, 1e-6, 8, 2, 20, 1, FAKE, None) == 4


def test_fused_decode_rejects_bad_arguments(lib):
    f = lib.kda_decode_step_fused  # q k v gate A beta state o u w eps y B H dk dv dt stream
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None, 0.0, None, 1, 1, 16, 16, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 0.0, FAKE, 1, 1, 16, 16, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 0.0, FAKE, 1, 1, 16, 16, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, -1.0, FAKE, 1, 1, 16, 16, 1, None) == 3
    g = lib.kda_decode_window_fused  # q k v gate A beta state o acc u w eps y B T H dk dv dt stream
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, None, 0.0, FAKE, 1, 2, 1, 16, 16, 1,
             None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None, None, 0.0, None, 1, 0, 1, 16, 16, 1,
             None) == 3


def test_decode_layer_step_rejects_bad_arguments(lib):
    f = lib.kda_decode_layer_step  # qkv w cache eps gate A beta state o u nw neps y B H dk dv dt stream
    assert f(FAKE, None, FAKE, 1e-6, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 16, 1,
             None) == 1
    assert f(FAKE, FAKE, None, 1e-6, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 16, 1,
             None) == 1
    assert f(FAKE, FAKE + 4, FAKE, 1e-6, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 16, 1,
             None) == 2
    assert f(FAKE, FAKE, FAKE, -1.0, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 16, 1,
             None) == 3
    assert f(FAKE, FAKE, FAKE, 1e-6, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0, None, 1, 1, 16, 48, 1,
             None) == 4


def test_layer_passes_reject_too_many_rows(lib):
    N, H = 1 << 26, 64  # N * H = 2^32 (token, head) rows
    assert lib.kda_gate(FAKE, FAKE, N, H, 16, 1, FAKE, None) == 3
    assert lib.kda_out_norm_gate(FAKE, FAKE, FAKE, 1e-6, N, H, 16, 1, FAKE, None) == 3
    assert lib.kda_short_conv(FAKE, FAKE, None, None, FAKE, 1, N, H, 16, 0, 1e-6, 1, FAKE + 64, None) == 3


def test_backward_workspace_and_arguments(lib):
    nb = lib.kda_prefill_backward_workspace_bytes(64, 2, 3, 16, 32, 1)
    slots = 64 // 16 + 2
    assert nb == 4 * (2 * slots * 3 * 16 * 32 + 2 * slots * 3 * 16 * 32 + slots * 3 * 4 * 256)
    assert lib.kda_prefill_backward_workspace_bytes(64, 0, 3, 16, 32, 1) == 0
    f = lib.kda_prefill_backward
    # q k v g b init cu nseq N H dk dv dt dO dF dq dk dv dg db dinit ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 64, 1, 16, 16, 1, FAKE, None, FAKE, FAKE, FAKE, FAKE,
            FAKE, None, FAKE, 1 << 30, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a13=None) == 1          # d_o missing
    assert call(a18=None) == 1          # d_log_alpha missing
    assert call(a15=FAKE + 2) == 2      # d_q misaligned
    assert call(a21=None) == 5          # no workspace
    assert call(a22=16) == 5            # workspace too small
    assert call(a10=24) == 4            # dk
    assert call(a7=0) == 3              # nseq


def test_prefill_cp_workspace_and_arguments(lib):
    # per segment and head: S~ and S_in (dk x dv) and M (dk x dk); the chunk-local operands of
    # the segments; the segment list; each region 256-byte aligned
    N, nseq, H, dk, dv, R = 64, 2, 3, 16, 32, 4
    up = lambda x: (x + 255) // 256 * 256
    segs = nseq * R
    cl = (N // 16 + segs) * H * 512 * 4
    want = up(cl) + up((segs + 1) * 4) + 2 * up(segs * H * dk * dv * 4) + up(segs * H * dk * dk * 4)
    assert lib.kda_prefill_cp_workspace_bytes(N, nseq, H, dk, dv, 1, R) == want
    assert lib.kda_prefill_cp_workspace_bytes(N, nseq, H, dk, dv, 1, 0) == 0    # segments < 1
    assert lib.kda_prefill_cp_workspace_bytes(N, nseq, H, dk, dv, 1, 65) == 0   # segments > 64
    f = lib.kda_prefill_cp
    # q k v g b init cu nseq N H dk dv dt R o fin ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 64, 1, 16, 16, 1, 2, FAKE, FAKE, FAKE, 1 << 30, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a13=0) == 3             # no segments
    assert call(a13=65) == 3            # too many segments
    assert call(a14=None) == 1          # o missing
    assert call(a4=None) == 1           # beta missing
    assert call(a16=None) == 5          # no workspace
    assert call(a17=16) == 5            # workspace too small
    assert call(a10=24) == 4            # dk
    assert call(a12=7) == 4             # dtype
    assert call(a15=FAKE + 4) == 2      # final_state misaligned

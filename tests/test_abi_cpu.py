"""The C-ABI library on the CPU: it builds for gfx950, loads, exports every symbol that
include/kda.h declares, and rejects bad arguments on the host before any launch.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest
import torch

import gated_delta_rule_51_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    # KDA_ABI_TEST_LIBRARY: the validation layer built on the CPU with sanitizers
    # (test_sanitizers_cpu.py) instead of the product library
    alt = os.environ.get("KDA_ABI_TEST_LIBRARY")
    if alt:
        return kda.load_library(alt)
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
    assert kda.kda_chunk_workspace_bytes(65536, 1, 96, 128, 128) == (4096 + 1) * 96 * 2048
    assert kda.kda_chunk_workspace_bytes(0, 3, 2, 16, 16) == 3 * 2 * 2048
    # kda_prefill: bf16 with dk = dv = 128 and >= 256 chains runs in one kernel without a workspace
    assert kda.kda_prefill_workspace_bytes(65536, 3, 96, 128, 128) == 0
    assert kda.kda_prefill_workspace_bytes(65536, 1, 96, 128, 128) == (4096 + 1) * 96 * 2048
    assert kda.kda_prefill_workspace_bytes(65536, 1, 96, 128, 128, torch.float32) == (4096 + 1) * 96 * 2048
    assert kda.kda_prefill_workspace_bytes(65536, 1, 96, 64, 128) == (4096 + 1) * 96 * 2048
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


def test_decode_layer_window_replay_rejects_bad_arguments(lib):
    f = lib.kda_decode_layer_window_replay
    # pqkv pg pb replay Tp | qkv g b conv_w cache l2eps A state o u nw neps y B T H dk dv dt ws ws_bytes stream
    base = [FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, FAKE, None, None, 0.0,
            None, 2, 3, 1, 16, 16, kda.KDA_BF16, None, 0, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a3=None) == 1            # replay counts missing with Tp > 0
    assert call(a9=None) == 1            # no convolution cache
    assert call(a8=None) == 1            # no taps
    assert call(a13=None) == 1           # o is required
    assert call(a9=FAKE + 2) == 2        # cache 4-byte aligned
    assert call(a8=FAKE + 4) == 2        # taps 16-byte aligned
    assert call(a10=-1.0) == 3           # l2_eps
    assert call(a4=-1) == 3
    assert call(a19=0) == 3
    assert call(a21=24) == 4
    assert call(a3=None, a4=0, a0=None, a1=None, a2=None, a19=0) == 3  # Tp = 0 allows NULL p*, T still checked
    # the one-chunk form's workspace (bf16, dk = dv = 128, T + Tp = 7): 16-byte aligned, large enough
    need = lib.kda_decode_layer_window_workspace_bytes(2, 3, 4, 1, 128, 128, kda.KDA_BF16)
    assert need == 1024 * 2 * 1 * 7
    assert call(a4=4, a21=128, a22=128, a24=FAKE + 8, a25=need) == 2
    assert call(a4=4, a21=128, a22=128, a24=FAKE, a25=need - 1) == 3


def test_layer_window_workspace_bytes(lib):
    f = lib.kda_decode_layer_window_workspace_bytes
    # B T Tp H dk dv dt: 1,024 bytes per (sequence, head, token) where the one-chunk form serves the shape
    assert f(256, 4, 4, 96, 128, 128, kda.KDA_BF16) == 1024 * 256 * 96 * 8
    assert f(3, 6, 0, 2, 128, 128, kda.KDA_BF16) == 1024 * 3 * 2 * 6
    assert f(3, 16, 0, 2, 128, 128, kda.KDA_BF16) == 1024 * 3 * 2 * 16
    assert f(3, 5, 0, 2, 128, 128, kda.KDA_BF16) == 0     # below 6 tokens: token by token
    assert f(3, 12, 5, 2, 128, 128, kda.KDA_BF16) == 0    # more than one chunk
    assert f(3, 8, 0, 2, 128, 128, kda.KDA_F32) == 0      # bf16 only
    assert f(3, 8, 0, 2, 64, 128, kda.KDA_BF16) == 0      # dk = dv = 128 only
    assert f(0, 8, 0, 2, 128, 128, kda.KDA_BF16) == 0     # invalid shape
    assert f(3, 8, -1, 2, 128, 128, kda.KDA_BF16) == 0
    assert f(1, (1 << 31) - 1, (1 << 31) - 1, 1, 128, 128, kda.KDA_BF16) == 0  # no int overflow in T + Tp


def test_decode_window_form_rejects_bad_arguments(lib):
    f = lib.kda_decode_window_form
    # q k v g beta state o accept B T H dk dv dt form stream
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 128, 128, 1, 3, None) == 3   # no such form
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 128, 128, 1, -1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 128, 128, 0, 2, None) == 4   # chunk: bf16 only
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 64, 128, 1, 2, None) == 4    # dk = dv = 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 17, 1, 128, 128, 1, 2, None) == 4  # one chunk
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 1, 8, 1, 128, 128, 1, 2, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 8, 1, 128, 128, 1, 2, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 0, 1, 128, 128, 1, 1, None) == 3


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


def test_decode_window_replay_rejects_bad_arguments(lib):
    f = lib.kda_decode_window_replay
    # pq pk pv pg pb replay Tp | q k v g A b state o u nw neps y B T H dk dv dt stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 0.0,
            None, 2, 3, 1, 16, 16, kda.KDA_BF16, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a5=None) == 1            # replay counts missing with Tp > 0
    assert call(a0=None) == 1            # previous window's q missing
    assert call(a5=FAKE + 2) == 2        # replay misaligned
    assert call(a1=FAKE + 2) == 2        # previous window's k misaligned
    assert call(a6=-1) == 3              # Tp < 0
    assert call(a20=0) == 3              # T < 1
    assert call(a23=48) == 4             # dv
    assert call(a12=None) == 1           # state missing
    assert call(a14=FAKE, a15=FAKE, a18=FAKE, a13=None) == 1   # epilogue without o


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


def _prefill_layer(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, cin=None, cout=None, l2=1e-6, z=FAKE, A=FAKE, b=FAKE, init=None,
             cu=FAKE, nseq=1, N=64, H=1, dk=128, dv=128, dt=kda.KDA_BF16, ws=FAKE, wsb=1 << 30, o=FAKE, fin=None,
             u=None, nw=None, neps=1e-6, y=None, stream=None)
    a.update(kw)
    return lib.kda_prefill_layer(a["q"], a["k"], a["v"], a["w"], a["cin"], a["cout"], a["l2"], a["z"], a["A"],
                                 a["b"], a["init"], a["cu"], a["nseq"], a["N"], a["H"], a["dk"], a["dv"], a["dt"],
                                 a["ws"], a["wsb"], a["o"], a["fin"], a["u"], a["nw"], a["neps"], a["y"],
                                 a["stream"])


def test_prefill_layer_workspace_and_arguments(lib):
    # the chunk workspace (256-byte aligned end) plus bf16 q, k, log-decay (768 bytes per (token, head))
    ws = (4096 + 1) * 96 * 2048
    assert kda.kda_prefill_layer_workspace_bytes(65536, 1, 96) == ws + 65536 * 96 * 768
    assert kda.kda_prefill_layer_workspace_bytes(17, 2, 3) == 256 * ((1 + 2) * 3 * 2048 // 256) + 17 * 3 * 768
    assert kda.kda_prefill_layer_workspace_bytes(64, 1, 1, 64, 128) == 0              # dk = dv = 128 only
    assert kda.kda_prefill_layer_workspace_bytes(64, 1, 1, 128, 128, torch.float32) == 0
    assert _prefill_layer(lib, q=None) == 1                                            # KDA_ERR_NULL
    assert _prefill_layer(lib, w=None) == 1
    assert _prefill_layer(lib, A=None) == 1
    assert _prefill_layer(lib, o=None) == 1
    assert _prefill_layer(lib, u=FAKE, y=FAKE, nw=None) == 1                           # epilogue without norm_w
    assert _prefill_layer(lib, w=FAKE + 4) == 2                                        # KDA_ERR_ALIGN
    assert _prefill_layer(lib, cin=FAKE + 2) == 2
    assert _prefill_layer(lib, u=FAKE + 8, y=FAKE, nw=FAKE) == 2
    assert _prefill_layer(lib, l2=-1.0) == 3                                           # KDA_ERR_SHAPE
    assert _prefill_layer(lib, u=FAKE, y=FAKE, nw=FAKE, neps=float("inf")) == 3
    assert _prefill_layer(lib, nseq=0) == 3
    assert _prefill_layer(lib, dk=64) == 4                                             # KDA_ERR_UNSUPPORTED
    assert _prefill_layer(lib, dt=kda.KDA_F32) == 4
    assert _prefill_layer(lib, wsb=1000) == 5                                          # KDA_ERR_WORKSPACE
    assert _prefill_layer(lib, ws=None) == 5
    assert _prefill_layer(lib, ws=FAKE + 8) == 2


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


def test_backward_slabbed_workspace_and_arguments(lib):
    # one slab's backward workspace, the slab lists, one state per inner boundary, two adjoints
    up = lambda x: (x + 255) // 256 * 256
    N, H, dk, dv, L = 1000, 3, 32, 64, 256
    nslab = 4
    state = H * dk * dv * 4
    slab_ws = int(lib.kda_prefill_backward_workspace_bytes(L, 1, H, dk, dv, 1))
    want = up(nslab * 8) + up((nslab - 1) * state) + up(2 * state) + up(slab_ws)
    assert kda.kda_prefill_backward_slabbed_workspace_bytes(N, H, dk, dv, L) == want
    assert kda.kda_prefill_backward_slabbed_workspace_bytes(N, H, dk, dv, 100) == 0   # not a multiple of 16
    assert kda.kda_prefill_backward_slabbed_workspace_bytes(N, H, dk, dv, 0) == 0
    # 262,144 tokens x 96 heads in slabs of 16,384: about 15 GB (the unsliced backward: 238 GB)
    assert kda.kda_prefill_backward_slabbed_workspace_bytes(262144, 96, 128, 128, 16384) < 16 * 2**30
    f = lib.kda_prefill_backward_slabbed
    # q k v g b init N H dk dv dt dO dF dq dk dv dg db dinit L ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 1, 16, 16, kda.KDA_BF16, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
            None, 32, FAKE, 1 << 30, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a19=40) == 3          # slab not a multiple of 16
    assert call(a11=None) == 1        # d_o missing
    assert call(a13=FAKE + 2) == 2    # d_q misaligned
    assert call(a21=16) == 5          # workspace too small
    assert call(a20=None) == 5        # no workspace
    assert call(a8=48) == 4           # dk


def test_prefill_cp_workspace_and_arguments(lib):
    # per segment and head: S~ and S_in (dk x dv), M (dk x dk) and a flag; the chunk-local
    # operands of the segments; the segment list; each region 256-byte aligned
    N, nseq, H, dk, dv, R = 64, 2, 3, 16, 32, 4
    up = lambda x: (x + 255) // 256 * 256
    segs = nseq * R
    cl = (N // 16 + segs) * H * 512 * 4
    want = up(cl) + up((segs + 1) * 4) + 2 * up(segs * H * dk * dv * 4) + up(segs * H * dk * dk * 4) + \
        up(segs * H * 4)
    assert lib.kda_prefill_cp_workspace_bytes(N, nseq, H, dk, dv, 1, R) == want
    # kda_prefill takes context parallelism for <= 64 chains of >= 16,384 tokens on average (bf16,
    # dk >= 32), with R = clamp(128 / chains, 2, 16): its workspace is then kda_prefill_cp's
    assert kda.kda_prefill_workspace_bytes(65536, 1, 12, 128, 128) == \
        lib.kda_prefill_cp_workspace_bytes(65536, 1, 12, 128, 128, 1, 10)
    assert kda.kda_prefill_workspace_bytes(65536, 2, 32, 128, 128) == \
        lib.kda_prefill_cp_workspace_bytes(65536, 2, 32, 128, 128, 1, 2)
    assert kda.kda_prefill_workspace_bytes(65536, 1, 65, 128, 128) == (4096 + 1) * 65 * 2048   # 65 chains
    assert kda.kda_prefill_workspace_bytes(16383, 1, 12, 128, 128) == (1023 + 1) * 12 * 2048   # short
    assert kda.kda_prefill_workspace_bytes(65536, 1, 12, 16, 128) == (4096 + 1) * 12 * 2048    # dk = 16
    assert kda.kda_prefill_workspace_bytes(65536, 1, 12, 128, 128, torch.float32) == (4096 + 1) * 12 * 2048
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


def test_launch_limits_are_checked_before_any_launch(lib):
    """Shapes whose launches would exceed 2^32 work-items in a grid dimension (or 32-bit row
    extents) are rejected on the host with KDA_ERR_SHAPE, at each bound."""
    # (sequence, head) chains: nseq * H < 2^20
    assert lib.kda_chunk_workspace_bytes(0, (1 << 20) // 96 + 1, 96, 128, 128, 1) == 0
    assert lib.kda_chunk_workspace_bytes(0, (1 << 20) // 96, 96, 128, 128, 1) > 0
    assert _prefill(lib, nseq=1 << 14, H=64, wsb=1 << 40) == 3
    assert _prefill(lib, nseq=(1 << 14) - 1, H=64, wsb=16) == 5           # in range: fails later, on the workspace
    # 16-token row extents: H * max(dk, dv) < 2^24
    assert _prefill(lib, H=1 << 17, dk=128, dv=16, wsb=1 << 40) == 3
    assert _prefill(lib, H=(1 << 17) - 1, dk=128, dv=16, wsb=16) == 5
    # fp32 chunk-local grid: floor(N/16) + nseq < 2^26 slots
    assert _prefill(lib, N=1 << 30, dt=kda.KDA_F32, wsb=1 << 40) == 3
    assert _prefill(lib, N=1 << 30, dt=kda.KDA_BF16, wsb=16) == 5         # bf16 launches in batches
    # backward per-(slot, head) kernels: slots * H < 2^24
    assert lib.kda_prefill_backward_workspace_bytes(1 << 24, 1, 16, 16, 16, 1) == 0
    assert lib.kda_prefill_backward_workspace_bytes(1 << 24, 1, 15, 16, 16, 1) > 0
    # context-parallel identity / final-copy grids: segs * H * dk * max(dk, dv) < 2^31
    assert lib.kda_prefill_cp_workspace_bytes(64, 64, 64, 128, 128, 1, 32) == 0    # exactly 2^31
    assert lib.kda_prefill_cp_workspace_bytes(64, 64, 64, 128, 128, 1, 16) > 0


def test_noalloc_rejects_problems_above_the_scratch_on_the_host(lib):
    # (floor(N/16) + nseq) * H * 2 KiB > 128 MiB: rejected before the scratch is looked up
    f = lib.kda_prefill_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1 << 20, 96, 64, 128, 1, FAKE, None, None) == 7
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1 << 20, 96, 128, 128, 0, FAKE, None, None) == 7
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1 << 20, 96, 128, 128, 1, FAKE, None, None) == 7
    assert kda.kda_status_string(7).startswith("KDA_ERR_TOO_LARGE")


def test_check_cu_seqlens_rejects_bad_arguments(lib):
    f = lib.kda_check_cu_seqlens  # cu nseq N result stream
    assert f(None, 2, 10, FAKE, None) == 1
    assert f(FAKE, 2, 10, None, None) == 1
    assert f(FAKE + 2, 2, 10, FAKE, None) == 2
    assert f(FAKE, 2, 10, FAKE + 1, None) == 2
    assert f(FAKE, 0, 10, FAKE, None) == 3
    assert f(FAKE, 2, -1, FAKE, None) == 3
    assert f(FAKE, 2, 1 << 31, FAKE, None) == 3

"""MI355X-native Kimi Delta Attention (KDA): Python binding of the C ABI in include/kda.h.

This module only marshals arguments: it checks devices, dtypes and shapes,
allocates outputs and workspaces with torch (device memory is the only thing
torch provides here), and calls the HIP library through ctypes on torch's
current stream.  Every step of the computation runs in the library's kernels;
there is no CPU or PyTorch fallback.  If the library has not been built the
first call raises.

Names mirror the C entry points:
    kda_prefill, kda_prefill_noalloc, kda_chunk_local, kda_inter_chunk, kda_decode_step,
    kda_decode_window, kda_prefill_workspace_bytes, kda_status_string,
    kda_gate, kda_short_conv, kda_out_norm_gate (the layer's passes around the recurrence).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libkda_mi355x.so")
CHUNK = 16
GATE_LOWER_BOUND = -5.0

KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_ALIGN", 3: "KDA_ERR_SHAPE",
          4: "KDA_ERR_UNSUPPORTED", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_HIP", 7: "KDA_ERR_TOO_LARGE"}
EXPORTS = ("kda_prefill_workspace_bytes", "kda_chunk_workspace_bytes", "kda_prefill", "kda_prefill_single_pass",
           "kda_inter_chunk_shaped", "kda_prefill_noalloc", "kda_chunk_local", "kda_inter_chunk",
           "kda_decode_step", "kda_decode_window", "kda_decode_window_form", "kda_decode_step_fused",
           "kda_decode_window_fused",
           "kda_decode_window_replay", "kda_decode_layer_window_replay", "kda_decode_layer_window_workspace_bytes",
           "kda_decode_layer_step", "kda_prefill_backward_workspace_bytes", "kda_prefill_backward",
           "kda_prefill_backward_slabbed_workspace_bytes", "kda_prefill_backward_slabbed",
           "kda_prefill_cp_workspace_bytes", "kda_prefill_cp",
           "kda_gate", "kda_short_conv", "kda_out_norm_gate", "kda_prefill_layer_workspace_bytes",
           "kda_prefill_layer", "kda_check_cu_seqlens", "kda_status_string", "kda_last_hip_error")

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"KDA HIP library not found at {path}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_prefill_workspace_bytes.restype = sz
    lib.kda_prefill_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_workspace_bytes.restype = sz
    lib.kda_chunk_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                vp, vp, vp, sz, vp]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                        vp, vp, vp]
    lib.kda_prefill_single_pass.restype = ctypes.c_int
    lib.kda_prefill_single_pass.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                            i32, i32, vp, vp, vp]
    lib.kda_inter_chunk_shaped.restype = ctypes.c_int
    lib.kda_inter_chunk_shaped.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                           vp, sz, i32, i32, vp, vp, vp]
    lib.kda_chunk_local.restype = ctypes.c_int
    lib.kda_chunk_local.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, ctypes.c_int, vp, sz, vp]
    lib.kda_inter_chunk.restype = ctypes.c_int
    lib.kda_inter_chunk.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                    vp, sz, vp, vp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.kda_decode_window.restype = ctypes.c_int
    lib.kda_decode_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                      vp]
    lib.kda_decode_window_form.restype = ctypes.c_int
    lib.kda_decode_window_form.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                           i32, vp]
    i64, f32 = ctypes.c_int64, ctypes.c_float
    lib.kda_decode_step_fused.restype = ctypes.c_int
    lib.kda_decode_step_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32,
                                          ctypes.c_int, vp]
    lib.kda_decode_window_fused.restype = ctypes.c_int
    lib.kda_decode_window_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32,
                                            i32, i32, ctypes.c_int, vp]
    lib.kda_decode_window_replay.restype = ctypes.c_int
    lib.kda_decode_window_replay.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             f32, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.kda_decode_layer_window_replay.restype = ctypes.c_int
    lib.kda_decode_layer_window_replay.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                                   f32, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp,
                                                   ctypes.c_size_t, vp]
    lib.kda_decode_layer_window_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_decode_layer_window_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_decode_layer_step.restype = ctypes.c_int
    lib.kda_decode_layer_step.argtypes = [vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32,
                                          i32, ctypes.c_int, vp]
    lib.kda_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_backward_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_prefill_backward.restype = ctypes.c_int
    lib.kda_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_prefill_backward_slabbed_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_backward_slabbed_workspace_bytes.argtypes = [i64, i32, i32, i32, ctypes.c_int, i64]
    lib.kda_prefill_backward_slabbed.restype = ctypes.c_int
    lib.kda_prefill_backward_slabbed.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, ctypes.c_int, vp, vp,
                                                 vp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
    lib.kda_prefill_cp_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_cp_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int, i32]
    lib.kda_prefill_cp.restype = ctypes.c_int
    lib.kda_prefill_cp.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int, i32,
                                   vp, vp, vp, ctypes.c_size_t, vp]
    lib.kda_gate.restype = ctypes.c_int
    lib.kda_gate.argtypes = [vp, vp, i64, i32, i32, ctypes.c_int, vp, vp]
    lib.kda_short_conv.restype = ctypes.c_int
    lib.kda_short_conv.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, ctypes.c_int, vp, vp]
    lib.kda_out_norm_gate.restype = ctypes.c_int
    lib.kda_out_norm_gate.argtypes = [vp, vp, vp, f32, i64, i32, i32, ctypes.c_int, vp, vp]
    lib.kda_prefill_layer_workspace_bytes.restype = sz
    lib.kda_prefill_layer_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_prefill_layer.restype = ctypes.c_int
    lib.kda_prefill_layer.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                      ctypes.c_int, vp, sz, vp, vp, vp, vp, f32, vp, vp]
    lib.kda_check_cu_seqlens.restype = ctypes.c_int
    lib.kda_check_cu_seqlens.argtypes = [vp, i32, i64, vp, vp]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_hip_error.restype = i32
    lib.kda_last_hip_error.argtypes = []
    if path == LIBRARY:
        _lib = lib
    return lib


def kda_status_string(code: int) -> str:
    return load_library().kda_status_string(int(code)).decode()


def _check(code: int) -> None:
    if code != 0:
        lib = load_library()
        msg = lib.kda_status_string(code).decode()
        if code == 6:
            msg += f" (hipError {lib.kda_last_hip_error()})"
        raise KDAError(code, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KDA_BF16
    if t == torch.float32:
        return KDA_F32
    raise TypeError(f"KDA inputs must be bfloat16 or float32, got {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_tensors(q, k, v, log_alpha, beta):
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU (got {t.device}); the KDA library has no CPU path")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, log_alpha and beta must share one dtype")


def _check_inputs(q, k, v, log_alpha, beta):
    _check_tensors(q, k, v, log_alpha, beta)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (N, H, dk) or log_alpha.shape != (N, H, dk) or v.shape != (N, H, dv) or beta.shape != (N, H):
        raise ValueError("expected q, k, log_alpha [N, H, dk], v [N, H, dv], beta [N, H]")
    return N, H, dk, dv


def _check_dev(name, t, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device}); the KDA library has no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_gpu(name, t):
    """t is a contiguous tensor on a GPU (the first operand, whose device the others must share)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); the KDA library has no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws, device, nbytes: int):
    """A caller-supplied workspace: a contiguous tensor on the inputs' device of at least nbytes."""
    _check_dev("workspace", ws, device)
    have = ws.numel() * ws.element_size()
    if have < nbytes:
        raise ValueError(f"workspace holds {have} bytes, {nbytes} needed")


def _prefill_outputs(N, H, dk, dv, nseq, device, o, final_state, init_state, output_final_state):
    """Allocate or check kda_prefill's outputs (o fp32 [N, H, dv], final_state fp32 [nseq, H, dk, dv])
    and check init_state, so no wrong-sized or host buffer reaches a kernel."""
    if o is None:
        o = torch.empty((N, H, dv), dtype=torch.float32, device=device)
    _check_dev("o", o, device, torch.float32, (N, H, dv))
    if output_final_state and final_state is None:
        final_state = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=device)
    if final_state is not None:
        _check_dev("final_state", final_state, device, torch.float32, (nseq, H, dk, dv))
    if init_state is not None:
        _check_dev("init_state", init_state, device, torch.float32, (nseq, H, dk, dv))
    return o, final_state


def kda_prefill_workspace_bytes(total_tokens: int, nseq: int, H: int, dk: int, dv: int,
                                dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes kda_prefill needs (0: none -- bf16 with dk = dv = 128 and at least 256
    (sequence, head) chains runs in one kernel)."""
    return int(load_library().kda_prefill_workspace_bytes(total_tokens, nseq, H, dk, dv, _dtype_code(dtype)))


def kda_chunk_workspace_bytes(total_tokens: int, nseq: int, H: int, dk: int, dv: int,
                              dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of the two phases (kda_chunk_local, kda_inter_chunk)."""
    return int(load_library().kda_chunk_workspace_bytes(total_tokens, nseq, H, dk, dv, _dtype_code(dtype)))


def _cu(cu_seqlens, N, device):
    if cu_seqlens is None:
        return torch.tensor([0, N], dtype=torch.int32, device=device)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor on the inputs' device")
    return cu_seqlens


def alloc_workspace(total_tokens: int, nseq: int, H: int, dk: int, dv: int, dtype, device) -> torch.Tensor:
    """A workspace for the two phases (kda_chunk_local, kda_inter_chunk)."""
    nbytes = kda_chunk_workspace_bytes(total_tokens, nseq, H, dk, dv, dtype)
    return torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=device)


def kda_prefill(q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None, *,
                output_final_state: bool = True, o=None, final_state=None, workspace=None,
                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill over packed sequences (see include/kda.h).

    q, k, log_alpha: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; one dtype (bf16 or fp32).
    cu_seqlens: int32 [nseq + 1] on the device (None = one sequence of N tokens).
    init_state: fp32 [nseq, H, dk, dv] or None.  Returns (o fp32 [N, H, dv], final_state).
    """
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    cu = _cu(cu_seqlens, N, q.device)
    nseq = cu.numel() - 1
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, q.device, o, final_state, init_state,
                                      output_final_state)
    nbytes = kda_prefill_workspace_bytes(N, nseq, H, dk, dv, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, q.device, nbytes)
    _check(load_library().kda_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N,
        H, dk, dv, _dtype_code(q.dtype), _ptr(o), _ptr(final_state), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, final_state


def kda_prefill_layer_workspace_bytes(total_tokens: int, nseq: int, H: int, dk: int = 128, dv: int = 128,
                                      dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of kda_prefill_layer (0: shape not supported)."""
    return int(load_library().kda_prefill_layer_workspace_bytes(total_tokens, nseq, H, dk, dv, _dtype_code(dtype)))


def kda_prefill_layer(q, k, v, conv_w, z, A_log, beta, cu_seqlens=None, init_state=None, *, conv_cache=None,
                      conv_cache_out=None, l2_eps: float = 1e-6, out_gate=None, norm_w=None, norm_eps: float = 1e-6,
                      output_final_state: bool = True, o=None, final_state=None, y=None, workspace=None,
                      stream=None):
    """The layer core of a prefill with the prologue fused into the recurrence's loads (see
    include/kda.h): q, k, v raw projections [N, H, 128] (bf16), conv_w fp32 [H, 384, 4] (q | k | v
    channels), z decay logits [N, H, 128], A_log fp32 [H], beta [N, H]; conv_cache / conv_cache_out
    fp32 [nseq, H, 384, 3] (or None); out_gate [N, H, 128] with norm_w fp32 [128] adds the epilogue.
    Returns (o fp32 [N, H, 128], final_state or None, y or None)."""
    N, H, dk, dv = _check_inputs(q, k, v, z, beta)
    dev = q.device
    C = 2 * dk + dv
    cu = _cu(cu_seqlens, N, dev)
    nseq = cu.numel() - 1
    _check_dev("conv_w", conv_w, dev, torch.float32, (H, C, 4))
    _check_dev("A_log", A_log, dev, torch.float32, (H,))
    for name, c in (("conv_cache", conv_cache), ("conv_cache_out", conv_cache_out)):
        if c is not None:
            _check_dev(name, c, dev, torch.float32, (nseq, H, C, 3))
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, dev, o, final_state, init_state, output_final_state)
    if out_gate is not None:
        _check_dev("out_gate", out_gate, dev, q.dtype, (N, H, dv))
        _check_dev("norm_w", norm_w, dev, torch.float32, (dv,))
        if y is None:
            y = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
        _check_dev("y", y, dev, q.dtype, (N, H, dv))
    nbytes = kda_prefill_layer_workspace_bytes(N, nseq, H, dk, dv, q.dtype)
    if nbytes == 0:
        raise KDAError(4, "kda_prefill_layer: bf16 with dk = dv = 128 only")
    if workspace is None:
        workspace = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=dev)
    _check_workspace(workspace, dev, nbytes)
    _check(load_library().kda_prefill_layer(
        _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w), _ptr(conv_cache), _ptr(conv_cache_out), float(l2_eps), _ptr(z),
        _ptr(A_log), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N, H, dk, dv, _dtype_code(q.dtype),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(o), _ptr(final_state),
        _ptr(out_gate), _ptr(norm_w), float(norm_eps), _ptr(y if out_gate is not None else None),
        _stream(stream)))
    return o, final_state, (y if out_gate is not None else None)


def kda_prefill_single_pass(q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None, *, consumers: int = 0,
                            slices: int = 0, output_final_state: bool = True, o=None, final_state=None,
                            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The single-pass prefill kernel (bf16, dk = dv = 128) with an explicit workgroup shape
    (consumers, slices) in {(2, 1), (4, 1), (4, 2)}; (0, 0) chooses.  For tuning and tests."""
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    cu = _cu(cu_seqlens, N, q.device)
    nseq = cu.numel() - 1
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, q.device, o, final_state, init_state,
                                      output_final_state)
    _check(load_library().kda_prefill_single_pass(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N,
        H, dk, dv, _dtype_code(q.dtype), int(consumers), int(slices), _ptr(o), _ptr(final_state),
        _stream(stream)))
    return o, final_state


def kda_prefill_noalloc(q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None, *,
                        output_final_state: bool = True, o=None, final_state=None,
                        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_prefill with the workspace in the library's static device scratch (no device
    allocation by the library; pass ``o`` and ``final_state`` to allocate nothing here either).
    Problems above the scratch size raise KDAError (KDA_ERR_TOO_LARGE); calls that overlap on one
    GPU race on the shared scratch."""
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    cu = _cu(cu_seqlens, N, q.device)
    nseq = cu.numel() - 1
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, q.device, o, final_state, init_state,
                                      output_final_state)
    _check(load_library().kda_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N,
        H, dk, dv, _dtype_code(q.dtype), _ptr(o), _ptr(final_state), _stream(stream)))
    return o, final_state


def kda_prefill_cp(q, k, v, log_alpha, beta, cu_seqlens=None, init_state=None, *, segments: int = 2,
                   output_final_state: bool = True, o=None, final_state=None, workspace=None,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_prefill with every sequence split into ``segments`` chunk-aligned pieces run as
    independent chains, their incoming states recovered by a scan (see include/kda.h).
    Same arguments and results as kda_prefill."""
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    cu = _cu(cu_seqlens, N, q.device)
    nseq = cu.numel() - 1
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, q.device, o, final_state, init_state,
                                      output_final_state)
    lib = load_library()
    nbytes = int(lib.kda_prefill_cp_workspace_bytes(N, nseq, H, dk, dv, _dtype_code(q.dtype), int(segments)))
    if nbytes == 0:
        raise KDAError(3, "kda_prefill_cp: unsupported shape or segment count")
    if workspace is None:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    _check_workspace(workspace, q.device, nbytes)
    _check(lib.kda_prefill_cp(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N,
        H, dk, dv, _dtype_code(q.dtype), int(segments), _ptr(o), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, final_state


def kda_chunk_local(q, k, log_alpha, beta, cu_seqlens, workspace, *, stream=None) -> torch.Tensor:
    """Chunk-local phase only; writes T' and A_qk per (chunk slot, head) into ``workspace``."""
    _check_gpu("q", q)
    for name, t in (("k", k), ("log_alpha", log_alpha), ("beta", beta)):
        _check_dev(name, t, q.device, q.dtype)
    N, H, dk = q.shape
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(beta.shape) != (N, H):
        raise ValueError("expected q, k, log_alpha [N, H, dk], beta [N, H]")
    _check_dev("cu_seqlens", cu_seqlens, q.device, torch.int32)
    nseq = cu_seqlens.numel() - 1
    _check_workspace(workspace, q.device, kda_chunk_workspace_bytes(N, nseq, H, dk, 16, q.dtype))
    _check(load_library().kda_chunk_local(
        _ptr(q), _ptr(k), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), nseq, N, H, dk,
        _dtype_code(q.dtype), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace


def kda_inter_chunk(q, k, v, log_alpha, cu_seqlens, workspace, init_state=None, *, o=None,
                    final_state=None, output_final_state: bool = True, consumers: int = 0, producers: int = 0,
                    stream=None):
    """Inter-chunk phase only; reads the workspace written by kda_chunk_local.  ``consumers`` and
    ``producers`` pick the warp-specialised kernel's workgroup shape (0, 0 = choose)."""
    _check_gpu("q", q)
    for name, t in (("k", k), ("v", v), ("log_alpha", log_alpha)):
        _check_dev(name, t, q.device, q.dtype)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(v.shape) != (N, H, dv):
        raise ValueError("expected q, k, log_alpha [N, H, dk], v [N, H, dv]")
    _check_dev("cu_seqlens", cu_seqlens, q.device, torch.int32)
    nseq = cu_seqlens.numel() - 1
    o, final_state = _prefill_outputs(N, H, dk, dv, nseq, q.device, o, final_state, init_state,
                                      output_final_state)
    _check_workspace(workspace, q.device, kda_chunk_workspace_bytes(N, nseq, H, dk, dv, q.dtype))
    _check(load_library().kda_inter_chunk_shaped(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(init_state), _ptr(cu_seqlens), nseq, N, H,
        dk, dv, _dtype_code(q.dtype), _ptr(workspace), workspace.numel() * workspace.element_size(),
        int(consumers), int(producers), _ptr(o), _ptr(final_state), _stream(stream)))
    return o, final_state


def kda_decode_step(q, k, v, log_alpha, beta, state, *, o=None, stream=None) -> torch.Tensor:
    """One decode token for B x H heads; ``state`` (fp32 [B, H, dk, dv]) is updated in place.

    q, k, log_alpha: [B, H, dk]; v: [B, H, dv]; beta: [B, H].  Returns o fp32 [B, H, dv].
    """
    B, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv) or not state.is_contiguous() \
            or state.device != q.device:
        raise ValueError("state must be contiguous fp32 [B, H, dk, dv] on the inputs' device")
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    _check_dev("o", o, q.device, torch.float32, (B, H, dv))
    _check(load_library().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state), _ptr(o), B, H, dk, dv,
        _dtype_code(q.dtype), _stream(stream)))
    return o


def kda_decode_window(q, k, v, log_alpha, beta, state, accept=None, *, o=None, output_o: bool = True,
                      form=None, stream=None) -> Optional[torch.Tensor]:
    """A window of T tokens per sequence (speculative verification); ``state`` is updated in place.

    q, k, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H].  ``accept``: int32 [B] on
    the device (None = all T accepted); the state ends after the first clamp(accept[b], 0, T)
    tokens of sequence b.  Returns o fp32 [B, T, H, dv] (the output of every token of the
    window), or None with ``output_o=False``.  ``form`` (kda_decode_window_form): None or 0 =
    automatic, 1 = token by token, 2 = one chunk on the matrix cores.
    """
    _check_tensors(q, k, v, log_alpha, beta)
    if q.dim() != 4:
        raise ValueError("expected q, k, log_alpha [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, dk) or log_alpha.shape != (B, T, H, dk) or v.shape != (B, T, H, dv) \
            or beta.shape != (B, T, H):
        raise ValueError("expected q, k, log_alpha [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv) or not state.is_contiguous() \
            or state.device != q.device:
        raise ValueError("state must be contiguous fp32 [B, H, dk, dv] on the inputs' device")
    if accept is not None and (accept.dtype != torch.int32 or tuple(accept.shape) != (B,)
                               or accept.device != q.device or not accept.is_contiguous()):
        raise ValueError("accept must be a contiguous int32 [B] tensor on the inputs' device")
    if output_o and o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if output_o:
        _check_dev("o", o, q.device, torch.float32, (B, T, H, dv))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state), _ptr(o if output_o else None),
            _ptr(accept), B, T, H, dk, dv, _dtype_code(q.dtype))
    if form is None:
        _check(load_library().kda_decode_window(*args, _stream(stream)))
    else:
        _check(load_library().kda_decode_window_form(*args, int(form), _stream(stream)))
    return o if output_o else None


def kda_gate(z, A_log, *, out=None, stream=None) -> torch.Tensor:
    """Bounded decay gate log_alpha = -5 * Sigmoid(exp(A_log[h]) * z); z [N, H, dk] (bf16 or fp32),
    A_log fp32 [H].  Returns log_alpha in z's dtype (``out`` may be z itself)."""
    if not isinstance(z, torch.Tensor) or z.device.type != "cuda":
        raise ValueError("z must be a tensor on a GPU; the KDA library has no CPU path")
    N, H, dk = z.shape
    _check_dev("z", z, z.device)
    _check_dev("A_log", A_log, z.device, torch.float32, (H,))
    if out is None:
        out = torch.empty_like(z)
    _check_dev("out", out, z.device, z.dtype, z.shape)
    _check(load_library().kda_gate(_ptr(z), _ptr(A_log), N, H, dk, _dtype_code(z.dtype), _ptr(out),
                                   _stream(stream)))
    return out


def kda_short_conv(x, w, cu_seqlens=None, cache=None, *, l2norm: bool = False, eps: float = 1e-6,
                   cache_out=None, y=None, stream=None):
    """ShortConv prologue: y = Swish(causal 4-tap depthwise convolution of x) [L2-normalised over d].

    x [N, H, d] (bf16 or fp32); w fp32 [H, d, 4] (tap j multiplies x_{t-j}); cu_seqlens int32
    [nseq + 1] on the device (None = one sequence; "decode" = every token its own sequence, as in a
    decode step); cache fp32 [nseq, H, d, 3] (the 3 inputs before each sequence, oldest first) or
    None.  Returns (y, cache_out) with cache_out the 3 last inputs
    per sequence (``cache_out`` may be ``cache`` to update it in place).
    """
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a tensor on a GPU; the KDA library has no CPU path")
    N, H, d = x.shape
    if isinstance(cu_seqlens, str) and cu_seqlens == "decode":  # one token per sequence
        cu, nseq = None, N
    else:
        cu = _cu(cu_seqlens, N, x.device)
        nseq = cu.numel() - 1
    _check_dev("x", x, x.device)
    _check_dev("w", w, x.device, torch.float32, (H, d, 4))
    if cache is not None:
        _check_dev("cache", cache, x.device, torch.float32, (nseq, H, d, 3))
    if cache_out is None:
        cache_out = torch.empty((nseq, H, d, 3), dtype=torch.float32, device=x.device)
    _check_dev("cache_out", cache_out, x.device, torch.float32, (nseq, H, d, 3))
    if y is None:
        y = torch.empty_like(x)
    _check_dev("y", y, x.device, x.dtype, x.shape)
    _check(load_library().kda_short_conv(
        _ptr(x), _ptr(w), _ptr(cache), _ptr(cache_out), _ptr(cu), nseq, N, H, d, int(bool(l2norm)),
        float(eps), _dtype_code(x.dtype), _ptr(y), _stream(stream)))
    return y, cache_out


def kda_out_norm_gate(o, u, w, eps: float = 1e-6, *, y=None, stream=None) -> torch.Tensor:
    """Output epilogue y = Sigmoid(u) * RMSNorm(o) * w per (token, head); o fp32 [N, H, dv], u [N, H, dv]
    (bf16 or fp32), w fp32 [dv].  Returns y in u's dtype."""
    if not isinstance(o, torch.Tensor) or o.device.type != "cuda":
        raise ValueError("o must be a tensor on a GPU; the KDA library has no CPU path")
    N, H, dv = o.shape
    _check_dev("o", o, o.device, torch.float32)
    _check_dev("u", u, o.device, None, (N, H, dv))
    _check_dev("w", w, o.device, torch.float32, (dv,))
    if y is None:
        y = torch.empty_like(u)
    _check_dev("y", y, o.device, u.dtype, u.shape)
    _check(load_library().kda_out_norm_gate(_ptr(o), _ptr(u), _ptr(w), float(eps), N, H, dv,
                                            _dtype_code(u.dtype), _ptr(y), _stream(stream)))
    return y


def _fusion_args(o_shape, dtype, device, H, dv, gate_A_log, out_gate, norm_w, y, want_y):
    if gate_A_log is not None:
        _check_dev("gate_A_log", gate_A_log, device, torch.float32, (H,))
    if out_gate is None:
        return None
    _check_dev("out_gate", out_gate, device, dtype, o_shape)
    _check_dev("norm_w", norm_w, device, torch.float32, (dv,))
    if y is None and want_y:
        y = torch.empty(o_shape, dtype=dtype, device=device)
    _check_dev("y", y, device, dtype, o_shape)
    return y


def kda_decode_step_fused(q, k, v, gate, beta, state, *, gate_A_log=None, out_gate=None, norm_w=None,
                          norm_eps: float = 1e-6, o=None, output_o: bool = True, y=None, stream=None):
    """kda_decode_step with the layer's gate (``gate_A_log``: ``gate`` holds decay logits) and
    output epilogue (``out_gate``, ``norm_w``: y = Sigmoid(out_gate) RMSNorm(o) norm_w) fused in.
    Returns (o or None, y or None)."""
    B, H, dk, dv = _check_inputs(q, k, v, gate, beta)
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv) or not state.is_contiguous() \
            or state.device != q.device:
        raise ValueError("state must be contiguous fp32 [B, H, dk, dv] on the inputs' device")
    y = _fusion_args((B, H, dv), q.dtype, q.device, H, dv, gate_A_log, out_gate, norm_w, y, True)
    if not output_o and out_gate is None:
        raise ValueError("output_o=False needs out_gate (nothing would be written)")
    if output_o and o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    if output_o:
        _check_dev("o", o, q.device, torch.float32, (B, H, dv))
    _check(load_library().kda_decode_step_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(gate_A_log), _ptr(beta), _ptr(state),
        _ptr(o if output_o else None), _ptr(out_gate), _ptr(norm_w), float(norm_eps), _ptr(y), B, H, dk, dv,
        _dtype_code(q.dtype), _stream(stream)))
    return (o if output_o else None), y


def kda_decode_window_fused(q, k, v, gate, beta, state, accept=None, *, gate_A_log=None, out_gate=None,
                            norm_w=None, norm_eps: float = 1e-6, o=None, output_o: bool = True, y=None,
                            stream=None):
    """kda_decode_window with the gate and output epilogue fused in (see kda_decode_step_fused);
    out_gate and y are [B, T, H, dv].  Returns (o or None, y or None)."""
    _check_tensors(q, k, v, gate, beta)
    if q.dim() != 4:
        raise ValueError("expected q, k, gate [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, dk) or gate.shape != (B, T, H, dk) or v.shape != (B, T, H, dv) \
            or beta.shape != (B, T, H):
        raise ValueError("expected q, k, gate [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv) or not state.is_contiguous() \
            or state.device != q.device:
        raise ValueError("state must be contiguous fp32 [B, H, dk, dv] on the inputs' device")
    if accept is not None:
        _check_dev("accept", accept, q.device, torch.int32, (B,))
    y = _fusion_args((B, T, H, dv), q.dtype, q.device, H, dv, gate_A_log, out_gate, norm_w, y, True)
    # the window's epilogue runs over o, so o is materialised whenever out_gate is given
    if (output_o or out_gate is not None) and o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if o is not None:
        _check_dev("o", o, q.device, torch.float32, (B, T, H, dv))
    _check(load_library().kda_decode_window_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(gate_A_log), _ptr(beta), _ptr(state),
        _ptr(o), _ptr(accept), _ptr(out_gate), _ptr(norm_w), float(norm_eps), _ptr(y),
        B, T, H, dk, dv, _dtype_code(q.dtype), _stream(stream)))
    return (o if output_o else None), y


def kda_decode_window_replay(prev, replay, q, k, v, gate, beta, state, *, gate_A_log=None, out_gate=None,
                             norm_w=None, norm_eps: float = 1e-6, o=None, y=None, stream=None):
    """One speculative-decoding call as a serving loop makes it: replay the accepted prefix of
    the previous window (``prev`` = dict or tuple of its q, k, v, gate, beta [B, Tp, H, .] or
    None; ``replay`` int32 [B] accepted counts, known only now), commit the state after it, then
    run this window's T tokens (q, k, v, gate [B, T, H, .], beta [B, T, H]) without committing
    them.  Returns (o [B, T, H, dv], y or None)."""
    _check_tensors(q, k, v, gate, beta)
    if q.dim() != 4:
        raise ValueError("expected q, k, gate [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, dk) or gate.shape != (B, T, H, dk) or v.shape != (B, T, H, dv) \
            or beta.shape != (B, T, H):
        raise ValueError("expected q, k, gate [B, T, H, dk], v [B, T, H, dv], beta [B, T, H]")
    _check_dev("state", state, q.device, torch.float32, (B, H, dk, dv))
    Tp = 0
    p = (None,) * 5
    if prev is not None:
        p = tuple(prev[n] for n in ("q", "k", "v", "gate", "beta")) if isinstance(prev, dict) else tuple(prev)
        Tp = p[0].shape[1]
        for name, t, shp in zip(("q", "k", "v", "gate", "beta"), p,
                                ((B, Tp, H, dk), (B, Tp, H, dk), (B, Tp, H, dv), (B, Tp, H, dk), (B, Tp, H))):
            _check_dev("prev " + name, t, q.device, q.dtype, shp)
        _check_dev("replay", replay, q.device, torch.int32, (B,))
    y = _fusion_args((B, T, H, dv), q.dtype, q.device, H, dv, gate_A_log, out_gate, norm_w, y, True)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    _check_dev("o", o, q.device, torch.float32, (B, T, H, dv))
    _check(load_library().kda_decode_window_replay(
        *(_ptr(t) for t in p), _ptr(replay if Tp > 0 else None), Tp, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
        _ptr(gate_A_log), _ptr(beta), _ptr(state), _ptr(o), _ptr(out_gate), _ptr(norm_w), float(norm_eps), _ptr(y),
        B, T, H, dk, dv, _dtype_code(q.dtype), _stream(stream)))
    return o, y


def kda_decode_layer_step(qkv, conv_w, conv_cache, gate, beta, state, *, dk: int, l2_eps: float = 1e-6,
                          gate_A_log=None, out_gate=None, norm_w=None, norm_eps: float = 1e-6, o=None,
                          output_o: bool = True, y=None, stream=None):
    """One decode step of the layer core in one launch: ShortConv + Swish (+ L2 for q, k) of the
    new token from ``conv_cache`` (updated in place), the gate, the recurrence and the epilogue.

    qkv [B, H, 2 dk + dv] (q | k | v channels per head); conv_w fp32 [H, 2 dk + dv, 4]; conv_cache
    fp32 [B, H, 2 dk + dv, 3]; gate [B, H, dk] (decay logits with ``gate_A_log``, else log-decay);
    beta [B, H]; state fp32 [B, H, dk, dv].  Returns (o or None, y or None)."""
    if not isinstance(qkv, torch.Tensor) or qkv.device.type != "cuda":
        raise ValueError("qkv must be a tensor on a GPU; the KDA library has no CPU path")
    B, H, C = qkv.shape
    dv = C - 2 * dk
    dev = qkv.device
    _check_dev("qkv", qkv, dev)
    _check_dev("conv_w", conv_w, dev, torch.float32, (H, C, 4))
    _check_dev("conv_cache", conv_cache, dev, torch.float32, (B, H, C, 3))
    _check_dev("gate", gate, dev, qkv.dtype, (B, H, dk))
    _check_dev("beta", beta, dev, qkv.dtype, (B, H))
    _check_dev("state", state, dev, torch.float32, (B, H, dk, dv))
    y = _fusion_args((B, H, dv), qkv.dtype, dev, H, dv, gate_A_log, out_gate, norm_w, y, True)
    if not output_o and out_gate is None:
        raise ValueError("output_o=False needs out_gate (nothing would be written)")
    if output_o and o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    if output_o:
        _check_dev("o", o, dev, torch.float32, (B, H, dv))
    _check(load_library().kda_decode_layer_step(
        _ptr(qkv), _ptr(conv_w), _ptr(conv_cache), float(l2_eps), _ptr(gate), _ptr(gate_A_log), _ptr(beta),
        _ptr(state), _ptr(o if output_o else None), _ptr(out_gate), _ptr(norm_w), float(norm_eps), _ptr(y),
        B, H, dk, dv, _dtype_code(qkv.dtype), _stream(stream)))
    return (o if output_o else None), y


def kda_decode_layer_window_workspace_bytes(B: int, T: int, Tp: int, H: int, dk: int, dv: int, dtype) -> int:
    """Workspace bytes of kda_decode_layer_window_replay's one-chunk form (0: the shape runs token by token)."""
    return int(load_library().kda_decode_layer_window_workspace_bytes(B, T, Tp, H, dk, dv, _dtype_code(dtype)))


def kda_decode_layer_window_replay(prev, replay, qkv, gate, beta, conv_w, conv_cache, state, *, dk: int,
                                   l2_eps: float = 1e-6, gate_A_log=None, out_gate=None, norm_w=None,
                                   norm_eps: float = 1e-6, o=None, y=None, form=None, workspace=None, stream=None):
    """The layer core's speculative-decoding call: replay the previous window's accepted prefix
    (``prev`` = dict or tuple of its qkv, gate, beta [B, Tp, H, .] or None; ``replay`` int32 [B])
    through ShortConv (+ L2 for q, k), the gate and the recurrence, commit state and
    ``conv_cache`` after it, then run this window's T tokens (qkv [B, T, H, 2 dk + dv], gate
    [B, T, H, dk], beta [B, T, H]) without committing them.  Returns (o [B, T, H, dv], y or None).
    ``form``: None chooses (the one-chunk form where the library serves the shape, with a
    workspace allocated here unless ``workspace`` is given), 1 token by token, 2 the one-chunk
    form (ValueError where the shape has none)."""
    if not isinstance(qkv, torch.Tensor) or qkv.device.type != "cuda":
        raise ValueError("qkv must be a tensor on a GPU; the KDA library has no CPU path")
    if qkv.dim() != 4:
        raise ValueError("expected qkv [B, T, H, 2 dk + dv]")
    B, T, H, C = qkv.shape
    dv = C - 2 * dk
    dev = qkv.device
    _check_dev("qkv", qkv, dev)
    _check_dev("gate", gate, dev, qkv.dtype, (B, T, H, dk))
    _check_dev("beta", beta, dev, qkv.dtype, (B, T, H))
    _check_dev("conv_w", conv_w, dev, torch.float32, (H, C, 4))
    _check_dev("conv_cache", conv_cache, dev, torch.float32, (B, H, C, 3))
    _check_dev("state", state, dev, torch.float32, (B, H, dk, dv))
    Tp = 0
    p = (None,) * 3
    if prev is not None:
        p = tuple(prev[n] for n in ("qkv", "gate", "beta")) if isinstance(prev, dict) else tuple(prev)
        Tp = p[0].shape[1]
        for name, t, shp in zip(("qkv", "gate", "beta"), p, ((B, Tp, H, C), (B, Tp, H, dk), (B, Tp, H))):
            _check_dev("prev " + name, t, dev, qkv.dtype, shp)
        _check_dev("replay", replay, dev, torch.int32, (B,))
    y = _fusion_args((B, T, H, dv), qkv.dtype, dev, H, dv, gate_A_log, out_gate, norm_w, y, True)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _check_dev("o", o, dev, torch.float32, (B, T, H, dv))
    if form not in (None, 1, 2):
        raise ValueError("form must be None, 1 (token by token) or 2 (one chunk)")
    need = kda_decode_layer_window_workspace_bytes(B, T, Tp, H, dk, dv, qkv.dtype)
    if form == 2 and need == 0:
        raise ValueError("the one-chunk form serves bf16 with dk = dv = 128 and 6 <= T + Tp <= 16")
    ws, ws_bytes = None, 0
    if form != 1 and need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check_dev("workspace", workspace, dev)
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    _check(load_library().kda_decode_layer_window_replay(
        *(_ptr(t) for t in p), _ptr(replay if Tp > 0 else None), Tp, _ptr(qkv), _ptr(gate), _ptr(beta),
        _ptr(conv_w), _ptr(conv_cache), float(l2_eps), _ptr(gate_A_log), _ptr(state), _ptr(o), _ptr(out_gate),
        _ptr(norm_w), float(norm_eps), _ptr(y), B, T, H, dk, dv, _dtype_code(qkv.dtype), _ptr(ws), ws_bytes,
        _stream(stream)))
    return o, y


def kda_check_cu_seqlens(cu_seqlens, total_tokens: int, *, result=None, stream=None) -> torch.Tensor:
    """Check a device cu_seqlens (int32 [nseq + 1]) against the layout contract on the GPU.
    Returns the int32 device tensor [1] the kernel writes: -1 when valid, else the first index
    that breaks it (read it with .item(), which synchronises)."""
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.device.type != "cuda":
        raise ValueError("cu_seqlens must be a tensor on a GPU; the KDA library has no CPU path")
    _check_dev("cu_seqlens", cu_seqlens, cu_seqlens.device, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [nseq + 1] with nseq >= 1")
    if result is None:
        result = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device)
    _check_dev("result", result, cu_seqlens.device, torch.int32, (1,))
    _check(load_library().kda_check_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(total_tokens),
                                               _ptr(result), _stream(stream)))
    return result


def kda_prefill_backward(q, k, v, log_alpha, beta, d_o, cu_seqlens=None, init_state=None, d_final=None, *,
                         need_d_init: bool = True, workspace=None, stream=None):
    """Gradients of kda_prefill for a loss with dL/do = d_o (fp32 [N, H, dv]) and
    dL/d(final state) = d_final (fp32 [nseq, H, dk, dv] or None).  Returns a dict of fp32 tensors:
    dq, dk, dlog_alpha [N, H, dk], dv [N, H, dv], dbeta [N, H], dinit [nseq, H, dk, dv] (or None)."""
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    dev = q.device
    cu = _cu(cu_seqlens, N, dev)
    nseq = cu.numel() - 1
    _check_dev("d_o", d_o, dev, torch.float32, (N, H, dv))
    if d_final is not None:
        _check_dev("d_final", d_final, dev, torch.float32, (nseq, H, dk, dv))
    if init_state is not None:
        _check_dev("init_state", init_state, dev, torch.float32, (nseq, H, dk, dv))
    lib = load_library()
    nbytes = int(lib.kda_prefill_backward_workspace_bytes(N, nseq, H, dk, dv, _dtype_code(q.dtype)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=dev)
    _check_workspace(workspace, dev, nbytes)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((N, H, dk), **f32), "dk": torch.empty((N, H, dk), **f32),
           "dv": torch.empty((N, H, dv), **f32), "dlog_alpha": torch.empty((N, H, dk), **f32),
           "dbeta": torch.empty((N, H), **f32),
           "dinit": torch.empty((nseq, H, dk, dv), **f32) if need_d_init else None}
    _check(lib.kda_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), _ptr(cu), nseq, N, H, dk, dv,
        _dtype_code(q.dtype), _ptr(d_o), _ptr(d_final), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dinit"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kda_prefill_backward_slabbed_workspace_bytes(total_tokens: int, H: int, dk: int, dv: int, slab_tokens: int,
                                                 dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of kda_prefill_backward_slabbed (0: invalid arguments)."""
    return int(load_library().kda_prefill_backward_slabbed_workspace_bytes(total_tokens, H, dk, dv,
                                                                          _dtype_code(dtype), slab_tokens))


def kda_prefill_backward_slabbed(q, k, v, log_alpha, beta, d_o, init_state=None, d_final=None, *,
                                 slab_tokens: int = 16384, need_d_init: bool = True, workspace=None, stream=None):
    """kda_prefill_backward for one long sequence (q ... [N, H, .]) with the memory of one slab of
    ``slab_tokens`` tokens (a multiple of 16).  Returns the same dict as kda_prefill_backward."""
    N, H, dk, dv = _check_inputs(q, k, v, log_alpha, beta)
    dev = q.device
    _check_dev("d_o", d_o, dev, torch.float32, (N, H, dv))
    if d_final is not None:
        _check_dev("d_final", d_final, dev, torch.float32, (1, H, dk, dv))
    if init_state is not None:
        _check_dev("init_state", init_state, dev, torch.float32, (1, H, dk, dv))
    lib = load_library()
    nbytes = kda_prefill_backward_slabbed_workspace_bytes(N, H, dk, dv, slab_tokens, q.dtype)
    if nbytes == 0:
        raise KDAError(3, "kda_prefill_backward_slabbed: invalid shape or slab_tokens")
    if workspace is None:
        workspace = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=dev)
    _check_workspace(workspace, dev, nbytes)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((N, H, dk), **f32), "dk": torch.empty((N, H, dk), **f32),
           "dv": torch.empty((N, H, dv), **f32), "dlog_alpha": torch.empty((N, H, dk), **f32),
           "dbeta": torch.empty((N, H), **f32),
           "dinit": torch.empty((1, H, dk, dv), **f32) if need_d_init else None}
    _check(lib.kda_prefill_backward_slabbed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state), N, H, dk, dv,
        _dtype_code(q.dtype), _ptr(d_o), _ptr(d_final), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dinit"]), int(slab_tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out

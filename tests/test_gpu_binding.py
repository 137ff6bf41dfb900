"""The Python binding rejects wrong buffers before any launch: host tensors, wrong dtypes,
shapes or sizes of the outputs, the initial state and the workspace raise in Python, so no
kernel is handed a host pointer or an undersized buffer."""
import pytest
import torch

import gated_delta_rule_51_amd as kda
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    kda.load_library()
    dev = torch.device("cuda:0")
    w = workloads.custom([40, 24], 2, 32, 32, torch.bfloat16)
    x = workloads.prefill_inputs(w, device=dev, seed=0)
    return dev, w, x


def _args(x):
    return x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["cu_seqlens"]


@pytest.mark.parametrize("fn", [kda.kda_prefill, lambda *a, **kw: kda.kda_prefill_cp(*a, segments=2, **kw)])
def test_prefill_rejects_bad_buffers(case, fn):
    dev, w, x = case
    N, H, nseq = w.total_tokens, w.H, w.nseq
    f32 = dict(dtype=torch.float32, device=dev)
    bad = [
        dict(init_state=torch.zeros((nseq, H, 32, 32), dtype=torch.float32)),          # host init_state
        dict(init_state=torch.zeros((nseq, H, 32, 16), **f32)),                        # wrong shape
        dict(o=torch.zeros((N, H, 32), dtype=torch.float32)),                          # host o
        dict(o=torch.zeros((N, H, 32), dtype=torch.bfloat16, device=dev)),             # bf16 o
        dict(o=torch.zeros((N - 1, H, 32), **f32)),                                    # undersized o
        dict(o=torch.zeros((N, H, 64), **f32)[..., :32]),                              # not contiguous
        dict(final_state=torch.zeros((nseq, H, 32, 32), dtype=torch.float32)),         # host final_state
        dict(final_state=torch.zeros((nseq - 1, H, 32, 32), **f32)),                   # wrong shape
        dict(workspace=torch.zeros(16, **f32)),                                        # too small
        dict(workspace=torch.zeros(1 << 20, dtype=torch.float32)),                     # host workspace
    ]
    for kw in bad:
        o_guard = torch.full((N, H, 32), 7.0, **f32)
        with pytest.raises((ValueError, TypeError)):
            if "o" in kw:
                fn(*_args(x), **kw)
            else:
                fn(*_args(x), o=o_guard, **kw)
        torch.cuda.synchronize()
        assert torch.all(o_guard == 7.0), f"a launch happened for {list(kw)}"


def test_phase_entry_points_reject_bad_buffers(case):
    dev, w, x = case
    N, H, nseq = w.total_tokens, w.H, w.nseq
    ws = kda.alloc_workspace(N, nseq, H, 32, 32, torch.bfloat16, dev)
    with pytest.raises(ValueError):
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"].cpu(), x["cu_seqlens"], ws)
    with pytest.raises(ValueError):
        kda.kda_chunk_local(x["q"], x["k"], x["log_alpha"], x["beta"], x["cu_seqlens"], ws[:16])
    with pytest.raises(TypeError):
        kda.kda_chunk_local(x["q"], x["k"].float(), x["log_alpha"], x["beta"], x["cu_seqlens"], ws)
    with pytest.raises(ValueError):
        kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"], ws,
                            o=torch.zeros((N, H, 16), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        kda.kda_inter_chunk(x["q"], x["k"], x["v"], x["log_alpha"], x["cu_seqlens"].cpu(), ws)


def test_decode_rejects_bad_output(case):
    dev, _, _ = case
    w = workloads.custom([1] * 3, 2, 32, 32)
    d = workloads.decode_step_inputs(w, 0, device=dev)
    state = torch.zeros((3, 2, 32, 32), dtype=torch.float32, device=dev)
    with pytest.raises((ValueError, TypeError)):
        kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state,
                            o=torch.zeros((3, 2, 16), dtype=torch.float32, device=dev))
    with pytest.raises((ValueError, TypeError)):
        kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state,
                            o=torch.zeros((3, 2, 32), dtype=torch.float32))

"""Helpers for the GPU tests: numpy (synth/oracle layout) -> device tensors."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev(a: np.ndarray) -> torch.Tensor:
    """uint16 arrays are bf16 bits; float32 stays float32; int32 stays int32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def banner(msg: str):
    print(f"[gpu-test] {msg}", flush=True)

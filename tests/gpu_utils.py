"""Helpers shared by the GPU parity tests (test code only)."""
import numpy as np
import pytest


def torch_mod():
    return pytest.importorskip("torch")


def require_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_sign_amd import ckda
    ckda.lib()            # raises if the HIP library is missing: no silent fallback
    return torch


def dev_tensor(arr: np.ndarray):
    """numpy storage array -> torch tensor on cuda:0 (uint16 bit arrays are bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if arr.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to("cuda:0")


def tok_to_dev(tok):
    return dict(q=dev_tensor(tok.q), k=dev_tensor(tok.k), v=dev_tensor(tok.v), g=dev_tensor(tok.g),
                s=dev_tensor(tok.s), beta=dev_tensor(tok.beta))


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / RMS(ref) over all elements."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(gpu - ref))) / max(rms, 1e-30)


def banner(msg: str) -> None:
    print(f"[case] {msg}", flush=True)

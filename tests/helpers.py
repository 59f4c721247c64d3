"""Shared helpers for the GPU parity tests (host <-> device marshalling and
comparison metrics).  No method arithmetic lives here."""
import numpy as np
import torch

import video_diffusion_transformer_block_amd as V
from oracle import formats as F


def need_gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    V.lib()  # raises if the library is missing: no fallback path exists


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_fro(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return F.bf16_to_f32(bits).astype(np.float64)


def log(msg: str):
    print(msg, flush=True)

"""Helpers shared by the GPU parity tests: host <-> device copies of the
generator's bytes and the error measures the tolerances are stated in."""
import sys

import numpy as np

from attention_shards_amd import synthetic as syn

# Tolerances (max-abs error over the compared elements / RMS of the oracle
# over the same elements): fp32 inputs 1e-4, bf16 inputs with fp32
# accumulation 2e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == syn.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def from_dev(t) -> np.ndarray:
    """Exact float64 value of a device tensor (bf16 or fp32)."""
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return syn.to_f64(bits, syn.BF16)
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / rms


def bf16_floor(ref: np.ndarray) -> float:
    """Error a perfect kernel would show after rounding its output to bf16."""
    r = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    return rel_err(r, ref)


def empty(shape, dtype: str):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == syn.BF16 else torch.float32,
                       device="cuda")

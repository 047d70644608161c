"""Shared helpers of the test-suite: moving bit patterns between numpy and
torch, and loading the HIP binding (GPU tests only)."""
import numpy as np
import pytest
import torch


def gpu_available() -> bool:
    return torch.cuda.is_available() and torch.cuda.device_count() > 0


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    """numpy uint16 bf16 bits -> torch.bfloat16 on cuda:0 (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def u8_to_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to("cuda:0")


def f32_to_dev(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to("cuda:0")


def to_u8(t: torch.Tensor) -> np.ndarray:
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    return t.cpu().numpy()


def to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().astype(np.float32)


def binding():
    """The HIP binding; GPU tests fail (not skip) if the library is missing."""
    import fp8_block_scaled_act_amd as fb
    fb.lib()
    return fb


def say(*args):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *args, flush=True)


def report(label, res):
    """Print a GEMM comparison: normwise error, worst elementwise ratio and
    the share of outputs within plain 4 bf16 ulp + the fp32 floor first
    proposed for the comparison (oracle.gemm.s13_tau)."""
    print(f"[gemm] {label}: normwise {res['normwise']:.3e}, elementwise ratio {res['elem_ratio']:.3f}, "
          f"within 4 ulp + fp32 floor {res['frac_plain']:.6f} ({res['n'] - res['n_plain']} of {res['n']} outside)",
          flush=True)

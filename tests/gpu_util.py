"""Helpers for the GPU parity tests: move synth's bf16 bit patterns to the
device, run the HIP path through the binding, bring results back as numpy."""
import numpy as np
import torch

import fp8_scaled_matmul_amd as fm


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_quantize(x: torch.Tensor, fmt, gran=fm.TENSOR, mode=fm.FROM_AMAX, scale=None, want_t=False):
    ctr = fm.Counters()
    s_dev = dev_f32(scale) if scale is not None else None
    q, qt, s = fm.quantize(x, fmt, gran, mode, scale=s_dev, want_t=want_t, counters=ctr)
    torch.cuda.synchronize()
    c = ctr.read()
    return host(q), (host(qt) if qt is not None else None), host(s), c


def same_counters(gpu: dict, orc: dict, fields=("saturated", "underflow", "nan")) -> bool:
    return all(gpu[f] == orc[f] for f in fields)


def assert_gemm_close(y_bits: np.ndarray, y_ref: np.ndarray, what: str = ""):
    """The GEMM tolerance: max|y - y_ref| <= 1e-2 max|y_ref| and relative
    Frobenius error <= 5e-3, against the fp64 oracle before output rounding."""
    y = bf16_to_f64(y_bits)
    err = np.abs(y - y_ref)
    ref_max = np.abs(y_ref).max()
    fro = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert err.max() <= 1e-2 * ref_max, f"{what}: max err {err.max():.4g} vs {1e-2 * ref_max:.4g}"
    assert fro <= 5e-3, f"{what}: rel Frobenius {fro:.4g}"
    return float(err.max() / max(ref_max, 1e-300)), float(fro)

"""Helpers shared by the GPU tests: moving workload arrays to the device and
the parity gates."""
import numpy as np
import torch

# |gpu - ref| <= RTOL * |ref| + ATOL for bf16 / fp16 outputs
RTOL, ATOL = 1.6e-2, 1e-2
# fp32 dequantised values before the output cast
DEQUANT_RTOL = 1e-5

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "i8": torch.int8, "f32": torch.float32,
          "i32": torch.int32}


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype == "bf16" or a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def torch_dtype(name):
    return _TORCH[name]


def to_f64(t):
    if t.dtype in (torch.int32, torch.int8):
        return t.cpu().numpy().astype(np.int64)
    return t.float().cpu().numpy().astype(np.float64)


def assert_tol(gpu, ref, what="", rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = rtol * np.abs(ref) + atol
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside |d| <= {rtol}|ref| + {atol}; "
            f"worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}")
    # a systematic slip hidden under the absolute term still shows in the RMS
    rms_ref = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rms_err = float(np.sqrt(np.mean(err ** 2))) if ref.size else 0.0
    assert rms_err <= 0.02 * rms_ref + 1e-6, f"{what}: rms err {rms_err} vs rms ref {rms_ref}"
    return rms_err / (rms_ref or 1.0)


def assert_rel(gpu, ref, rtol, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.abs(gpu - ref) / np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
    assert rel.max() <= rtol, f"{what}: max relative error {rel.max()} > {rtol}"

"""Helpers shared by the GPU parity tests: host<->device moves and the tolerance gate."""
import numpy as np
import torch

# bf16 inputs with fp32 accumulation, compared with the fp64 oracle
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
# fp32 inputs and arithmetic
F32_TOL = 1e-5


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    """Host buffer (float32, or uint16 bf16 bit patterns) -> device tensor of that dtype."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    raise TypeError(x.dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, want: np.ndarray):
    err = np.abs(got - want)
    return float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, fp32=False, what=""):
    """O and LSE each within the gate: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 both <= 1e-5."""
    o = to_f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    l = to_f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert o.shape == o_ref.shape and l.shape == lse_ref.shape, (o.shape, o_ref.shape, l.shape, lse_ref.shape)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what + ": non-finite output"
    mx_o, mn_o = errors(o, o_ref)
    mx_l, mn_l = errors(l, lse_ref)
    if fp32:
        ok = mx_o <= F32_TOL and mn_o <= F32_TOL and mx_l <= F32_TOL and mn_l <= F32_TOL
    else:
        ok = mx_o <= BF16_MAX_ABS and mn_o <= BF16_MEAN_ABS and mx_l <= BF16_MAX_ABS and mn_l <= BF16_MEAN_ABS
    msg = "%s: O max/mean %.3g/%.3g, LSE max/mean %.3g/%.3g" % (what, mx_o, mn_o, mx_l, mn_l)
    print(msg, flush=True)
    assert ok, msg
    return mx_o, mn_o, mx_l, mn_l

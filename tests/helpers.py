"""Shared test helpers: tolerance check and host<->device bf16 transfers."""
import numpy as np

from workloads import bf16_bits_to_f64

ATOL, RTOL = 2e-3, 1e-2   # |err| <= 2e-3 + 1e-2 |ref| on bf16-input, fp32-accumulate outputs


def assert_close(got, ref, what="", atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    ratio = float((err / bound)[worst])
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    print(f"[parity] {what}: max err/bound {ratio:.3f} at {worst}, max|err| {err.max():.3e}, "
          f"||err||/||ref|| {rel:.3e}", flush=True)
    assert ratio <= 1.0, f"{what}: err {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"
    return ratio


def to_dev(bits, device="cuda"):
    """uint16 bf16 bit pattern array -> torch.bfloat16 device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def from_dev(t):
    """bf16 device tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f64(bits)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False

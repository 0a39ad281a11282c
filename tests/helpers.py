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


def pow2_bf16(bits, k):
    """bf16 bit patterns times 2^k, exactly (the exponent field is raised by k;
    zeros stay zero).  Used to sharpen the softmax: q times 4 or 8 spreads the
    scores over many units, so a few rows dominate every head."""
    b = np.asarray(bits, dtype=np.uint16)
    nz = (b & 0x7FFF) != 0
    exp = (b >> 7) & 0xFF
    if np.any(nz & (exp + k >= 255)) or np.any(nz & (exp == 0)):
        raise ValueError("pow2_bf16: exponent out of range")
    return np.where(nz, (b.astype(np.uint32) + (k << 7)).astype(np.uint16), b)


class Guarded:
    """A device tensor of `shape` placed between two canary bands of `band`
    bytes each (the band size keeps the view 256-byte aligned).  `view` is
    handed to an entry point as an output or workspace; check() asserts that
    no byte of either band changed."""

    def __init__(self, shape, dtype, band=4096, seed=0):
        import torch
        esize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        nbytes = n * esize
        self.band = band
        rng = np.random.default_rng(seed)
        total = band + ((nbytes + 255) // 256) * 256 + band
        self.raw = torch.from_numpy(rng.integers(0, 256, size=total, dtype=np.uint8)).cuda()
        self.expect = self.raw.clone()
        self.view = self.raw[band:band + nbytes].view(dtype).view(shape)
        self.nbytes = nbytes

    def check(self, what=""):
        import torch
        torch.cuda.synchronize()
        lo = self.band
        hi = self.band + self.nbytes
        assert torch.equal(self.raw[:lo], self.expect[:lo]), f"{what}: canary before the buffer changed"
        assert torch.equal(self.raw[hi:], self.expect[hi:]), f"{what}: canary after the buffer changed"


# The decode kernels' own precision: K and V are exact bf16 inputs, q and P
# enter the products as hi + lo bf16 (~2^-17), sums are fp32, so the error is
# the final bf16 rounding of the output (at most 2^-8 of it) plus fp32
# rounding well under 5e-5.  Checked beside the contract tolerance so that an
# error far below 2e-3 + 1e-2 |ref| (outputs of ~0.006 at 32K rows) still shows.
KERNEL_ATOL, KERNEL_RTOL = 5e-5, 2.0 ** -7


def check_every_head(got, q, k, v, lens, scale, rope, Hq, Hkv, what, qmul=1.0):
    """Every (b, h) output of a full-size decode against the oracle: per
    (batch, kv head) the group's g heads at once over that context's rows,
    to the contract tolerance and to the kernels' own precision bound."""
    g = Hq // Hkv
    from oracle import attention as oatt
    from workloads import bf16_tensor_to_f64
    qf = bf16_tensor_to_f64(q) * qmul
    worst = tight = 0.0
    for b in range(len(lens)):
        L = int(lens[b])
        for kv in range(Hkv):
            kb = bf16_tensor_to_f64(k[b, kv, :L])
            vb = bf16_tensor_to_f64(v[b, kv, :L])
            ref = oatt.decode_group(qf[b, kv * g:(kv + 1) * g], kb, vb, L, scale, rope)
            worst = max(worst, assert_close(got[b, kv * g:(kv + 1) * g], ref,
                                            f"{what} (b={b}, kv={kv}, L={L})"))
            tight = max(tight, assert_close(got[b, kv * g:(kv + 1) * g], ref,
                                            f"{what} (b={b}, kv={kv}, L={L}) kernel precision",
                                            atol=KERNEL_ATOL, rtol=KERNEL_RTOL))
    print(f"[parity] {what}: every head, worst err/bound {worst:.3f} (kernel precision bound "
          f"{tight:.3f})", flush=True)

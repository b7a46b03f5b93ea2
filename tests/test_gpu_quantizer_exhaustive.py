"""The GPU quantiser's FP8 encoding of every fp32 value in range: each block
of 32 holds the format's largest finite value (so the E8M0 exponent is 0,
scale byte 127) and 31 values of a chunk of consecutive fp32 bit patterns;
all of |v| <= 448 (E4M3) and |v| <= 57344 (E5M2), both signs.  The codes
are compared with torch's float8 casts, which the CPU tests pin to the
oracle's encoders over the same values."""
import numpy as np
import pytest

from gpu_common import say, torch_cuda

pytestmark = pytest.mark.gpu

CHUNK = 31 * (1 << 21)      # values per launch (a multiple of 31)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_gpu_quantizer_every_fp32_value(fmt):
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    top, limit, tdt, code = {"e4m3": (448.0, 0x43E00000, torch.float8_e4m3fn, pkg.FMT_E4M3),
                             "e5m2": (57344.0, 0x47600000, torch.float8_e5m2, pkg.FMT_E5M2)}[fmt]
    for sign in (0, 0x80000000):
        say(f"[quant-all] {fmt} sign {'-' if sign else '+'}: {limit + 1} values")
        for lo in range(0, limit + 1, CHUNK):
            hi = min(lo + CHUNK, limit + 1)
            vals = (np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign)).view(np.float32)
            nblk = -(-vals.size // 31)
            body = np.zeros(nblk * 31, dtype=np.float32)
            body[:vals.size] = vals
            x = np.empty((nblk, 32), dtype=np.float32)
            x[:, 0] = top
            x[:, 1:] = body.reshape(nblk, 31)
            q, s = pkg.quantize_mxfp8(torch.from_numpy(x).cuda(), fmt=code)
            torch.cuda.synchronize()
            assert bool((s == 127).all()), f"{fmt}: scale byte not 127 in [{lo:#x}, {hi:#x})"
            got = q[:, 1:].reshape(-1)[:vals.size].cpu().numpy()
            ref = torch.from_numpy(vals).to(tdt).view(torch.uint8).numpy()
            if not np.array_equal(got, ref):
                i = int(np.nonzero(got != ref)[0][0])
                raise AssertionError(f"{fmt}: {float(vals[i])!r}: gpu {int(got[i]):#04x}, torch {int(ref[i]):#04x}")

"""GPU parity of the decoded-frame compaction (h3_frames_to_uint8_bthwc):
every byte equal to the oracle's exact map, on the vector path and the
per-pixel path, including inputs next to every rounding midpoint and tiny
values of both signs (where a float32 evaluation would differ)."""
import numpy as np
import pytest

import oracle
from _gpu_helpers import announce, torch_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return torch_device()


@pytest.fixture(scope="module")
def ops():
    from audio_diffusion_transformer_packed_amd import ops as o
    return o


def _special_values() -> np.ndarray:
    """Exact ties (0 -> 127.5), the ends, NaN, infinities, the float32
    values next to each of the 255 midpoints (255 (1 + x) / 2 = k + 1/2) and
    tiny values of both signs down to the smallest subnormal."""
    vals = [0.0, -0.0, 1.0, -1.0, np.nan, np.inf, -np.inf, 2.0 / 255 - 1]
    for k in range(255):
        c = np.float32((2 * k + 1) / 255.0 - 1.0)
        vals += [np.nextafter(c, np.float32(-2)), c, np.nextafter(c, np.float32(2))]
    for n in list(range(17, 150, 3)) + [149]:
        vals += [2.0 ** -n, -(2.0 ** -n)]
    return np.array(vals, np.float32)


def _frames(shape, seed):
    """Values over [-1.5, 1.5] with the special values scattered in."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1.5, 1.5, size=shape).astype(np.float32)
    flat = x.reshape(-1)
    sp = _special_values()
    idx = rng.choice(flat.size, size=min(flat.size, sp.size), replace=False)
    flat[idx] = sp[:idx.size]
    return x


@pytest.mark.parametrize("shape", [(2, 3, 3, 16, 24), (1, 1, 2, 8, 8), (1, 4, 1, 4, 12),
                                   (1, 3, 1, 5, 7), (2, 5, 2, 3, 16)])
def test_frames_to_uint8_bit_exact(dev, ops, shape):
    import torch
    announce(f"frames to uint8 {shape}")
    x = _frames(shape, 500 + sum(shape))
    got = ops.frames_to_uint8_bthwc(torch.from_numpy(x).to(dev)).cpu().numpy()
    assert np.array_equal(got, oracle.frames_to_uint8_bthwc(x))


def test_frames_unaligned_output_takes_pixel_path(dev, ops):
    import torch
    announce("frames to uint8, output offset by one byte")
    shape = (1, 3, 2, 16, 16)
    x = _frames(shape, 510)
    n = int(np.prod(shape))
    buf = torch.zeros(n + 16, dtype=torch.uint8, device=dev)
    out = buf[1:1 + n].view(1, 2, 16, 16, 3)
    ops.frames_to_uint8_bthwc(torch.from_numpy(x).to(dev), out=out)
    assert np.array_equal(out.cpu().numpy(), oracle.frames_to_uint8_bthwc(x))
    assert int(buf[0]) == 0 and int(buf[1 + n:].sum()) == 0


def test_frames_full_resolution(dev, ops):
    """1344 x 768 frames (the 10 s clip's resolution) in the launch the
    bench times, 31 frames."""
    import torch
    announce("frames to uint8 1 x 3 x 31 x 768 x 1344")
    x = _frames((1, 3, 31, 768, 1344), 520)
    got = ops.frames_to_uint8_bthwc(torch.from_numpy(x).to(dev)).cpu().numpy()
    assert np.array_equal(got, oracle.frames_to_uint8_bthwc(x))

"""NVFP4 codec on the GPU: codes and scales bit-exact against the oracle, and
exact dequantisation [App. C.3 of the Polestar page]."""
import numpy as np
import pytest
import torch

from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests.harness import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,d", [(1, 16), (97, 256), (96, 4096), (3, 3584)])
def test_nvfp4_pack_unpack_bit_exact(rows, d):
    log(f"[nvfp4] rows={rows} d={d}")
    rng = np.random.default_rng(rows * 7 + d)
    x = (rng.normal(size=(rows, d)) * np.exp(rng.uniform(-14, 9, size=(rows, 1)))).astype(np.float32)
    x[0, :16] = np.float32([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, 0, -0.0, 4, 3, 2])
    if rows > 3:
        x[1, :16] = 0.0
        x[2, :16] = np.float32(1e6)
        x[3, :16] = np.float32(2.0 ** -14)
    xt = torch.tensor(x, device="cuda")
    codes = torch.zeros(rows, d // 2, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(rows, d // 16, dtype=torch.uint8, device="cuda")
    B.polestar_nvfp4_pack(xt, rows, d, codes, scales)
    back = torch.zeros(rows, d, dtype=torch.float32, device="cuda")
    B.polestar_nvfp4_unpack(codes, scales, rows, d, back)
    torch.cuda.synchronize()
    oc, osc = O.nvfp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), osc)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(back.cpu().numpy(), O.nvfp4_dequantize(oc, osc))

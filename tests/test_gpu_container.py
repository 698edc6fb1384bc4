"""The .wcpk container end to end on the GPU: save encodes with the GPU
codec, get_tensor decodes one tensor (checking every chunk's CRC-32 on the
GPU) and restores dtype and shape bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, container as C  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _tensors(dev):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(1000, 700, generator=g) * 0.02
    return {
        "w_bf16": x.to(torch.bfloat16).to(dev),
        "w_fp32": (torch.randn(300, 257, generator=g) * 0.05).to(dev),
        "w_fp16": x[:333].to(torch.float16).to(dev),
        "w_fp8": (x * (448.0 / float(x.abs().max()))).to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
                 .view(torch.float8_e4m3fn),
        "empty": torch.empty(0, 16, dtype=torch.bfloat16, device=dev),
    }


@pytest.mark.parametrize("opts", [dict(), dict(reorder=True, tensor_table=True, raw_fallback=True)])
def test_save_and_load(dev, tmp_path, opts):
    ts = _tensors(dev)
    path = str(tmp_path / "m.wcpk")
    C.save(path, ts, crc=True, **opts)
    idx = C.TensorIndex.open(path)
    assert set(idx.keys()) == set(ts)
    for name, t in ts.items():
        y = idx.get_tensor(name, dev)
        assert y.dtype == t.dtype and tuple(y.shape) == tuple(t.shape)
        assert torch.equal(y.view(torch.uint8).cpu(), t.view(torch.uint8).cpu()), name
    got = C.load(path, ["w_fp32"], dev)
    assert list(got) == ["w_fp32"] and torch.equal(got["w_fp32"], ts["w_fp32"])


def test_damaged_payload_is_caught_on_the_gpu(dev, tmp_path):
    ts = {"w": (torch.randn(2000, 300) * 0.02).to(torch.bfloat16).to(dev)}
    path = str(tmp_path / "d.wcpk")
    C.save(path, ts, crc=True)
    idx = C.TensorIndex.open(path)
    off, length = idx.meta("w")["sections"]["payload"]
    with open(path, "r+b") as f:
        f.seek(off + length - 9)
        b = f.read(1)
        f.seek(off + length - 9)
        f.write(bytes([b[0] ^ 0x01]))
    with pytest.raises(C.ContainerError):
        idx.get_tensor("w", dev)
    with pytest.raises(B.WcError, match="CRC"):
        idx.get_tensor("w", dev, verify=False)

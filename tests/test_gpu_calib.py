"""The measurement utilities on the GPU: they run, read every byte of a buffer with a
ragged tail, leave the sink alone, and refuse bad arguments."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_verify_amd import api
    return api


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 37, 64 << 20])
def test_calib_read(nbytes):
    api = _api()
    print(f"[gpu-case] calib read {nbytes} bytes", flush=True)
    buf = torch.arange(nbytes, dtype=torch.int32, device="cuda").to(torch.uint8)
    sink = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    api.spec_calib_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7.0


def test_calib_read_rejects_misaligned():
    api = _api()
    from lossless_rejection_sampling_verify_amd import _lib as L
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(L.SpecVerifyError):
        api.spec_calib_read(buf[4:4 + 1024], sink)
    with pytest.raises(L.SpecVerifyError):
        api.spec_calib_read(buf[:1000], sink)


def test_calib_exp():
    api = _api()
    print("[gpu-case] calib exp", flush=True)
    sink = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    api.spec_calib_exp(64, 16, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7.0

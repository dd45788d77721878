"""Helpers for the GPU parity tests: host bit arrays <-> device tensors."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_precision_quantization_amd as mx
    mx.lib()  # a missing library is an error, not a skip
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_dev_u8(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype not in (torch.uint8, torch.int64, torch.int32):
        t = t.view(torch.uint8)
    return t.cpu().numpy()


def sentinel(shape, dev, value=0xCD):
    return torch.full(shape, value, dtype=torch.uint8, device=dev)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, "%s: shape %s != %s" % (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        idx = np.argwhere(got != want)
        n = idx.shape[0]
        first = [tuple(int(v) for v in i) for i in idx[:5]]
        vals = [(int(got[tuple(i)]), int(want[tuple(i)])) for i in idx[:5]]
        raise AssertionError("%s: %d bytes differ; first at %s (got, want) = %s" % (what, n, first, vals))

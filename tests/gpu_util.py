"""Helpers shared by the GPU parity tests: host <-> device copies of the seeded inputs."""

import numpy as np
import torch

DEV = torch.device("cuda", 0)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def poison(shape, dtype) -> torch.Tensor:
    """An output buffer filled with 0xA5 bytes, so unwritten elements show up."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    return buf.view(dtype).view(*shape) if len(shape) else buf.view(dtype)


def assert_same(name, got, want):
    """Bit-exact comparison with a readable report of where the arrays differ."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if got.dtype.kind == "f":
        gb, wb = got.view(np.uint32 if got.itemsize == 4 else np.uint16), want.view(np.uint32 if want.itemsize == 4 else np.uint16)
    else:
        gb, wb = got, want
    bad = np.argwhere(gb != wb)
    if bad.size:
        first = [tuple(int(v) for v in b) for b in bad[:6]]
        vals = [(got[tuple(b)], want[tuple(b)]) for b in bad[:6]]
        rows = np.unique(bad[:, 0])
        raise AssertionError(f"{name}: {len(bad)} of {gb.size} differ; rows {rows[:12].tolist()} "
                             f"({rows.size} rows); first {first}; got/want {vals}")

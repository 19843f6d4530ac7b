"""Helpers for the GPU tests: byte-level uploads and downloads of numpy
arrays through torch CUDA tensors, and a progress print that names the case
before each GPU step."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*args) -> None:
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray) -> torch.Tensor:
    """Upload the bytes of a numpy array; returns a uint8 CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(DEV)


def down(t: torch.Tensor, dtype=np.uint8) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(dtype)


def filled(nbytes: int, value: int) -> torch.Tensor:
    return torch.full((nbytes,), value, dtype=torch.uint8, device=DEV)


def zeros(nbytes: int) -> torch.Tensor:
    return torch.zeros(nbytes, dtype=torch.uint8, device=DEV)


def random_bf16(n: int, seed: int, allow_nan: bool = True) -> np.ndarray:
    import datagen as dg
    w = dg.random_u64((n + 3) // 4, seed).view(np.uint16)[:n].copy()
    if not allow_nan:
        nan = (w & 0x7FFF) > 0x7F80
        w[nan] &= 0xBF7F  # clear an exponent bit: a finite value
    return w


def random_f32_bits(n: int, seed: int) -> np.ndarray:
    import datagen as dg
    return dg.random_u64((n + 1) // 2, seed).view(np.uint32)[:n].copy()

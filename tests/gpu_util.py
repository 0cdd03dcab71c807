"""Helpers shared by the GPU tests: moving seeded numpy inputs onto the GPU
and bringing results back as numpy bit patterns."""
from __future__ import annotations

import numpy as np


def torch():
    import torch as _t
    return _t


def bf16_gpu(u16: np.ndarray):
    """uint16 bf16 bit patterns -> torch.bfloat16 on cuda:0."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(t.bfloat16).to("cuda")


def f32_gpu(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def weights_gpu(w: np.ndarray):
    return bf16_gpu(w) if w.dtype == np.uint16 else f32_gpu(w)


def u32(t) -> np.ndarray:
    """int32 tensor holding uint32 words -> numpy uint32."""
    return t.cpu().numpy().view(np.uint32)


def f32_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def report(tag: str):
    """Print (and flush) what the next GPU step is, so a failing run names its case."""
    print("[gpu] " + tag, flush=True)

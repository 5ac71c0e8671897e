"""Device buffers fenced by sentinel bytes (guard canaries), for GPU tests.

A ``Guarded`` buffer is one allocation laid out as [head pad | tensor | tail
pad]; both pads hold the byte SENTINEL.  The tensor part starts on a 256-byte
boundary (the allocator's base is 256-aligned and the pad is a multiple of
256), so the library's 16-byte alignment rule holds.  After a call,
``assert_intact`` checks that no byte before or after the tensor changed:
a write past either end of an output or workspace fails the test even where
poisoning the tensor itself (NaN) cannot see it.
"""
from __future__ import annotations

import math

import torch

SENTINEL = 0xA5
PAD = 4096


class Guarded:
    def __init__(self, shape, dtype, device, fill=None, pad: int = PAD):
        shape = tuple(int(s) for s in shape)
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = math.prod(shape) * itemsize
        self.pad = pad
        self.buf = torch.full((2 * pad + self.nbytes,), SENTINEL, dtype=torch.uint8, device=device)
        self.t = self.buf[pad:pad + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    @property
    def ptr(self) -> int:
        return self.t.data_ptr()

    def assert_intact(self, what: str) -> None:
        head = self.buf[:self.pad]
        tail = self.buf[self.pad + self.nbytes:]
        assert bool((head == SENTINEL).all()), f"{what}: bytes before the buffer were written"
        assert bool((tail == SENTINEL).all()), f"{what}: bytes after the buffer were written"

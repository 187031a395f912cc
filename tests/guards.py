"""Guard bands around device buffers (test helper).

A guarded tensor sits in the middle of a larger allocation whose margins hold a
sentinel byte; check() fails if any byte of a margin changed, i.e. if a kernel
wrote before or past the tensor. Outputs start filled with NaN (or a given
value), so an element a kernel should write and does not also shows up.
"""
import torch

GUARD = 4096      # bytes on each side; a multiple of 256, so the tensor keeps the allocation's alignment
SENTINEL = 0xA5


class Guarded:
    def __init__(self, shape, dtype, device="cuda", fill=float("nan")):
        self.shape = tuple(shape)
        n = 1
        for s in self.shape:
            n *= s
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=device)
        self.t = self.buf[GUARD:GUARD + self.nbytes].view(dtype).view(self.shape)
        if fill is not None:
            self.t.fill_(fill)

    @classmethod
    def like(cls, src, device="cuda"):
        """A guarded device copy of src."""
        g = cls(src.shape, src.dtype, device, fill=None)
        g.t.copy_(src)
        return g

    def check(self, name="buffer"):
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        assert bool((head == SENTINEL).all()), f"{name}: bytes before the tensor were written"
        assert bool((tail == SENTINEL).all()), f"{name}: bytes past the tensor were written"


def check_all(**guards):
    torch.cuda.synchronize()
    for name, g in guards.items():
        g.check(name)

"""The guard bands of the GPU forward tests (tests/gpu_helpers.py), checked
on CPU tensors: a write one byte past either end of a buffer, or anywhere in
the bands, must be reported; writes inside the buffer must not."""
from __future__ import annotations

import pytest
import torch

from gpu_helpers import GUARD, add_guards, check_guards


class _Bufs:
    def __init__(self):
        self.o = torch.zeros(3, 5, 7, dtype=torch.float32)
        self.lifted = torch.zeros(1000, dtype=torch.uint8)


def test_inside_writes_pass():
    f = add_guards(_Bufs(), ("o", "lifted"))
    assert f.o.shape == (3, 5, 7) and f.o.dtype == torch.float32
    f.o.fill_(float("nan"))
    f.lifted.fill_(255)
    check_guards(f)


@pytest.mark.parametrize("name,offset", [("o", -1), ("o", 0), ("lifted", -GUARD), ("lifted", GUARD - 1)])
def test_writes_past_an_end_fail(name, offset):
    """offset < 0: that many bytes before the buffer; offset >= 0: that many
    bytes after its last byte."""
    f = add_guards(_Bufs(), ("o", "lifted"))
    _, raw, nb = next(g for g in f._guards if g[0] == name)
    pos = GUARD + offset if offset < 0 else GUARD + nb + offset
    raw[pos] = 0
    with pytest.raises(AssertionError, match=name):
        check_guards(f)

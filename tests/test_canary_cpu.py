"""The guard-band checker of the canary GPU tests (tests/gpu_util.Arena),
exercised on CPU tensors: an untouched arena passes, and a single changed byte
just before or just after a view is reported."""

import pytest
import torch

from gpu_util import GUARD, Arena


@pytest.mark.parametrize("where", [None, "before", "after"])
def test_arena_detects_writes_outside_a_view(where):
    a = Arena("cpu")
    v = a.alloc((3, 5), torch.float32)
    w = a.alloc((7,), torch.int32)
    v.fill_(1.0)
    w.fill_(2)
    raw, off, n = a.bufs[0]
    if where == "before":
        raw[off - 1] = 0
    elif where == "after":
        raw[off + n] = 0
    if where is None:
        a.check("clean")
    else:
        with pytest.raises(AssertionError, match="guard bytes changed"):
            a.check(where)
    assert off >= GUARD and (raw.data_ptr() + off) % 256 == 0

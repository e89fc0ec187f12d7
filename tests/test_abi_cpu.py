"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe.h declares, and its host-side checks (capacity, row bound,
workspace sizes, argument validation) behave as documented. No kernel runs:
every call here returns before anything is enqueued."""

import ctypes
import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_steps():
    names = _declared()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(moelib):
    lib = ctypes.CDLL(moelib.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(moelib.EXPORTED)


def _p(moelib, **kw):
    base = dict(T=1000, d_model=64, d_ff=128, E=8, k=2, dtype="bf16", act="gelu", renormalize=True)
    base.update(kw)
    return moelib.make_params(**base)


def test_capacity_and_row_bound(moelib):
    assert moelib.moe_capacity(_p(moelib, T=16384, E=128, k=1, capacity_factor=1.25)) == 160
    assert moelib.moe_capacity(_p(moelib, T=32768, E=64, k=2, capacity_factor=2.0)) == 2048
    assert moelib.moe_capacity(_p(moelib)) == -1
    assert moelib.moe_capacity(_p(moelib, capacity=5, capacity_factor=3.0)) == 5
    assert moelib.moe_max_rows(_p(moelib)) == 2000
    assert moelib.moe_max_rows(_p(moelib, capacity=5)) == 40
    assert moelib.moe_max_rows(_p(moelib, capacity=0)) == 0
    assert moelib.moe_capacity(_p(moelib, E=0)) == -2


def test_workspace_sizes(moelib):
    for op in range(5):
        small = moelib.moe_workspace_size(_p(moelib, T=100), op)
        big = moelib.moe_workspace_size(_p(moelib, T=10000), op)
        assert 0 < small <= big and small % 256 == 0
    fwd = moelib.moe_workspace_size(_p(moelib), moelib.MOE_OP_FORWARD)
    assert fwd >= sum(moelib.moe_workspace_size(_p(moelib), op) for op in range(3))
    # the expert FFN workspace holds the bf16 hidden activations of every row
    assert moelib.moe_workspace_size(_p(moelib), moelib.MOE_OP_EXPERT_FFN) >= 2000 * 128 * 2
    # the backward keeps the permuted rows, both hidden tensors, outputs and upstream rows
    assert moelib.moe_workspace_size(_p(moelib), moelib.MOE_OP_BACKWARD) >= 2000 * (2 * 64 + 2 * 128 + 64) * 2


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), "MOE_ERR_INVALID_ARG"),
    (dict(E=2000, k=2), "MOE_ERR_UNSUPPORTED"),
    (dict(k=0), "MOE_ERR_INVALID_ARG"),
    (dict(k=9, E=16), "MOE_ERR_UNSUPPORTED"),
    (dict(k=9, E=8), "MOE_ERR_INVALID_ARG"),
    (dict(d_model=60), "MOE_ERR_UNSUPPORTED"),
    (dict(d_ff=0), "MOE_ERR_INVALID_ARG"),
    (dict(T=-1), "MOE_ERR_INVALID_ARG"),
    (dict(T=2**30, k=2), "MOE_ERR_UNSUPPORTED"),
    (dict(gate_mode=4), "MOE_ERR_INVALID_ARG"),
    (dict(gate_mode=-1), "MOE_ERR_INVALID_ARG"),
    (dict(drop_order=2), "MOE_ERR_INVALID_ARG"),
    (dict(drop_order=-1), "MOE_ERR_INVALID_ARG"),
])
def test_invalid_params_rejected(moelib, kw, status):
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_workspace_size(_p(moelib, **kw), 0)
    assert moelib.status_string(ei.value.status) == status


def test_entry_points_validate_before_launch(moelib):
    p = _p(moelib)
    fake = 1 << 20  # aligned non-null addresses; never dereferenced because validation fails first
    with pytest.raises(moelib.MoEError) as ei:  # x NULL
        moelib.moe_route(p, None, fake, None, None, None, fake, fake, fake, None, None, None, stream=0)
    assert ei.value.status == moelib.MOE_ERR_INVALID_ARG and "x is NULL" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:  # w_noise without noise
        moelib.moe_route(p, fake, fake, None, fake, None, fake, fake, fake, None, None, None, stream=0)
    assert ei.value.status == moelib.MOE_ERR_INVALID_ARG
    with pytest.raises(moelib.MoEError) as ei:  # misaligned
        moelib.moe_route(p, fake + 2, fake, None, None, None, fake, fake, fake, None, None, None, stream=0)
    assert "aligned" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:  # no workspace
        moelib.moe_route(p, fake, fake, None, None, None, fake, fake, fake, None, None, None, stream=0)
    assert ei.value.status == moelib.MOE_ERR_WORKSPACE
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_dispatch(p, fake, fake, fake, None, fake, fake, fake, stream=0)
    assert "offsets" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_expert_ffn(p, fake, fake, None, fake, fake, stream=0)
    assert "w1" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_combine(p, fake, fake, None, fake, stream=0)
    assert "topk_gate" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_forward(p, fake, fake, None, None, None, fake, fake, None, stream=0)
    assert "y is NULL" in str(ei.value)


def test_backward_validates_before_launch(moelib):
    p = _p(moelib)
    fake = 1 << 20
    args = dict(x=fake, w_gate=fake, gate_bias=None, w_noise=None, noise=None, w1=fake, w2=fake, dy=fake,
                loss_weights=(0.0, 0.0, 0.0), dx=fake, dw_gate=fake, dgate_bias=None, dw_noise=None, dw1=fake,
                dw2=fake, dlogits=None, ws=None, stream=0)
    with pytest.raises(moelib.MoEError) as ei:  # no workspace
        moelib.moe_backward(p, **args)
    assert ei.value.status == moelib.MOE_ERR_WORKSPACE
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_backward(p, **{**args, "dw1": None})
    assert "dw1 is NULL" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:  # noisy gate without dw_noise
        moelib.moe_backward(p, **{**args, "w_noise": fake, "noise": fake})
    assert "dw_noise" in str(ei.value)
    with pytest.raises(moelib.MoEError) as ei:
        moelib.moe_backward(p, **{**args, "loss_weights": (float("nan"), 0.0, 0.0)})
    assert "finite" in str(ei.value)

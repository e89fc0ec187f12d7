"""GPU parity of the hierarchical MoE entry points (moe_route_hier,
moe_forward_hier) against the oracle's route_hier / forward_hier.

Routing (expert ids, counts, dispatch slots) bit-exact; gates within 1e-5
(fp32 logits on both sides); losses within 1e-4 relative; y within the bf16 /
fp32 tolerance on every token (sampled on the full-size workload).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import GATE_ATOL, TOL, aux_ok, as_f64, rel_rows_ok, say
from synthetic import HIER_CONFIGS, hier_scaled, make_hier_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev(moelib):
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def _params(moelib, cfg, cap=-1):
    return moelib.make_params(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.slots, cfg.dtype, cfg.act, True,
                              cfg.capacity_factor, cap, 0, 0, cfg.groups, cfg.k_group)


def _forward(moelib, dev, cfg, inp, cap=-1):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import to_device, to_numpy, workspace

    p = _params(moelib, cfg, cap)
    d = {k_: to_device(v, dev) for k_, v in inp.items()}
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    K = cfg.slots
    y = torch.full((cfg.T, cfg.d_model), float("nan"), dtype=dt, device=dev)
    aux = torch.full((4,), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, K), dtype=torch.float32, device=dev)
    cr = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    ck = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    sd = torch.empty((cfg.T, K), dtype=torch.int32, device=dev)
    ws = workspace(p, moelib.MOE_OP_FORWARD_HIER, dev)
    moelib.moe_forward_hier(p, d["x"], d["w_gate_p"], None, d["w_noise_p"], d["noise_p"], d["w_gate_s"], None,
                            d["w_noise_s"], d["noise_s"], d["w1"], d["w2"], y, aux, idx, gate, cr, ck, sd, ws)
    torch.cuda.synchronize()
    return {k_: to_numpy(v) for k_, v in dict(y=y, aux=aux, idx=idx, gate=gate, cr=cr, ck=ck, sd=sd).items()}


def _check(cfg, got, ref, tokens):
    assert np.array_equal(got["idx"], ref["topk_idx"])
    assert np.array_equal(got["cr"], ref["counts_routed"])
    assert np.array_equal(got["ck"], ref["counts_kept"])
    assert np.array_equal(got["sd"], ref["slot_dest"])
    assert np.abs(got["gate"] - ref["topk_gate"]).max(initial=0.0) <= GATE_ATOL["f32"]
    aux_ok(got["aux"], ref["aux"], 1e-4)
    rel_rows_ok(as_f64(got["y"][tokens], cfg.dtype), ref["y"], TOL[cfg.dtype], f"y {cfg.name}")


SMALL = [
    ("hier_tiny", {}, -1),
    ("hier_tiny", dict(T=300), 20),  # binding capacity
    ("hier_tiny", dict(groups=1, experts_per_group=6, k_group=1, k=3), -1),  # one group: the flat layer
    ("hier_tiny", dict(groups=5, experts_per_group=1, k_group=2, k=1), -1),  # one expert per group
    ("hier_top2x2", dict(T=1000), -1),
    ("hier_top2x2", dict(T=777, groups=8, experts_per_group=100, k_group=2, k=4, d_model=128, d_ff=256), 300),
    ("hier_top2x2", dict(T=500, groups=64, experts_per_group=2, k_group=4, k=2, d_model=64, d_ff=128), -1),
]


@pytest.mark.parametrize("name,over,cap", SMALL,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in o.items())}-C{c}" for n, o, c in SMALL])
def test_forward_hier_small(moelib, dev, name, over, cap):
    base = HIER_CONFIGS[name]
    cfg = hier_scaled(base, **over) if over else base
    inp = make_hier_inputs(cfg)
    say(f"[forward-hier] {cfg.name} C={cap}")
    got = _forward(moelib, dev, cfg, inp, cap)
    ref = oracle.forward_hier(oracle.HierSpec.of(cfg, capacity=cap), inp)
    _check(cfg, got, ref, np.arange(cfg.T))
    dead = np.flatnonzero((ref["slot_dest"] < 0).all(axis=1))
    assert np.all(as_f64(got["y"][dead], cfg.dtype) == 0.0)


def test_forward_hier_full_size(moelib, dev):
    cfg = HIER_CONFIGS["hier_top2x2"]
    inp = make_hier_inputs(cfg)
    say(f"[forward-hier] {cfg.name}")
    got = _forward(moelib, dev, cfg, inp)
    assert np.isfinite(as_f64(got["y"], cfg.dtype)).all()
    tokens = np.arange(cfg.T)  # every token: about 70 GFLOP of oracle FFN
    ref = oracle.forward_hier(oracle.HierSpec.of(cfg), inp, tokens=tokens)
    _check(cfg, got, ref, tokens)


def test_route_hier_matches_forward_routing(moelib, dev):
    """The gate entry point alone gives the same ids, gates, counts and losses."""
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import to_device, to_numpy, workspace

    cfg = hier_scaled(HIER_CONFIGS["hier_top2x2"], T=2000)
    inp = make_hier_inputs(cfg)
    p = _params(moelib, cfg)
    d = {k_: to_device(v, dev) for k_, v in inp.items()}
    idx = torch.empty((cfg.T, cfg.slots), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.slots), dtype=torch.float32, device=dev)
    cr = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    aux = torch.empty(4, dtype=torch.float32, device=dev)
    say("[route-hier]")
    moelib.moe_route_hier(p, d["x"], d["w_gate_p"], None, d["w_noise_p"], d["noise_p"], d["w_gate_s"], None,
                          d["w_noise_s"], d["noise_s"], idx, gate, cr, aux, workspace(p, moelib.MOE_OP_ROUTE_HIER, dev))
    torch.cuda.synchronize()
    ref = oracle.route_hier(oracle.HierSpec.of(cfg), inp)
    assert np.array_equal(to_numpy(idx), ref["topk_idx"])
    assert np.array_equal(to_numpy(cr), ref["counts_routed"])
    assert np.abs(to_numpy(gate) - ref["topk_gate"]).max() <= GATE_ATOL["f32"]
    aux_ok(to_numpy(aux), ref["aux"], 1e-4)

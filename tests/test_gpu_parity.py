"""GPU parity: every entry point of the C ABI against the CPU oracle on the
same seeded inputs.

Full-size cases run the five layer workloads at their real shapes in the
launch configuration the benchmark times; the oracle checks all integer
outputs and the gate logits exactly, the layer output on every token of the
three smaller workloads and, on the two largest, on 1024 random tokens plus
every dropped token and the tokens at every expert segment's edges, and the
expert FFN on segment edges plus random rows. Over the whole output, every
row must be finite and fully dropped tokens' rows exactly zero.
Small cases cover ragged and degenerate shapes element by element.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import GATE_ATOL, TOL, aux_ok, as_f64, rel_rows_ok, sample_rows, say
from synthetic import CONFIGS, f32_to_bf16_bits, make_inputs, scaled

pytestmark = pytest.mark.gpu

FULL = ["tiny_fp32", "switch_top1", "noisy_top4", "gshard_top2", "dropless_top1"]


@pytest.fixture(scope="module")
def dev(moelib):
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


_CACHE: dict = {}


def _case(name, **over):
    """Seeded inputs, the oracle's routing + dispatch, and device copies (cached per case)."""
    key = (name, tuple(sorted(over.items())))
    if key in _CACHE:
        return _CACHE[key]
    from sparsely_gated_mixture_gate_amd.buffers import to_device

    base = CONFIGS[name]
    cap = over.pop("capacity", -1)
    first_choice = bool(over.pop("first_choice", False))
    cfg = scaled(base, **over) if over else base
    say(f"[case] generating {cfg.name}")
    inp = make_inputs(cfg)
    spec = oracle.LayerSpec.of(cfg, capacity=cap, slot_major=first_choice)
    r = oracle.route(spec, inp)
    C = oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor, cap)
    disp = oracle.dispatch(r["topk_idx"], cfg.E, C, slot_major=first_choice)
    d_inp = {k_: to_device(v) for k_, v in inp.items()}
    out = dict(cfg=cfg, spec=spec, inp=inp, route=r, C=C, disp=disp, dev=d_inp, cap=cap, first_choice=first_choice)
    _CACHE[key] = out
    return out


def _params(moelib, c, gate_mode=0):
    cfg = c["cfg"]
    return moelib.make_params(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, cfg.renormalize,
                              cfg.capacity_factor, c["cap"], gate_mode, int(c.get("first_choice", False)))


def test_canonical_softplus_bitwise(moelib, dev):
    import torch

    rng = np.random.default_rng(0)
    lo, hi = np.float32(-100.0), np.float32(100.0)
    # every 61st fp32 bit pattern in [-100, 100] plus random values and edges
    pos = np.arange(0, int(np.array([hi]).view(np.uint32)[0]) + 1, 61, dtype=np.uint32).view(np.float32)
    z = np.concatenate([pos, -pos, rng.uniform(lo, hi, 1 << 20).astype(np.float32),
                        np.array([0.0, -0.0, 20.0, 20.000002, 19.999998, -87.0, -87.00001, 86.99999, -86.99999,
                                  1e-30, -1e-30, 1e-45, -1e-45], np.float32)])
    say(f"[softplus] n={z.size}")
    zt = torch.from_numpy(z).to(dev)
    out = torch.empty_like(zt)
    moelib.moe_canonical_softplus(zt, out)
    got = out.cpu().numpy()
    ref = oracle.softplus(z)
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} mismatches, e.g. z={z[bad[:5]]} gpu={got[bad[:5]]} cpu={ref[bad[:5]]}"


@pytest.mark.parametrize("name", FULL)
def test_route_full_size(moelib, dev, name):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import StepBuffers, to_numpy

    c = _case(name)
    cfg, r, d = c["cfg"], c["route"], c["dev"]
    p = _params(moelib, c)
    b = StepBuffers.alloc(p, dev)
    say(f"[route] {cfg.name}")
    moelib.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], b.topk_idx, b.topk_gate,
                     b.counts_routed, b.aux, b.logits, b.ws_route)
    torch.cuda.synchronize()
    H = to_numpy(b.logits)
    mism = np.flatnonzero(H.view(np.uint32).ravel() != r["H"].view(np.uint32).ravel())
    assert mism.size == 0, f"{mism.size} logits differ bitwise (first flat index {mism[:3]})"
    assert np.array_equal(to_numpy(b.topk_idx), r["topk_idx"])
    assert np.array_equal(to_numpy(b.counts_routed), r["counts_routed"])
    assert np.abs(to_numpy(b.topk_gate) - r["topk_gate"]).max() <= GATE_ATOL["f32"]
    aux_ok(to_numpy(b.aux), r["aux"], 1e-4)


MODES = {"auto": 0, "canonical": 1, "fallback": 2}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", FULL)
def test_route_gate_modes_full_size(moelib, dev, name, mode):
    """Without logits_out the bf16 layers (E <= 256) route through the
    certified MFMA gate; every mode must give the canonical routing."""
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import StepBuffers, to_numpy

    c = _case(name)
    cfg, r, d = c["cfg"], c["route"], c["dev"]
    p = _params(moelib, c, MODES[mode])
    b = StepBuffers.alloc(p, dev)
    say(f"[route-{mode}] {cfg.name}")
    moelib.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], b.topk_idx, b.topk_gate,
                     b.counts_routed, b.aux, None, b.ws_route)
    torch.cuda.synchronize()
    idx = to_numpy(b.topk_idx)
    bad = np.flatnonzero((idx != r["topk_idx"]).any(axis=1))
    assert bad.size == 0, f"{bad.size} tokens routed differently, e.g. {bad[:5]}: {idx[bad[:3]]} vs {r['topk_idx'][bad[:3]]}"
    assert np.array_equal(to_numpy(b.counts_routed), r["counts_routed"])
    tol = GATE_ATOL["f32"] if mode != "auto" else GATE_ATOL[cfg.dtype]
    gerr = np.abs(to_numpy(b.topk_gate) - r["topk_gate"]).max()
    say(f"  max gate error {gerr:.2e}")
    assert gerr <= tol
    aux_ok(to_numpy(b.aux), r["aux"], 1e-4)


@pytest.mark.parametrize("name", FULL)
def test_dispatch_full_size(moelib, dev, name):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import StepBuffers, to_device, to_numpy

    c = _case(name)
    cfg, disp, d = c["cfg"], c["disp"], c["dev"]
    p = _params(moelib, c)
    b = StepBuffers.alloc(p, dev)
    idx = to_device(c["route"]["topk_idx"])
    say(f"[dispatch] {cfg.name} R={disp['R']}")
    moelib.moe_dispatch(p, d["x"], idx, b.counts_kept, b.offsets, b.slot_dest, b.row_src, b.x_perm, b.ws_dispatch)
    torch.cuda.synchronize()
    R = disp["R"]
    assert np.array_equal(to_numpy(b.counts_kept), disp["counts_kept"])
    assert np.array_equal(to_numpy(b.offsets), disp["offsets"])
    assert np.array_equal(to_numpy(b.slot_dest), disp["slot_dest"])
    assert np.array_equal(to_numpy(b.row_src)[:R], disp["row_src"])
    xp = to_numpy(b.x_perm)[:R]
    assert np.array_equal(xp, c["inp"]["x"][disp["row_src"]])  # bit-exact copy


@pytest.mark.parametrize("name", FULL)
def test_expert_ffn_full_size(moelib, dev, name):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import StepBuffers, to_device, to_numpy

    c = _case(name)
    cfg, disp, d, inp = c["cfg"], c["disp"], c["dev"], c["inp"]
    p = _params(moelib, c)
    b = StepBuffers.alloc(p, dev)
    R = disp["R"]
    b.x_perm[:R] = to_device(inp["x"][disp["row_src"]])
    offs = to_device(disp["offsets"])
    say(f"[expert_ffn] {cfg.name} R={R}")
    moelib.moe_expert_ffn(p, b.x_perm, offs, d["w1"], d["w2"], b.y_perm, b.ws_ffn)
    torch.cuda.synchronize()
    rows = np.arange(R) if R * cfg.d_model * cfg.d_ff <= 2**27 else sample_rows(disp["offsets"], 64)
    row_exp = np.repeat(np.arange(cfg.E), disp["counts_kept"])
    ref = oracle.expert_ffn_rows(inp["x"], disp["row_src"][rows], row_exp[rows], inp["w1"], inp["w2"], cfg.act,
                                 cfg.dtype)
    got = as_f64(to_numpy(b.y_perm)[rows], cfg.dtype)
    rel_rows_ok(got, ref, TOL[cfg.dtype], f"y_perm {cfg.name}")


@pytest.mark.parametrize("name", FULL)
def test_combine_full_size(moelib, dev, name):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import StepBuffers, to_device, to_numpy

    c = _case(name)
    cfg, disp = c["cfg"], c["disp"]
    p = _params(moelib, c)
    b = StepBuffers.alloc(p, dev)
    R = disp["R"]
    rng = np.random.default_rng(1)
    yp = rng.standard_normal((max(R, 1), cfg.d_model)).astype(np.float32)
    if cfg.dtype == "bf16":
        yp = f32_to_bf16_bits(yp)
    gates32 = c["route"]["topk_gate"].astype(np.float32)
    b.y_perm[: yp.shape[0]] = to_device(yp)
    say(f"[combine] {cfg.name}")
    moelib.moe_combine(p, b.y_perm, to_device(disp["slot_dest"]), to_device(gates32), b.y)
    torch.cuda.synchronize()
    ref = oracle.combine(np.arange(cfg.T), disp["slot_dest"], gates32.astype(np.float64), as_f64(yp, cfg.dtype))
    rel_rows_ok(as_f64(to_numpy(b.y), cfg.dtype), ref, TOL[cfg.dtype], f"y {cfg.name}")


def _run_forward(moelib, c, dev, gate_mode=0):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import ForwardBuffers

    d = c["dev"]
    p = _params(moelib, c, gate_mode)
    fb = ForwardBuffers.alloc(p, dev)
    fb.y.fill_(float("nan"))  # every row must be written (dropped tokens' rows as exact zeros)
    fb.aux.fill_(float("nan"))  # aux has 3 values; the 4th (alignment padding) is never written
    moelib.moe_forward(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], d["w1"], d["w2"], fb.y,
                       fb.aux, fb.topk_idx, fb.topk_gate, fb.counts_routed, fb.counts_kept, fb.slot_dest, fb.ws)
    torch.cuda.synchronize()
    return fb


def _check_forward(c, fb, tokens):
    from sparsely_gated_mixture_gate_amd.buffers import to_numpy

    cfg, r, disp = c["cfg"], c["route"], c["disp"]
    assert np.array_equal(to_numpy(fb.topk_idx), r["topk_idx"])
    assert np.array_equal(to_numpy(fb.counts_routed), r["counts_routed"])
    assert np.array_equal(to_numpy(fb.counts_kept), disp["counts_kept"])
    assert np.array_equal(to_numpy(fb.slot_dest), disp["slot_dest"])
    assert np.abs(to_numpy(fb.topk_gate) - r["topk_gate"]).max(initial=0.0) <= GATE_ATOL[cfg.dtype]
    aux_ok(to_numpy(fb.aux), r["aux"], 1e-4)
    ref = oracle.forward(c["spec"], c["inp"], tokens=tokens)
    got = as_f64(to_numpy(fb.y)[tokens], cfg.dtype)
    rel_rows_ok(got, ref["y"], TOL[cfg.dtype], f"y {cfg.name}")


# workloads whose every token the oracle evaluates in seconds; the larger two check
# 1024 random tokens, every dropped token and the first / last token of every
# expert segment (the ragged edges of the GEMM tiles)
ALL_TOKENS = {"tiny_fp32", "switch_top1", "noisy_top4"}


def _forward_tokens(c):
    cfg, disp = c["cfg"], c["disp"]
    if cfg.name in ALL_TOKENS:
        return np.arange(cfg.T)
    rng = np.random.default_rng(2)
    dropped = np.flatnonzero((disp["slot_dest"] < 0).any(axis=1))
    edges = disp["row_src"][sample_rows(disp["offsets"], 0)] if disp["R"] else np.zeros(0, np.int64)
    return np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 1024), dropped, edges]))


def _check_whole_y(c, fb):
    """Over the whole output: every row finite (the NaN pre-fill is gone) and the
    row of every token whose slots were all dropped exactly zero."""
    import torch

    cfg, disp = c["cfg"], c["disp"]
    assert bool(torch.isfinite(fb.y).all()), "y has non-finite entries (a row was not written?)"
    dead = np.flatnonzero((disp["slot_dest"] < 0).all(axis=1))
    if dead.size:
        rows = fb.y[torch.from_numpy(dead).to(fb.y.device)]
        assert bool((rows == 0).all()), "a fully dropped token's row is not zero"
    say(f"  whole y finite; {dead.size} fully dropped rows are zero")


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size(moelib, dev, name):
    c = _case(name)
    cfg = c["cfg"]
    say(f"[forward] {cfg.name}")
    fb = _run_forward(moelib, c, dev)
    _check_whole_y(c, fb)
    tokens = _forward_tokens(c)
    say(f"  comparing {tokens.size} of {cfg.T} tokens with the oracle")
    _check_forward(c, fb, tokens)


@pytest.mark.parametrize("cap", [-1, 1024])
def test_forward_first_choice_full_size(moelib, dev, cap):
    """The top-2 workload with first-choice priority, at the capacity factor's
    C = 2048 and at C = 1024 (the T * cf / E reading, which drops ~4%)."""
    c = _case("gshard_top2", first_choice=True, capacity=cap)
    say(f"[forward-first-choice] C={c['C']} drops={int((c['disp']['slot_dest'] < 0).sum())}")
    fb = _run_forward(moelib, c, dev)
    _check_whole_y(c, fb)
    _check_forward(c, fb, _forward_tokens(c))


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_is_deterministic(moelib, dev, name):
    """Two forwards of the same inputs give the same bytes in every output."""
    from sparsely_gated_mixture_gate_amd.buffers import to_numpy

    c = _case(name)
    say(f"[determinism] {c['cfg'].name} x2")
    a = _run_forward(moelib, c, dev)
    b = _run_forward(moelib, c, dev)
    for f in ("y", "aux", "topk_idx", "topk_gate", "counts_routed", "counts_kept", "slot_dest"):
        assert to_numpy(getattr(a, f)).tobytes() == to_numpy(getattr(b, f)).tobytes(), f


SMALL = [
    # (workload, overrides) -- ragged T, tiny and degenerate shapes
    ("tiny_fp32", dict(T=1)),
    ("tiny_fp32", dict(T=77)),
    ("tiny_fp32", dict(T=300, E=1, k=1)),
    ("tiny_fp32", dict(T=129, E=3, k=3)),
    ("tiny_fp32", dict(T=200, capacity=20)),
    ("tiny_fp32", dict(T=100, capacity=0)),
    ("switch_top1", dict(T=1000)),
    ("switch_top1", dict(T=333, E=5, d_model=136, d_ff=200)),
    ("switch_top1", dict(T=700, capacity=3)),
    ("noisy_top4", dict(T=515)),
    ("noisy_top4", dict(T=64, E=8, k=8)),
    ("noisy_top4", dict(T=250, E=1000, k=8, d_model=64, d_ff=64)),
    ("gshard_top2", dict(T=1111, E=7, d_model=256, d_ff=1000)),
    ("gshard_top2", dict(T=2048, capacity=17)),
    ("dropless_top1", dict(T=999, d_model=512, d_ff=640)),
    # 256-row expert tiles: ragged K and N, more tiles than CUs (several per persistent block)
    ("dropless_top1", dict(T=40000, E=4, d_model=200, d_ff=328)),
    # 256-row tiles with d and f multiples of 64 (activation super-stages of 64 k): short K
    # (one or two super-stages, fewer than the rings hold), partial tiles, gathered and
    # scattered rows, top-2 through the combine
    ("dropless_top1", dict(T=20000, E=6, d_model=192, d_ff=320)),
    ("gshard_top2", dict(T=12000, E=8, d_model=64, d_ff=128)),
    ("dropless_top1", dict(T=9000, E=2, d_model=128, d_ff=64)),
    # count table too large for in-block prefixes (separate scan kernel)
    ("noisy_top4", dict(T=5000, E=512, k=8, d_model=64, d_ff=64)),
    # 256-row tiles with a capacity between 160 and 256 (row tiles past the segment skipped)
    ("gshard_top2", dict(T=4000, E=16, capacity=200, d_model=296, d_ff=520)),
    # first-choice priority drop order (GShard): binding capacities, k = 2, 3, 4, 8
    ("gshard_top2", dict(T=2048, capacity=17, first_choice=True)),
    ("gshard_top2", dict(T=1500, E=12, k=3, capacity=300, d_model=128, d_ff=256, first_choice=True)),
    ("noisy_top4", dict(T=515, capacity=9, first_choice=True)),
    ("noisy_top4", dict(T=64, E=8, k=8, capacity=50, first_choice=True)),
    ("tiny_fp32", dict(T=200, capacity=60, first_choice=True)),
]


@pytest.mark.parametrize("mode", ["auto", "fallback"])
@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in o.items())}" for n, o in SMALL])
def test_forward_small_shapes(moelib, dev, name, over, mode):
    c = _case(name, **over)
    say(f"[forward-small-{mode}] {c['cfg'].name} C={c['C']}")
    fb = _run_forward(moelib, c, dev, MODES[mode])
    _check_forward(c, fb, np.arange(c["cfg"].T))


def test_forward_empty_batch(moelib, dev):
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import ForwardBuffers, to_device, to_numpy

    cfg = scaled(CONFIGS["switch_top1"], T=8)
    inp = make_inputs(cfg)
    p = moelib.make_params(0, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, False, 1.25)
    fb = ForwardBuffers.alloc(p, dev)
    d = {k: to_device(v) for k, v in inp.items()}
    say("[forward-empty]")
    moelib.moe_forward(p, d["x"], d["w_gate"], None, None, None, d["w1"], d["w2"], fb.y, fb.aux, fb.topk_idx,
                       fb.topk_gate, fb.counts_routed, fb.counts_kept, fb.slot_dest, fb.ws)
    torch.cuda.synchronize()
    assert np.all(to_numpy(fb.counts_routed) == 0) and np.all(to_numpy(fb.counts_kept) == 0)


def test_zero_gate_ties_and_identity_experts(moelib, dev):
    """W_g = 0: every logit ties, expert 0 wins everywhere, capacity keeps the
    first C tokens; identity experts make y = gate * x exactly checkable."""
    import torch
    from sparsely_gated_mixture_gate_amd.buffers import ForwardBuffers, to_device, to_numpy

    cfg = scaled(CONFIGS["switch_top1"], T=3000)
    inp = make_inputs(cfg, with_weights=False)
    d, f, E = cfg.d_model, cfg.d_ff, cfg.E
    inp["w_gate"] = np.zeros_like(inp["w_gate"])
    w1 = np.zeros((E, d, f), np.float32)
    w2 = np.zeros((E, f, d), np.float32)
    w1[:, :, :d] = np.eye(d)
    w1[:, :, d:2 * d] = -np.eye(d)
    w2[:, :d, :] = np.eye(d)
    w2[:, d:2 * d, :] = -np.eye(d)
    inp["w1"], inp["w2"] = f32_to_bf16_bits(w1), f32_to_bf16_bits(w2)
    C = 500
    p = moelib.make_params(cfg.T, d, f, E, 1, "bf16", "gelu", False, 0.0, C)
    fb = ForwardBuffers.alloc(p, dev)
    dv = {k: to_device(v) for k, v in inp.items()}
    say("[forward-ties-identity]")
    moelib.moe_forward(p, dv["x"], dv["w_gate"], None, None, None, dv["w1"], dv["w2"], fb.y, fb.aux, fb.topk_idx,
                       fb.topk_gate, fb.counts_routed, fb.counts_kept, fb.slot_dest, fb.ws)
    torch.cuda.synchronize()
    assert np.all(to_numpy(fb.topk_idx) == 0)
    sd = to_numpy(fb.slot_dest)[:, 0]
    assert np.array_equal(sd[:C], np.arange(C)) and np.all(sd[C:] == -1)
    assert np.allclose(to_numpy(fb.topk_gate), 1.0 / E, rtol=1e-6)
    x = as_f64(inp["x"], "bf16")
    y = as_f64(to_numpy(fb.y), "bf16")
    rel_rows_ok(y[:C], x[:C] / E, TOL["bf16"], "identity y")
    assert np.all(y[C:] == 0.0)


@pytest.mark.parametrize("name,over", [("switch_top1", dict(T=2048)), ("gshard_top2", dict(T=1024)),
                                       ("noisy_top4", dict(T=2048, d_model=128, d_ff=64))])
def test_twin_gate_columns(moelib, dev, name, over):
    """Every gate column has an identical twin (column 2j+1 = column 2j), so every
    token's top-(k+1) ties exactly: no token is certified, and each block
    recomputes the tied candidates of all its tokens canonically (over a hundred
    (token, expert) pairs, several LDS rounds). Ties go to the lower expert index.
    The noisy case twins the noise columns too and draws no noise (eps = 0), so its
    logits tie the same way and every pair runs its gate and noise chains."""
    from sparsely_gated_mixture_gate_amd.buffers import to_device

    cfg = scaled(CONFIGS[name], **over)
    inp = make_inputs(cfg)
    wg = inp["w_gate"].copy()
    wg[:, 1::2] = wg[:, 0::2]
    inp["w_gate"] = wg
    if inp.get("w_noise") is not None:
        wn = inp["w_noise"].copy()
        wn[:, 1::2] = wn[:, 0::2]
        inp["w_noise"] = wn
        inp["noise"] = np.zeros_like(inp["noise"])
    spec = oracle.LayerSpec.of(cfg, capacity=-1)
    r = oracle.route(spec, inp)
    C = oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor, -1)
    c = dict(cfg=cfg, spec=spec, inp=inp, route=r, C=C, disp=oracle.dispatch(r["topk_idx"], cfg.E, C),
             dev={k_: to_device(v) for k_, v in inp.items()}, cap=-1)
    assert np.all(r["topk_idx"][:, 0] % 2 == 0)  # the oracle breaks the ties toward the lower index
    say(f"[forward-twin-columns] {cfg.name}")
    fb = _run_forward(moelib, c, dev)
    rng = np.random.default_rng(5)
    _check_forward(c, fb, np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, 48)])))


def test_forward_small_is_deterministic(moelib, dev):
    from sparsely_gated_mixture_gate_amd.buffers import to_numpy

    c = _case("noisy_top4", T=4000)
    say("[determinism] noisy_top4 T=4000 x2")
    a = _run_forward(moelib, c, dev)
    b = _run_forward(moelib, c, dev)
    for f in ("y", "aux", "topk_idx", "topk_gate", "counts_routed", "counts_kept", "slot_dest"):
        x, y = to_numpy(getattr(a, f)), to_numpy(getattr(b, f))
        assert x.tobytes() == y.tobytes(), f

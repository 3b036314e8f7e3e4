"""GPU parity of the gated variant (efla_fwd_chunked_gated and
efla_fwd_recurrent_step_gated, through the C ABI) against the fp64 oracle's
gated forward, on the same seeded inputs.

Reading (papernotes note: main results "Gated EFLA", key findings): Gated
DeltaNet's update with the exact-flow coefficient,
S_t = g_t (I - c_t k_t k_t^T) S_{t-1} + c_t k_t v_t^T, g_t = exp(log_g_t).
Bars and error metric as for the ungated forward: normwise per head,
1e-4 for fp32 inputs and 2e-2 for bf16.
"""
import sys

import pytest
import torch

import efla_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def efla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_efla_amd as m

    m.load_library()
    return m


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def normwise(x, ref):
    x = torch.as_tensor(x).double().cpu()
    ref = torch.as_tensor(ref).double()
    if x.dim() == 1:
        x, ref = x[None, None], ref[None, None]
    err = (x - ref).abs().flatten(-2).amax(-1)
    return float((err / ref.abs().flatten(-2).amax(-1).clamp_min(1e-30)).max())


def dev(x):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_gated(efla, x, lg, chunk, coef="exact"):
    g = dev(x)
    o, s = efla.efla_fwd_chunked_gated(g["q"], g["k"], g["v"], g["beta"], lg.cuda(), g["s0"], chunk=chunk,
                                       coef=coef)
    torch.cuda.synchronize()
    return o.float().cpu(), s.cpu()


CASES = [(dt, d, c) for dt in ("f32", "bf16") for d in (16, 32, 64, 128) for c in (16, 32, 64)]


@pytest.mark.parametrize("dt,d,c", CASES)
@pytest.mark.parametrize("with_s0", [False, True])
def test_gated_small_ragged(efla, dt, d, c, with_s0):
    T = 3 * c + 5
    note(f"[gated small] dtype={dt} d={d} chunk={c} T={T} s0={with_s0}")
    x = efla_inputs.random_case(7000 + d + c, B=2, H=3, T=T, d=d, dtype=dt, s0_std=0.5 if with_s0 else 0.0)
    lg = efla_inputs.log_decay(7100 + d + c, (2, 3, T))
    o, s = run_gated(efla, x, lg, c)
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"], nthreads=8)
    eo, es = normwise(o, o_ref), normwise(s, s_ref)
    note(f"   err o={eo:.3e} S_T={es:.3e} (tol {TOL[dt]})")
    assert eo <= TOL[dt] and es <= TOL[dt]


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("T", [1, 7, 64, 65, 200])
def test_gated_edge_lengths(efla, dt, d, T):
    x = efla_inputs.random_case(300 + T, B=1, H=2, T=T, d=d, dtype=dt, s0_std=0.3)
    lg = efla_inputs.log_decay(301 + T, (1, 2, T))
    o, s = run_gated(efla, x, lg, 64)
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"])
    assert normwise(o, o_ref) <= TOL[dt] and normwise(s, s_ref) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gated_strong_decays(efla, dt):
    """Decays down to e^-6 per token: the in-chunk factors span e^-378; every
    factor the kernel forms is exp of a nonpositive exponent, and outputs stay
    finite and match."""
    T, d = 300, 64
    x = efla_inputs.random_case(55, B=1, H=4, T=T, d=d, dtype=dt, s0_std=1.0)
    lg = -6.0 * torch.rand((1, 4, T), generator=torch.Generator().manual_seed(56))
    o, s = run_gated(efla, x, lg, 64)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"])
    assert normwise(o, o_ref) <= TOL[dt] and normwise(s, s_ref) <= TOL[dt]


def test_zero_log_decay_matches_ungated(efla):
    x = efla_inputs.random_case(77, B=2, H=2, T=333, d=128, dtype="bf16", s0_std=0.3)
    lg = torch.zeros((2, 2, 333))
    o, s = run_gated(efla, x, lg, 64)
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["s0"])
    assert normwise(o, o_ref) <= 2e-2 and normwise(s, s_ref) <= 2e-2


@pytest.mark.parametrize("dt,d,c", [("f32", 64, 32), ("bf16", 128, 64)])
@pytest.mark.parametrize("rule", ["euler", "rk4", "order2"])
def test_gated_step_rules(efla, rule, dt, d, c):
    """Every step rule, on the 4-wave kernel (fp32) and on the pipelined
    kernel's gated pass (bf16, 64-token chunks)."""
    modes = {"euler": oracle.EULER, "rk4": oracle.RK4, "order2": oracle.ORDER2}
    x = efla_inputs.random_case(90, B=1, H=3, T=150, d=d, dtype=dt, k_lo=0.3, k_hi=1.3, s0_std=0.3)
    lg = efla_inputs.log_decay(91, (1, 3, 150))
    note(f"[gated rule] {rule} dtype={dt} d={d} chunk={c}")
    o, s = run_gated(efla, x, lg, c, coef=rule)
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"], mode=modes[rule])
    assert normwise(o, o_ref) <= TOL[dt] and normwise(s, s_ref) <= TOL[dt]


@pytest.mark.parametrize("dt,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_gated_growth(efla, dt, d):
    """Log-decays of both signs (g up to e^0.05 > 1): the decay factors the
    kernels form then exceed 1 below the diagonal and must not be clamped."""
    T = 200
    x = efla_inputs.random_case(61, B=1, H=2, T=T, d=d, dtype=dt, s0_std=0.5)
    lg = -0.3 + 0.35 * torch.rand((1, 2, T), generator=torch.Generator().manual_seed(62))
    note(f"[gated growth] dtype={dt} d={d}")
    o, s = run_gated(efla, x, lg, 64)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"])
    assert normwise(o, o_ref) <= TOL[dt] and normwise(s, s_ref) <= TOL[dt]


def test_gated_in_place_state(efla):
    """s_final aliasing s0 (the state advanced in place) gives the same bits
    as separate buffers, and both match the oracle."""
    T, d = 333, 128
    x = efla_inputs.random_case(81, B=2, H=3, T=T, d=d, dtype="bf16", s0_std=0.4)
    lg = efla_inputs.log_decay(82, (2, 3, T))
    g = dev(x)
    lgd = lg.cuda()
    o1, s1 = efla.efla_fwd_chunked_gated(g["q"], g["k"], g["v"], g["beta"], lgd, g["s0"], chunk=64)
    st = g["s0"].clone()
    o2, s2 = efla.efla_fwd_chunked_gated(g["q"], g["k"], g["v"], g["beta"], lgd, st, chunk=64, s_final=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, st)
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"])
    assert normwise(o2.float().cpu(), o_ref) <= 2e-2 and normwise(st.cpu(), s_ref) <= 2e-2


def test_gated_deterministic_bitwise(efla):
    """Two launches of the gated forward on the same inputs give identical
    bits (no atomics, fixed reduction order)."""
    T, d = 1000, 128
    x = efla_inputs.random_case(83, B=2, H=8, T=T, d=d, dtype="bf16", s0_std=0.2)
    lg = efla_inputs.log_decay(84, (2, 8, T)).cuda()
    g = dev(x)
    o1, s1 = efla.efla_fwd_chunked_gated(g["q"], g["k"], g["v"], g["beta"], lg, g["s0"], chunk=64)
    o2, s2 = efla.efla_fwd_chunked_gated(g["q"], g["k"], g["v"], g["beta"], lg, g["s0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_gated_full_size_layer(efla):
    """The 1.3B-layer shape (128 heads x T = 4096, bf16, random S0) with
    per-token decays, every head against the oracle."""
    w = efla_inputs.WORKLOADS["layer1p3b_d128"]
    x = efla_inputs.make_inputs(w)
    lg = efla_inputs.log_decay(4343, (w.B, w.H, w.T))
    note(f"[gated full] {w.name} B={w.B} H={w.H} T={w.T}")
    o, s = run_gated(efla, x, lg, w.chunk)
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"], nthreads=16)
    eo, es = normwise(o, o_ref), normwise(s, s_ref)
    note(f"PARITY {{\"case\": \"gated {w.name}\", \"heads\": {w.B * w.H}, \"o\": {eo}, \"S_T\": {es}}}")
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_gated_decode_continues_chunked(efla, dt, d):
    """A gated chunked forward, then 10 gated decode steps from its final
    state, against the oracle over the whole sequence."""
    T, steps = 100, 10
    x = efla_inputs.random_case(500 + d, B=2, H=3, T=T + steps, d=d, dtype=dt, s0_std=0.4)
    lg = efla_inputs.log_decay(501 + d, (2, 3, T + steps))
    g = dev(x)
    lgd = lg.cuda()
    sl = lambda t: t[:, :, :T].contiguous()
    _, st = efla.efla_fwd_chunked_gated(sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(g["beta"]), sl(lgd), g["s0"],
                                        chunk=32)
    outs = []
    for i in range(T, T + steps):
        tok = lambda t: t[:, :, i].contiguous()
        outs.append(efla.efla_fwd_recurrent_step_gated(tok(g["q"]), tok(g["k"]), tok(g["v"]), tok(g["beta"]),
                                                       tok(lgd), st))
    od = torch.stack(outs, 2).float().cpu()
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd_gated(x["q"], x["k"], x["v"], x["beta"], lg, x["s0"])
    assert normwise(od, o_ref[:, :, T:]) <= TOL[dt] and normwise(st.cpu(), s_ref) <= TOL[dt]


def test_gated_rejects_missing_gate(efla):
    x = dev(efla_inputs.random_case(1, B=1, H=1, T=10, d=64, dtype="bf16"))
    with pytest.raises(ValueError):
        efla.efla_fwd_chunked_gated(x["q"], x["k"], x["v"], x["beta"], torch.zeros(1, 1, 9, device="cuda"))

"""GPU parity of the backward (efla_bwd_chunked, through the C ABI) against
the fp64 oracle's reverse mode, on the same seeded inputs and upstream
gradients.

Error metric as for the forward: per head and per output, max|x - x_ref| /
max|x_ref|. Bars: 1e-4 for fp32 inputs; 2e-2 for bf16 inputs (for bf16 the
recomputed forward states, the backward's products and the stored states and
state gradients use bf16 operands with fp32 accumulation, and the outputs are
rounded to bf16).
"""
import sys

import numpy as np
import pytest
import torch

import efla_inputs
import oracle

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": 1e-4, "bf16": 2e-2}
RULES = {"exact": oracle.EXACT, "euler": oracle.EULER, "rk4": oracle.RK4, "order2": oracle.ORDER2}


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
    if x.dim() == ref.dim() and x.dim() >= 2:
        err = (x - ref).abs().flatten(-2).amax(-1)
        scale = ref.abs().flatten(-2).amax(-1).clamp_min(1e-30)
    else:
        err = (x - ref).abs().amax(-1)
        scale = ref.abs().amax(-1).clamp_min(1e-30)
    return float((err / scale).max())


def upstream(seed, B, H, T, d, dt, with_ds):
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn((B, H, T, d), generator=g).to(DT[dt])
    dsT = torch.randn((B, H, d, d), generator=g) if with_ds else None
    return dout, dsT


def run_case(efla, dt, d, c, B, H, T, s0_std, with_ds, rule="exact", k_hi=3.0, seed=0):
    x = efla_inputs.random_case(9000 + seed + d + c + T, B=B, H=H, T=T, d=d, dtype=dt,
                                k_lo=0.3, k_hi=k_hi, s0_std=s0_std)
    dout, dsT = upstream(9100 + seed + T, B, H, T, d, dt, with_ds)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    got = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout.cuda(), dev["s0"],
                                None if dsT is None else dsT.cuda(), chunk=c, coef=rule)
    torch.cuda.synchronize()
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["beta"], dout, x["s0"], dsT, mode=RULES[rule],
                     nthreads=8)
    errs = {}
    for name, gv, rv in zip(("dq", "dk", "dv", "dbeta", "ds0"), got, ref):
        errs[name] = normwise(gv.float().cpu(), rv)
    return errs


CASES = [(dt, d, c) for dt in ("f32", "bf16") for d in (16, 32, 64, 128) for c in (16, 32, 64)
         if not (dt == "f32" and d == 128 and c == 64)]


@pytest.mark.parametrize("dt,d,c", CASES)
def test_backward_small_ragged(efla, dt, d, c):
    T = 3 * c + 5
    note(f"[bwd small] dtype={dt} d={d} chunk={c} T={T}")
    errs = run_case(efla, dt, d, c, 2, 2, T, 0.5, True)
    note("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (tol {TOL[dt]})")
    assert all(v <= TOL[dt] for v in errs.values()), errs


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("T", [1, 17, 64, 65])
def test_backward_edge_lengths(efla, dt, d, T):
    note(f"[bwd edge] dtype={dt} d={d} T={T}")
    errs = run_case(efla, dt, d, 64, 1, 2, T, 0.3, T % 2 == 1)
    assert all(v <= TOL[dt] for v in errs.values()), errs


@pytest.mark.parametrize("rule", ["euler", "rk4", "order2"])
@pytest.mark.parametrize("dt,d,c", [("f32", 64, 32), ("bf16", 128, 64)])
def test_backward_step_rules(efla, rule, dt, d, c):
    note(f"[bwd rule {rule}] dtype={dt} d={d} chunk={c}")
    errs = run_case(efla, dt, d, c, 1, 3, 150, 0.3, True, rule=rule, k_hi=1.3)
    note("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL[dt] for v in errs.values()), errs


def test_backward_longer_sequence_bf16(efla):
    note("[bwd long] bf16 d=128 C=64 T=1000, stiff keys")
    errs = run_case(efla, "bf16", 128, 64, 1, 2, 1000, 0.1, True, k_hi=10.0, seed=5)
    note("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_backward_without_optional_tensors(efla):
    """No s0, no dS_T, no ds0 output."""
    x = efla_inputs.random_case(4321, B=1, H=2, T=70, d=32, dtype="f32")
    dout, _ = upstream(4322, 1, 2, 70, 32, "f32", False)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    dq, dk, dv, db, ds0 = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"],
                                                dout.cuda(), None, None, chunk=32, want_ds0=False)
    torch.cuda.synchronize()
    assert ds0 is None
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["beta"], dout, None, None)
    for gv, rv in zip((dq, dk, dv, db), ref):
        assert normwise(gv.cpu(), rv) <= 1e-4


def test_backward_is_deterministic(efla):
    x = efla_inputs.random_case(77, B=2, H=2, T=300, d=64, dtype="bf16", s0_std=0.3)
    dout, dsT = upstream(78, 2, 2, 300, 64, "bf16", True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    runs = [efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout.cuda(), dev["s0"],
                                  dsT.cuda(), chunk=64) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_backward_full_size(efla):
    """The 1.3B-layer shape at full size (128 heads x T = 4096, bf16, random
    S0) in the launch configuration the bench times; the oracle's reverse mode
    on 32 heads spread over the grid: both column slices of a head, and heads
    whose workgroups land on each of the eight XCD positions (each head's
    gradients depend only on its own inputs)."""
    w = efla_inputs.WORKLOADS["layer1p3b_d128"]
    note(f"[bwd full] {w.name}: B={w.B} H={w.H} T={w.T} d={w.d} chunk={w.chunk} {w.dtype}")
    x = efla_inputs.make_inputs(w)
    dout, dsT = upstream(4242, w.B, w.H, w.T, w.d, w.dtype, True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    got = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout.cuda(), dev["s0"], dsT.cuda(),
                                chunk=w.chunk)
    torch.cuda.synchronize()
    nh = w.B * w.H
    # 32 heads: every 4th, offset so that the heads cover all residues mod 8
    heads = sorted({(4 * i + (i // 8)) % nh for i in range(32)})
    flat = lambda t: t.reshape((nh,) + tuple(t.shape[2:]))
    sel = lambda t: flat(t)[heads]
    ref = oracle.bwd(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["beta"]), sel(dout), sel(x["s0"]), sel(dsT),
                     nthreads=16)
    errs = {}
    for name, gv, rv in zip(("dq", "dk", "dv", "dbeta", "ds0"), got, ref):
        errs[name] = normwise(sel(gv.float().cpu()), rv)
    note("   heads " + str(heads) + ": " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs

"""GPU parity of the training-step pair (through the C ABI):
efla_fwd_chunked_train writes the forward's outputs and keeps the chunk-start
states in the backward's workspace; efla_bwd_chunked_saved takes them from
there instead of recomputing the forward.

Checked on the same seeded inputs: the outputs against the fp64 oracle's
forward (the forward's bars), the gradients against the oracle's reverse mode
(the backward's bars), and the gradients against efla_bwd_chunked, which must
give the same values: both run the same state pass (or the same states in the
same order) and the same gradient kernels.
"""
import sys

import pytest
import torch

import efla_inputs
import oracle

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
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
    err = (x - ref).abs().flatten(-2).amax(-1)
    scale = ref.abs().flatten(-2).amax(-1).clamp_min(1e-30)
    return float((err / scale).max())


def inputs(seed, dt, d, B, H, T):
    x = efla_inputs.random_case(seed, B=B, H=H, T=T, d=d, dtype=dt, k_lo=0.3, k_hi=3.0, s0_std=0.3)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn((B, H, T, d), generator=g).to(DT[dt])
    dsT = torch.randn((B, H, d, d), generator=g)
    return x, dout, dsT


# (dtype, d, chunk, T): single-pass cases, and fp32 C = 64 at d <= 64, where
# the forward runs the 4-wave kernel and the states pass runs at chunk 32
CASES = [("bf16", 128, 64, 150), ("bf16", 64, 32, 77), ("bf16", 32, 16, 40), ("bf16", 16, 64, 65),
         ("f32", 128, 32, 100), ("f32", 64, 16, 33), ("f32", 64, 64, 70), ("f32", 16, 64, 129)]


@pytest.mark.parametrize("dt,d,c,T", CASES)
def test_train_forward_and_saved_backward(efla, dt, d, c, T):
    B, H = 1, 3
    note(f"[train] dtype={dt} d={d} chunk={c} T={T}")
    x, dout, dsT = inputs(6000 + d + c + T, dt, d, B, H, T)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o, sT, saved = efla.efla_fwd_chunked_train(dev["q"], dev["k"], dev["v"], dev["beta"], dev["s0"], chunk=c)
    got_saved = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout.cuda(), None, dsT.cuda(),
                                      chunk=c, saved_workspace=saved)
    got_plain = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout.cuda(), dev["s0"],
                                      dsT.cuda(), chunk=c)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["s0"], nthreads=3)
    eo, es = normwise(o.float().cpu(), o_ref), normwise(sT.cpu(), s_ref)
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["beta"], dout, x["s0"], dsT, nthreads=3)
    errs = {n: normwise(gv.float().cpu(), rv) for n, gv, rv in zip(("dq", "dk", "dv", "dbeta", "ds0"), got_saved, ref)}
    note(f"   o={eo:.2e} sT={es:.2e} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert eo <= TOL[dt] and es <= TOL[dt]
    assert all(v <= TOL[dt] for v in errs.values()), errs
    for a, b in zip(got_saved, got_plain):
        assert torch.equal(a, b)


def test_train_forward_in_place_state(efla):
    """s_final aliasing s0 advances the state in place, as the plain forward."""
    x, _, _ = inputs(6100, "bf16", 64, 1, 2, 90)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o_ref, s_ref = efla.efla_fwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dev["s0"].clone(), chunk=64)
    st = dev["s0"].clone()
    o, s, _ = efla.efla_fwd_chunked_train(dev["q"], dev["k"], dev["v"], dev["beta"], st, chunk=64, s_final=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert normwise(o.float().cpu(), o_ref.float().cpu()) <= TOL["bf16"]
    assert normwise(st.cpu(), s_ref.cpu()) <= TOL["bf16"]


def test_train_step_full_size(efla):
    """The 1.3B-layer shape at full size (128 heads x T = 4096, bf16) in the
    launch configuration the bench times: the training forward equals the
    plain forward to the bf16 bar, and the saved-state backward equals the
    recomputing backward exactly."""
    w = efla_inputs.WORKLOADS["layer1p3b_d128"]
    note(f"[train full] {w.name}: B={w.B} H={w.H} T={w.T} d={w.d} chunk={w.chunk} {w.dtype}")
    x = efla_inputs.make_inputs(w)
    g = torch.Generator().manual_seed(4343)
    dout = torch.randn((w.B, w.H, w.T, w.d), generator=g).to(DT[w.dtype]).cuda()
    dsT = torch.randn((w.B, w.H, w.d, w.d), generator=g).cuda()
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o1, s1 = efla.efla_fwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dev["s0"], chunk=w.chunk)
    o2, s2, saved = efla.efla_fwd_chunked_train(dev["q"], dev["k"], dev["v"], dev["beta"], dev["s0"], chunk=w.chunk)
    gs = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout, None, dsT, chunk=w.chunk,
                               saved_workspace=saved)
    gp = efla.efla_bwd_chunked(dev["q"], dev["k"], dev["v"], dev["beta"], dout, dev["s0"], dsT, chunk=w.chunk)
    torch.cuda.synchronize()
    eo = normwise(o2.float().cpu(), o1.float().cpu())
    es = normwise(s2.cpu(), s1.cpu())
    note(f"   train vs plain forward: o={eo:.2e} sT={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    for a, b in zip(gs, gp):
        assert torch.equal(a, b)

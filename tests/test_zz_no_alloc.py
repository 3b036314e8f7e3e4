"""efla_fwd_chunked_noalloc (the entry point that allocates nothing) against
efla_fwd_chunked, through the C ABI, on two calls in a row: the second with
a smaller input. Both shapes take the time-segmented path, so the fixed
scratch array carries the segment maps and start states; the no-allocation
call must give exactly the workspace call's bits, and both the oracle's
results within the bf16 bar."""
import pytest
import torch

import efla_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def efla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_efla_amd as m

    m.load_library()
    return m


def normwise(x, ref):
    x = torch.as_tensor(x).double().cpu()
    ref = torch.as_tensor(ref).double()
    err = (x - ref).abs().flatten(-2).amax(-1)
    return float((err / ref.abs().flatten(-2).amax(-1).clamp_min(1e-30)).max())


# (B, H, T, d, chunk, s0): the larger call first, then a smaller one
CALLS = [(1, 3, 9000, 128, 64, True), (1, 2, 4133, 128, 64, False)]


def test_noalloc_matches_workspace_entry_two_calls(efla):
    for i, (B, H, T, d, c, with_s0) in enumerate(CALLS):
        need = efla.efla_fwd_chunked_workspace_bytes(B, H, T, d, d, c, torch.bfloat16)
        print(f"[noalloc call {i}] B={B} H={H} T={T} d={d} chunk={c} s0={with_s0} workspace={need}",
              flush=True)
        assert 0 < need <= 24 << 20, "shape meant to use the scratch"
        x = efla_inputs.random_case(31337 + i, B=B, H=H, T=T, d=d, dtype="bf16",
                                    s0_std=0.3 if with_s0 else 0.0)
        g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        o_ref, s_ref = efla.efla_fwd_chunked(g["q"], g["k"], g["v"], g["beta"], g["s0"], chunk=c)
        o = torch.full_like(o_ref, float("nan"))
        s = torch.full_like(s_ref, float("nan"))
        efla.efla_fwd_chunked_noalloc(g["q"], g["k"], g["v"], g["beta"], g["s0"], o, s, chunk=c)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(s, s_ref)
        oo, so = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["s0"], nthreads=16)
        assert normwise(o.float().cpu(), oo) <= 2e-2 and normwise(s.cpu(), so) <= 2e-2


def test_noalloc_one_pass_and_errors(efla):
    """A shape that needs no workspace runs without touching the scratch; bad
    arguments come back as the workspace entry point's errors."""
    x = efla_inputs.random_case(5, B=2, H=4, T=300, d=64, dtype="bf16", s0_std=0.2)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o_ref, s_ref = efla.efla_fwd_chunked(g["q"], g["k"], g["v"], g["beta"], g["s0"], chunk=32)
    o, s = torch.empty_like(o_ref), torch.empty_like(s_ref)
    efla.efla_fwd_chunked_noalloc(g["q"], g["k"], g["v"], g["beta"], g["s0"], o, s, chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(s, s_ref)
    with pytest.raises(efla.EflaError) as ei:
        efla.efla_fwd_chunked_noalloc(g["q"], g["k"], g["v"], g["beta"], None, o, None, chunk=48)
    assert ei.value.status == 3

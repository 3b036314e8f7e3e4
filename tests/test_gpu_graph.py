"""Decode steps captured in a HIP graph (the form a serving loop launches
them in: no host launch per step) against the same steps launched eagerly.

Each replay starts from the same state (reset by an eager copy outside the
graph), with other eager work and synchronizations between the replays, and
every replay must equal the eager steps bit for bit: the decode kernel has
no atomics and a fixed reduction order, and the graph records only kernel
launches (no memset nodes).
"""
import sys

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


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("gated", [False, True])
def test_decode_steps_in_a_hip_graph(efla, gated):
    B, H, d, steps = 2, 4, 128, 8
    x = efla_inputs.random_case(501, B=B, H=H, T=steps, d=d, dtype="bf16", s0_std=0.3)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    toks = [tuple(dev[n][:, :, i].contiguous() for n in ("q", "k", "v", "beta")) for i in range(steps)]
    lg = efla_inputs.log_decay(502, (B, H, steps)).cuda()
    lgs = [lg[:, :, i].contiguous() for i in range(steps)]
    st0 = dev["s0"].clone()

    def step(i, st, o):
        if gated:
            efla.efla_fwd_recurrent_step_gated(*toks[i], lgs[i], st, o=o)
        else:
            efla.efla_fwd_recurrent_step(*toks[i], st, o=o)

    # eager reference
    st_e = st0.clone()
    o_e = [torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    for i in range(steps):
        step(i, st_e, o_e[i])
    torch.cuda.synchronize()

    # the same steps captured once (capture runs nothing), then replayed
    st_g = st0.clone()
    o_g = [torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i, st_g, o_g[i])
    torch.cuda.synchronize()
    note(f"[graph decode] gated={gated} B={B} H={H} d={d} steps={steps}")
    for rep in range(3):
        st_g.copy_(st0)
        for o in o_g:
            o.zero_()
        junk = torch.randn(4096, device="cuda").square().sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(st_g, st_e), f"replay {rep}: state differs from the eager steps"
        for i in range(steps):
            assert torch.equal(o_g[i], o_e[i]), f"replay {rep}: output of step {i} differs"

    # and the eager steps themselves against the oracle's sequential steps
    S = x["s0"].double().numpy().copy()
    for i in range(steps):
        for b in range(B):
            for h in range(H):
                if gated:
                    S[b, h], _ = oracle.step_gated(toks[i][0][b, h].cpu(), toks[i][1][b, h].cpu(),
                                                   toks[i][2][b, h].cpu(), float(toks[i][3][b, h].float()),
                                                   float(lgs[i][b, h]), S[b, h])
                else:
                    S[b, h], _ = oracle.step(toks[i][0][b, h].cpu(), toks[i][1][b, h].cpu(),
                                             toks[i][2][b, h].cpu(), float(toks[i][3][b, h].float()), S[b, h])
    err = (st_e.double().cpu().numpy() - S).reshape(B * H, -1)
    rel = abs(err).max(axis=1) / abs(S.reshape(B * H, -1)).max(axis=1)
    assert rel.max() <= 2e-2

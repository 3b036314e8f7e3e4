"""CPU-side checks of the C ABI: the library loads, exports every function
that include/efla.h declares, and rejects bad arguments on the host before
any launch (no GPU call is made by these tests)."""
import ctypes
import os
import re

import pytest

import delta_rule_recurrent_efla_amd as efla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "efla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(efla.LIB_PATH),
                                reason="libefla.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(efla_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("efla_fwd_chunked", "efla_fwd_recurrent_step", "efla_fwd_chunked_workspace_bytes",
              "efla_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(efla.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in efla.STATUS_NAMES.items():
        assert efla.status_string(code).startswith(name)
    assert efla.status_string(99) == "EFLA_ERR_UNKNOWN"


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def chunked(lib, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, s0=None, o=FAKE, sf=None, ws=None, wsb=0,
            B=1, H=1, T=8, dk=64, dv=64, chunk=64, coef=0, dt=1):
    return lib.efla_fwd_chunked(q, k, v, beta, s0, o, sf, ws, wsb, B, H, T, dk, dv, chunk, coef,
                                dt, None)


def step(lib, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, state=FAKE, o=FAKE, B=1, H=1, dk=64, dv=64,
         coef=0, dt=1):
    return lib.efla_fwd_recurrent_step(q, k, v, beta, state, o, B, H, dk, dv, coef, dt, None)


def test_chunked_rejects_bad_arguments_before_launch():
    lib = efla.load_library()
    assert chunked(lib, q=None) == 1
    assert chunked(lib, beta=None) == 1
    assert chunked(lib, o=None) == 1
    assert chunked(lib, B=0) == 2
    assert chunked(lib, H=-1) == 2
    assert chunked(lib, T=0) == 2
    assert chunked(lib, dv=32) == 2
    assert chunked(lib, dk=48, dv=48) == 3
    assert chunked(lib, dk=256, dv=256) == 3
    assert chunked(lib, chunk=8) == 3
    assert chunked(lib, chunk=128) == 3
    assert chunked(lib, dt=2) == 3
    assert chunked(lib, coef=4) == 3
    assert chunked(lib, coef=-1) == 3
    assert chunked(lib, q=FAKE + 8) == 4
    assert chunked(lib, o=FAKE + 4) == 4
    assert chunked(lib, s0=FAKE + 4) == 4
    assert chunked(lib, sf=FAKE + 12) == 4
    assert chunked(lib, beta=FAKE + 1) == 4          # bf16 beta must be 2-byte aligned
    assert chunked(lib, beta=FAKE + 2, dt=0) == 4    # fp32 beta must be 4-byte aligned


def test_step_rejects_bad_arguments_before_launch():
    lib = efla.load_library()
    assert step(lib, state=None) == 1
    assert step(lib, q=None) == 1
    assert step(lib, B=0) == 2
    assert step(lib, dv=16) == 2
    assert step(lib, dk=96, dv=96) == 3
    assert step(lib, dt=7) == 3
    assert step(lib, coef=4) == 3
    assert step(lib, state=FAKE + 8) == 4
    assert step(lib, k=FAKE + 2) == 4


def test_workspace_query():
    lib = efla.load_library()
    # one pass fills the GPU (or the sequence is short): no workspace
    for d in efla.SUPPORTED_HEAD_DIMS:
        for c in efla.SUPPORTED_CHUNKS:
            assert lib.efla_fwd_chunked_workspace_bytes(2, 4, 1000, d, d, c, 1) == 0
    assert lib.efla_fwd_chunked_workspace_bytes(8, 16, 4096, 128, 128, 64, 1) == 0    # 256 workgroups
    assert lib.efla_fwd_chunked_workspace_bytes(16, 8, 2048, 128, 128, 64, 1) == 0
    # few heads, long sequence: time segments. 16 heads x 2 column slices = 32
    # workgroups -> 9 segments of 114 chunks (both big launches hold
    # 32 x 8 = 256 workgroups); per head the maps (P, R) of segments
    # 1 .. nseg - 2 plus a start state slot per segment
    nseg = 9
    assert lib.efla_fwd_chunked_workspace_bytes(1, 16, 65536, 128, 128, 64, 1) == \
        16 * (2 * (nseg - 2) + nseg) * 128 * 128 * 4
    # 2 heads x 2 slices = 4 workgroups: up to 65 segments fill the GPU, but
    # segments are at least 8 chunks long, so 65 chunks give 8 segments of 9
    # chunks (the last one 2); maps of segments 1 .. 6 and 8 start states
    nseg = 8
    assert lib.efla_fwd_chunked_workspace_bytes(1, 2, 4133, 128, 128, 64, 1) == \
        2 * (2 * (nseg - 2) + nseg) * 128 * 128 * 4
    # 64 chunks, the shortest sequence that takes segments: 8 of 8 chunks
    assert lib.efla_fwd_chunked_workspace_bytes(1, 2, 4096, 128, 128, 64, 1) == \
        2 * (2 * (nseg - 2) + nseg) * 128 * 128 * 4
    assert lib.efla_fwd_chunked_workspace_bytes(1, 2, 4032, 128, 128, 64, 1) == 0  # 63 chunks
    # fp32 with chunk 64 runs (and plans its segments) with chunk 16 when one
    # pass would leave the GPU idle (< 128 workgroups), else with chunk 32
    for d in (16, 64, 128):
        for T in (1000, 8229, 65536):
            assert lib.efla_fwd_chunked_workspace_bytes(1, 2, T, d, d, 64, 0) == \
                lib.efla_fwd_chunked_workspace_bytes(1, 2, T, d, d, 16, 0)
    assert lib.efla_fwd_chunked_workspace_bytes(1, 2, 8229, 128, 128, 16, 0) > 0
    assert lib.efla_fwd_chunked_workspace_bytes(8, 16, 9000, 128, 128, 64, 0) == \
        lib.efla_fwd_chunked_workspace_bytes(8, 16, 9000, 128, 128, 32, 0) == 0
    # unsupported or invalid sizes report 0
    assert lib.efla_fwd_chunked_workspace_bytes(1, 16, 65536, 128, 128, 48, 1) == 0
    assert lib.efla_fwd_chunked_workspace_bytes(0, 16, 65536, 128, 128, 64, 1) == 0


def test_segmented_call_checks_its_workspace_before_launch():
    lib = efla.load_library()
    need = lib.efla_fwd_chunked_workspace_bytes(1, 16, 65536, 128, 128, 64, 1)
    assert need > 0
    kw = dict(B=1, H=16, T=65536, dk=128, dv=128, chunk=64, dt=1)
    assert chunked(lib, ws=None, wsb=0, **kw) == 5
    assert chunked(lib, ws=FAKE, wsb=need - 1, **kw) == 5
    assert chunked(lib, ws=FAKE + 8, wsb=need, **kw) == 4  # workspace must be 16-byte aligned


def test_coefficient_names_match_the_header():
    text = open(os.path.join(ROOT, "include", "efla.h")).read()
    for name, value in efla.COEFS.items():
        assert f"EFLA_COEF_{name.upper()} = {value}" in text
    with pytest.raises(ValueError):
        efla._coef("heun")



def bwd(lib, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, s0=None, dout=FAKE, dsT=None, dq=FAKE, dk=FAKE,
        dv=FAKE, db=FAKE, ds0=None, ws=FAKE, wsb=1 << 40, B=1, H=1, T=8, dk_=64, dv_=64, chunk=64,
        coef=0, dt=1):
    return lib.efla_bwd_chunked(q, k, v, beta, s0, dout, dsT, dq, dk, dv, db, ds0, ws, wsb, B, H, T,
                                dk_, dv_, chunk, coef, dt, None)


def test_backward_rejects_bad_arguments_before_launch():
    lib = efla.load_library()
    assert bwd(lib, dout=None) == 1
    assert bwd(lib, db=None) == 1
    assert bwd(lib, B=0) == 2
    assert bwd(lib, dv_=32) == 2
    assert bwd(lib, chunk=48) == 3
    assert bwd(lib, coef=5) == 3
    assert bwd(lib, dq=FAKE + 4) == 4
    assert bwd(lib, db=FAKE + 1) == 4
    assert bwd(lib, ws=None) == 5
    assert bwd(lib, wsb=16) == 5


def test_backward_workspace_query():
    lib = efla.load_library()
    # bf16, d = 128, C = 64: per head 3 nc d^2 + Tp d + 3 Tp + 4 nc C^2 floats
    nc, Tp = 2, 128
    per = 3 * nc * 128 * 128 + Tp * 128 + 3 * Tp + 4 * nc * 64 * 64
    assert lib.efla_bwd_chunked_workspace_bytes(1, 3, 100, 128, 128, 64, 1) == 3 * per * 4
    # fp32 with C = 64 runs the backward with chunk 32
    nc, Tp = 4, 128
    per = 3 * nc * 64 * 64 + Tp * 64 + 3 * Tp + 4 * nc * 32 * 32
    assert lib.efla_bwd_chunked_workspace_bytes(1, 1, 100, 64, 64, 64, 0) == per * 4
    # fp32, d = 128, C = 64 runs with chunk 32 as well
    per = 3 * nc * 128 * 128 + Tp * 128 + 3 * Tp + 4 * nc * 32 * 32
    assert lib.efla_bwd_chunked_workspace_bytes(1, 1, 100, 128, 128, 64, 0) == per * 4
    assert lib.efla_bwd_chunked_workspace_bytes(1, 1, 100, 48, 48, 64, 1) == 0


def train(lib, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, s0=None, o=FAKE, sf=None, ws=FAKE, wsb=1 << 40,
          B=1, H=1, T=8, dk=64, dv=64, chunk=64, coef=0, dt=1):
    return lib.efla_fwd_chunked_train(q, k, v, beta, s0, o, sf, ws, wsb, B, H, T, dk, dv, chunk, coef, dt,
                                      None)


def saved(lib, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dout=FAKE, dsT=None, dq=FAKE, dk=FAKE, dv=FAKE,
          db=FAKE, ds0=None, ws=FAKE, wsb=1 << 40, B=1, H=1, T=8, dk_=64, dv_=64, chunk=64, coef=0, dt=1):
    return lib.efla_bwd_chunked_saved(q, k, v, beta, dout, dsT, dq, dk, dv, db, ds0, ws, wsb, B, H, T, dk_,
                                      dv_, chunk, coef, dt, None)


def test_train_forward_rejects_bad_arguments_before_launch():
    lib = efla.load_library()
    assert train(lib, q=None) == 1
    assert train(lib, o=None) == 1
    assert train(lib, B=0) == 2
    assert train(lib, dv=32) == 2
    assert train(lib, chunk=8) == 3
    assert train(lib, coef=7) == 3
    assert train(lib, q=FAKE + 8) == 4
    assert train(lib, ws=FAKE + 8) == 4
    assert train(lib, ws=None) == 5          # the backward's workspace is required
    need = lib.efla_bwd_chunked_workspace_bytes(1, 1, 8, 64, 64, 64, 1)
    assert need > 0
    assert train(lib, wsb=need - 1) == 5


def test_saved_backward_rejects_bad_arguments_before_launch():
    lib = efla.load_library()
    assert saved(lib, dout=None) == 1
    assert saved(lib, dq=None) == 1
    assert saved(lib, B=0) == 2
    assert saved(lib, chunk=48) == 3
    assert saved(lib, db=FAKE + 1) == 4
    assert saved(lib, ws=None) == 5
    assert saved(lib, wsb=16) == 5


def test_binding_rejects_undersized_outputs_before_launch():
    """The C ABI takes bare pointers and cannot see buffer sizes, so the
    binding checks caller-provided outputs against the exact shapes the
    kernels write (CPU tensors here: the check raises before any call into
    the library)."""
    import torch

    B, H, T, d = 1, 2, 40, 64
    q = torch.zeros(B, H, T, d, dtype=torch.bfloat16)
    beta = torch.zeros(B, H, T, dtype=torch.bfloat16)
    small_o = torch.zeros(B, H, T - 1, d, dtype=torch.bfloat16)
    small_s = torch.zeros(B, H, d, d - 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="o has shape"):
        efla.efla_fwd_chunked(q, q, q, beta, None, o=small_o)
    with pytest.raises(ValueError, match="s_final has shape"):
        efla.efla_fwd_chunked(q, q, q, beta, None, s_final=small_s)
    with pytest.raises(ValueError, match="o has shape"):
        efla.efla_fwd_chunked_train(q, q, q, beta, None, o=small_o)
    with pytest.raises(ValueError, match="s_final has shape"):
        efla.efla_fwd_chunked_train(q, q, q, beta, None, s_final=small_s)
    state = torch.zeros(B, H, d, d, dtype=torch.float32)
    with pytest.raises(ValueError, match="o has shape"):
        q1, b1 = q[:, :, 0].contiguous(), beta[:, :, 0].contiguous()
        efla.efla_fwd_recurrent_step(q1, q1, q1, b1, state,
                                     o=torch.zeros(B, H, d // 2, dtype=torch.bfloat16))


_NO_GPU_CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import delta_rule_recurrent_efla_amd as efla
lib = efla.load_library()
F = 0x100000
print(lib.efla_fwd_chunked(F, F, F, F, None, F, None, None, 0, 1, 1, 8, 64, 64, 64, 0, 1, None),
      lib.efla_fwd_recurrent_step(F, F, F, F, F, F, 1, 1, 64, 64, 0, 1, None))
"""


def test_well_formed_call_without_a_gpu_returns_hip_error():
    """On a host with no usable GPU a call that passes validation reaches the
    launch, which fails: the library reports EFLA_ERR_HIP (6) and does not
    crash. Runs in a child process with the GPUs hidden from HIP; skipped where
    a GPU is visible, so no kernel is ever launched on the stand-in pointers."""
    import subprocess
    import sys

    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", _NO_GPU_CHILD, ROOT], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[-2:] == ["6", "6"], r.stdout

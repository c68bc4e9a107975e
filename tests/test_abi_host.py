"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/kda.h, and rejects bad arguments on the host before
anything is enqueued (fake non-NULL pointers are never dereferenced there)."""
import ctypes
import os
import re

import pytest

import channel_gated_delta_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

P = ctypes.c_void_p(4096)   # stand-in device pointer: only compared, never dereferenced
NULL = None
BF16, F32 = 1, 0


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from channel_gated_delta_amd import build
        build.build(verbose=False)
    return kda.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"kda_short_conv", "kda_chunk_fwd", "kda_chunk_fwd_gated",
                          "kda_chunk_fwd_workspace_size", "kda_decode_step",
                          "kda_output_norm_gate", "kda_decode_step_conv", "kda_gdn_chunk_fwd",
                          "kda_gdn_decode_step", "kda_status_string", "kda_last_error",
                          "kda_version", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_phases"}
    for name in names:
        assert hasattr(lib, name), name


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_status_strings_and_version(lib):
    for st in range(5):
        assert lib.kda_status_string(st) != b"unknown status"
    assert lib.kda_status_string(99) == b"unknown status"
    assert lib.kda_version() >= 10000


def chunk(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=NULL, N=1, T=64, H=2, dk=128, dv=128, chunk=64,
             scale=0.1, lb=-5.0, h0=NULL, hT=NULL, o=ctypes.c_void_p(8192),
             ws=ctypes.c_void_p(1 << 20), wsb=1 << 30, dtype=BF16, odt=F32)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["T"],
                             a["H"], a["dk"], a["dv"], a["chunk"], a["scale"], a["lb"], a["h0"],
                             a["hT"], a["o"], a["ws"], a["wsb"], a["dtype"], a["odt"], NULL)


def phased(lib, phases, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=NULL, N=1, T=64, H=2, dk=128, dv=128, chunk=64,
             scale=0.1, lb=-5.0, h0=NULL, hT=NULL, o=ctypes.c_void_p(8192),
             ws=ctypes.c_void_p(1 << 20), wsb=1 << 30, dtype=BF16, odt=F32)
    a.update(kw)
    return lib.kda_chunk_fwd_phases(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"],
                                    a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["scale"],
                                    a["lb"], a["h0"], a["hT"], a["o"], a["ws"], a["wsb"],
                                    a["dtype"], a["odt"], phases, NULL)


@pytest.mark.parametrize("phases", [0, 4, -1, 7])
def test_chunk_fwd_phases_rejects_unknown_phases(lib, phases):
    assert phased(lib, phases) == kda.KDA_ERR_INVALID_ARG
    assert b"phases" in lib.kda_last_error()


@pytest.mark.parametrize("phases", [kda.PHASE_PREP, kda.PHASE_WALK, kda.PHASE_ALL])
@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(o=P), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(ws=NULL), kda.KDA_ERR_WORKSPACE),
    (dict(wsb=2 * 64 * 2 * 16 * 4 + 4096 - 1), kda.KDA_ERR_WORKSPACE),
])
def test_chunk_fwd_phases_checks_every_argument(lib, phases, kw, status):
    """Each part runs the full argument checks of kda_chunk_fwd (host only)."""
    assert phased(lib, phases, **kw) == status
    assert lib.kda_last_error()


def ws_size(lib, T=64, H=2, dk=128, dv=128, chunk=64, dtype=BF16, odt=F32):
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(T, H, dk, dv, chunk, dtype, odt, ctypes.byref(n))
    return st, n.value


def test_workspace_size(lib):
    # two fp32 rows of the internal 16-token chunk per token and head, and 4 KiB of
    # dispatch order for packed batches
    assert ws_size(lib) == (kda.KDA_OK, 2 * 64 * 2 * 16 * 4 + 4096)
    assert ws_size(lib, chunk=16) == (kda.KDA_OK, 2 * 64 * 2 * 16 * 4 + 4096)
    assert ws_size(lib, T=0) == (kda.KDA_OK, 0)
    assert ws_size(lib, dtype=F32, dk=16, dv=16, chunk=32) == \
        (kda.KDA_OK, 2 * 64 * 2 * 16 * 4 + 4096)
    assert ws_size(lib, dk=48)[0] == kda.KDA_ERR_UNSUPPORTED
    assert ws_size(lib, chunk=8)[0] == kda.KDA_ERR_UNSUPPORTED
    assert ws_size(lib, dtype=F32, odt=BF16)[0] == kda.KDA_ERR_UNSUPPORTED
    assert ws_size(lib, H=0)[0] == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_chunk_fwd_workspace_size(64, 2, 128, 128, 64, BF16, F32, None) == \
        kda.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(o=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(N=0), kda.KDA_ERR_INVALID_ARG),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG),            # cu_seqlens NULL with two sequences
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(dtype=7), kda.KDA_ERR_INVALID_ARG),
    (dict(odt=5), kda.KDA_ERR_INVALID_ARG),
    (dict(dtype=F32, odt=BF16), kda.KDA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID_ARG),
    (dict(o=P), kda.KDA_ERR_INVALID_ARG),            # o aliases q
    (dict(lb=0.5), kda.KDA_ERR_INVALID_ARG),
    (dict(lb=float("nan")), kda.KDA_ERR_INVALID_ARG),
    (dict(lb=-9.5), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=128), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=8), kda.KDA_ERR_UNSUPPORTED),
    (dict(ws=NULL), kda.KDA_ERR_WORKSPACE),
    (dict(wsb=2 * 64 * 2 * 16 * 4 + 4096 - 1), kda.KDA_ERR_WORKSPACE),   # one byte short
    (dict(o=ctypes.c_void_p(1 << 20)), kda.KDA_ERR_INVALID_ARG),     # o aliases the workspace
])
def test_chunk_fwd_rejects(lib, kw, status):
    assert chunk(lib, **kw) == status
    assert lib.kda_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(g=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(o=P), kda.KDA_ERR_INVALID_ARG),
    (dict(lb=-9.5), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(wsb=2 * 64 * 2 * 16 * 4 + 4096 - 1), kda.KDA_ERR_WORKSPACE),
])
def test_gdn_calls_reject(lib, kw, status):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=NULL, N=1, T=64, H=2, dk=128, dv=128, chunk=64,
             scale=0.1, lb=-5.0, h0=NULL, hT=NULL, o=ctypes.c_void_p(8192),
             ws=ctypes.c_void_p(1 << 20), wsb=1 << 30, dtype=BF16, odt=F32)
    a.update(kw)
    assert lib.kda_gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"],
                                 a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["scale"],
                                 a["lb"], a["h0"], a["hT"], a["o"], a["ws"], a["wsb"],
                                 a["dtype"], a["odt"], NULL) == status
    assert b"kda_gdn_chunk_fwd" in lib.kda_last_error()
    st = lib.kda_gdn_decode_step(P, P, P, a["g"], P, ctypes.c_void_p(12288), 4, 2, a["dk"], 128,
                                 0.1, a["o"], BF16, F32, NULL)
    if "g" in kw or "o" in kw or "dk" in kw:
        assert st == status and b"kda_gdn_decode_step" in lib.kda_last_error()


def chunk_gated(lib, **kw):
    a = dict(q=P, k=P, v=P, z=ctypes.c_void_p(4096 * 3), al=NULL, dt=NULL, lb=-5.0, beta=P,
             cu=NULL, N=1, T=64, H=2, dk=128, dv=128, chunk=64, scale=0.1, h0=NULL, hT=NULL,
             o=ctypes.c_void_p(8192), ws=ctypes.c_void_p(1 << 20), wsb=1 << 30, dtype=BF16,
             odt=F32)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["z"], a["al"], a["dt"], a["lb"],
                                   a["beta"], a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                   a["chunk"], a["scale"], a["h0"], a["hT"], a["o"], a["ws"],
                                   a["wsb"], a["dtype"], a["odt"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(z=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(beta=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(o=ctypes.c_void_p(4096 * 3)), kda.KDA_ERR_INVALID_ARG),   # o aliases z
    (dict(al=ctypes.c_void_p(8192)), kda.KDA_ERR_INVALID_ARG),      # o aliases a_log
    (dict(dt=ctypes.c_void_p(8192)), kda.KDA_ERR_INVALID_ARG),      # o aliases dt_bias
    (dict(lb=0.5), kda.KDA_ERR_INVALID_ARG),
    (dict(lb=float("nan")), kda.KDA_ERR_INVALID_ARG),
    (dict(lb=-9.5), kda.KDA_ERR_UNSUPPORTED),
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=F32, odt=BF16), kda.KDA_ERR_UNSUPPORTED),
    (dict(wsb=2 * 64 * 2 * 16 * 4 + 4096 - 1), kda.KDA_ERR_WORKSPACE),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG),
])
def test_chunk_fwd_gated_rejects(lib, kw, status):
    assert chunk_gated(lib, **kw) == status
    assert b"kda_chunk_fwd_gated" in lib.kda_last_error()


def conv(lib, **kw):
    a = dict(x=P, w=P, b=NULL, cu=NULL, N=1, T=16, H=2, D=128, W=4, sin=NULL, sout=NULL, silu=1,
             l2=1, eps=1e-6, dtype=BF16, y=ctypes.c_void_p(8192))
    a.update(kw)
    return lib.kda_short_conv(a["x"], a["w"], a["b"], a["cu"], a["N"], a["T"], a["H"], a["D"],
                              a["W"], a["sin"], a["sout"], a["silu"], a["l2"], a["eps"],
                              a["dtype"], a["y"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(x=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(y=P), kda.KDA_ERR_INVALID_ARG),            # y aliases x
    (dict(N=3), kda.KDA_ERR_INVALID_ARG),
    (dict(T=-5), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG),
    (dict(W=5), kda.KDA_ERR_UNSUPPORTED),
    (dict(W=0), kda.KDA_ERR_UNSUPPORTED),
    (dict(D=6), kda.KDA_ERR_UNSUPPORTED),            # not a multiple of 4 channels
    (dict(D=12), kda.KDA_ERR_UNSUPPORTED),           # 3 lanes per head: not a power of two
    (dict(D=24), kda.KDA_ERR_UNSUPPORTED),           # 6 lanes per head: not a power of two
    (dict(D=512), kda.KDA_ERR_UNSUPPORTED),          # 128 lanes per head
])
def test_short_conv_rejects(lib, kw, status):
    assert conv(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(state=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(B=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(o=P), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=8), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=F32, odt=BF16), kda.KDA_ERR_UNSUPPORTED),
])
def test_decode_step_rejects(lib, kw, status):
    a = dict(state=ctypes.c_void_p(12288), B=4, H=2, dk=128, dv=128, o=ctypes.c_void_p(8192),
             dtype=BF16, odt=F32)
    a.update(kw)
    assert lib.kda_decode_step(P, P, P, P, P, a["state"], a["B"], a["H"], a["dk"], a["dv"], 0.1,
                               a["o"], a["dtype"], a["odt"], NULL) == status


@pytest.mark.parametrize("kw,status", [
    (dict(o=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(gate=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(y=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(rows=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG),
    (dict(eps=float("inf")), kda.KDA_ERR_INVALID_ARG),
    (dict(odt=7), kda.KDA_ERR_INVALID_ARG),
    (dict(y=P), kda.KDA_ERR_INVALID_ARG),                      # fp32 o, bf16 y in the same place
    (dict(w=ctypes.c_void_p(8192)), kda.KDA_ERR_INVALID_ARG),  # y aliases the weight
    (dict(dv=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(odt=BF16, dt=F32), kda.KDA_ERR_UNSUPPORTED),
])
def test_output_norm_gate_rejects(lib, kw, status):
    a = dict(o=P, gate=ctypes.c_void_p(4096 * 3), w=NULL, eps=1e-6, rows=64, dv=128, odt=F32,
             dt=BF16, y=ctypes.c_void_p(8192))
    a.update(kw)
    assert lib.kda_output_norm_gate(a["o"], a["gate"], a["w"], a["eps"], a["rows"], a["dv"],
                                    a["odt"], a["dt"], a["y"], NULL) == status
    assert b"kda_output_norm_gate" in lib.kda_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(xq=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(cq=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(cv=ctypes.c_void_p(4096 * 20)), kda.KDA_ERR_INVALID_ARG),   # conv_v is conv_q
    (dict(o=ctypes.c_void_p(4096 * 20)), kda.KDA_ERR_INVALID_ARG),    # o aliases conv_q
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG),
    (dict(B=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=8), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=F32, odt=BF16), kda.KDA_ERR_UNSUPPORTED),
])
def test_decode_step_conv_rejects(lib, kw, status):
    a = dict(xq=P, cq=ctypes.c_void_p(4096 * 20), cv=ctypes.c_void_p(4096 * 22), eps=1e-6, B=4,
             dk=128, o=ctypes.c_void_p(8192), dtype=BF16, odt=F32)
    a.update(kw)
    assert lib.kda_decode_step_conv(
        a["xq"], P, P, P, P, P, a["cq"], ctypes.c_void_p(4096 * 21), a["cv"], a["eps"], P, P,
        ctypes.c_void_p(12288), a["B"], 2, a["dk"], 128, 0.1, a["o"], a["dtype"], a["odt"],
        NULL) == status
    assert b"kda_decode_step_conv" in lib.kda_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 2, 16)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, x, x[..., 0])


def noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=NULL, N=1, T=64, H=2, dk=128, dv=128, chunk=64,
             scale=0.1, lb=-5.0, h0=NULL, hT=NULL, o=ctypes.c_void_p(8192), dtype=BF16, odt=F32)
    a.update(kw)
    return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"],
                                     a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["scale"],
                                     a["lb"], a["h0"], a["hT"], a["o"], a["dtype"], a["odt"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), kda.KDA_ERR_INVALID_ARG),
    (dict(o=P), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=48), kda.KDA_ERR_UNSUPPORTED),
    (dict(lb=-9.5), kda.KDA_ERR_UNSUPPORTED),
    # the static scratch holds 64 MiB: 524288 token-heads of Tb and P rows
    (dict(T=5462, H=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(T=524289, H=1), kda.KDA_ERR_UNSUPPORTED),
])
def test_noalloc_rejects_before_any_device_call(lib, kw, status):
    """Argument and size checks run on the host before the scratch lookup (no GPU here)."""
    assert noalloc(lib, **kw) == status
    assert lib.kda_last_error()
    if status == kda.KDA_ERR_UNSUPPORTED and "T" in kw:
        assert b"scratch" in lib.kda_last_error()

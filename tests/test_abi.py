"""The C ABI without a GPU: the library loads, exports every declared entry
point, reports sizes, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import exact_attention_fwd_amd as fa
from exact_attention_fwd_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first, or there is no device

OK, NULL, SHAPE, UNSUP, WS, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.library_path()):
        pytest.fail("libfa.so is not built (run python -m exact_attention_fwd_amd.build)")
    return fa.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"fa_forward", "fa_backward", "fa_decode_paged"} <= set(names)
    for name in names:
        assert hasattr(L, name), f"{name} declared in fa.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(names) <= exported


def test_library_carries_gfx950_code_objects(L):
    # the offload bundle id of the embedded device code names the target
    blob = open(_lib.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings_and_version(L):
    for code in range(7):
        s = L.fa_status_str(code).decode()
        assert s.startswith(_lib.status_name(code))
    assert L.fa_version() >= 10000
    assert L.fa_last_hip_error() is not None


def test_workspace_sizes(L):
    assert L.fa_backward_workspace_bytes(2, 16, 8192, 128) == 2 * (2 * 16 * 8192 * 4)
    assert L.fa_backward_workspace_bytes(1, 1, 7, 64) == 2 * 256
    assert L.fa_backward_workspace_bytes(0, 1, 7, 64) == 0
    assert L.fa_decode_workspace_bytes(8, 32, 128, 32) == 8 * 32 * 32 * 2 * 130 * 4
    # linear in N: no N x N buffer anywhere
    assert L.fa_backward_workspace_bytes(1, 1, 32768, 128) == 2 * 32768 * 4


def fwd(L, dt=1, B=1, H=1, N=16, d=128, ptr=FAKE, lse=FAKE, causal=0, scale=0.1):
    return L.fa_forward(dt, B, H, N, d, ptr, ptr, ptr, ptr, lse, causal, scale, None)


def test_forward_validation(L):
    assert fwd(L, dt=7) == UNSUP
    assert fwd(L, B=0) == SHAPE
    assert fwd(L, H=-1) == SHAPE
    assert fwd(L, N=-5) == SHAPE
    assert fwd(L, d=96) == UNSUP
    assert fwd(L, d=0) == SHAPE
    assert fwd(L, scale=float("inf")) == SHAPE
    assert fwd(L, scale=float("nan")) == SHAPE
    assert fwd(L, ptr=None) == NULL
    assert fwd(L, N=0, ptr=None) == OK  # empty problem: nothing to do, nothing read
    assert fwd(L, B=1 << 20, H=1 << 20) == SHAPE


def test_backward_validation(L):
    def bwd(dt=1, N=16, d=128, ws=FAKE, wsb=1 << 20, ptr=FAKE):
        return L.fa_backward(dt, 1, 2, N, d, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ws, wsb, 1, 0.1, None)
    assert bwd(dt=0) == UNSUP
    assert bwd(d=80) == UNSUP
    assert bwd(N=-1) == SHAPE
    assert bwd(ptr=None) == NULL
    assert bwd(ws=None) == WS
    assert bwd(wsb=16) == WS
    assert bwd(N=0, ptr=None, ws=None) == OK


def test_decode_validation(L):
    def dec(S=2, H=4, d=128, page=256, P=4, mb=2, ws=FAKE, wsb=1 << 20, ptr=FAKE):
        return L.fa_decode_paged(S, H, d, page, P, mb, ptr, ptr, ptr, ptr, ptr, ptr, 0.1, ws, wsb, None)
    assert dec(page=128) == UNSUP
    assert dec(d=32) == UNSUP
    assert dec(S=0) == SHAPE
    assert dec(P=0) == SHAPE
    assert dec(mb=0) == SHAPE
    assert dec(ptr=None) == NULL
    assert dec(ws=None) == WS
    assert dec(wsb=100) == WS


def test_static_decode_validation(L):
    """The allocation-free decode validates like fa_decode_paged_gqa and refuses
    a problem whose partials exceed its static scratch, before any launch."""
    assert L.fa_decode_static_scratch_bytes() == 16 << 20

    def dec(S=2, H=8, Hkv=2, d=128, page=256, P=4, mb=2, ptr=FAKE):
        return L.fa_decode_paged_gqa_static(S, H, Hkv, d, page, P, mb, ptr, ptr, ptr, ptr, ptr, ptr, 0.1, None)
    assert dec(page=128) == UNSUP
    assert dec(d=32) == UNSUP
    assert dec(S=0) == SHAPE
    assert dec(Hkv=3) == SHAPE
    assert dec(ptr=None) == NULL
    # partials: S·H·2·mb·(d+2)·4 bytes; 8 x 32 x 2 x 64 x 130 x 4 = 17 MB > 16 MiB
    assert L.fa_decode_workspace_bytes(8, 32, 128, 64) > 16 << 20
    assert dec(S=8, H=32, Hkv=8, mb=64) == SCRATCH
    assert L.fa_decode_workspace_bytes(8, 32, 128, 63) <= 16 << 20
    if not torch.cuda.is_available():  # fits: reaches the device check (never launched with fake pointers)
        assert dec(S=8, H=32, Hkv=8, mb=63) == HIP
    assert L.fa_status_str(SCRATCH).decode().startswith("FA_ERR_SCRATCH_TOO_SMALL")


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_hip_error(L):
    assert fwd(L) == HIP
    assert L.fa_last_hip_error().decode() != "no error"
    with pytest.raises(fa.FaError):
        raise fa.FaError(HIP)


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)


def test_build_refuses_kernels_that_spill():
    from exact_attention_fwd_amd import build as b
    sample = "\n".join([
        "x.hip:10:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:10:1: remark:     VGPRs: 100 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:1: remark: Function Name: k_spill [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:1: remark:     VGPRs Spill: 53 [-Rpass-analysis=kernel-resource-usage]",
    ])
    res = b.kernel_resources(sample)
    assert res["k_ok"]["VGPRs"] == "100" and res["k_spill"]["VGPRs Spill"] == "53"
    with pytest.raises(RuntimeError, match="k_spill"):
        b._check_resources("x.hip", sample)
    b._check_resources("x.hip", "\n".join(sample.splitlines()[:3]))

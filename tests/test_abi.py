"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/spa.h declares, sizes its workspaces, and rejects invalid arguments before any
GPU call (no kernel is launched in these tests)."""
import ctypes
import math
import os
import re

import pytest

import block_sparse_attention_pooled_amd as spa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spa.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SPA_API\s+[\w\s\*]+?\b(spa_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert header_symbols() == sorted(spa.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = spa.load_library()
    for name in header_symbols():
        assert hasattr(lib, name), name
    assert lib.spa_version() == 100


def test_status_strings():
    for code in range(-7, 1):
        assert spa.status_string(code) not in ("", "unknown status")
    assert spa.status_string(7) == "unknown status"


def _dims(B=1, H=2, N=1000, d=128, bq=128, bk=64):
    return spa._Dims(B, H, N, d, bq, bk)


def test_mask_workspace_size_formula():
    B, H, N, d = 1, 12, 32760, 128
    nqb, nkb = math.ceil(N / 128), math.ceil(N / 64)
    want = B * H * nqb * d * 8 + B * H * d * nkb * 8
    got = spa.mask_workspace_bytes((B, H, N, d), 128, 64)
    assert want <= got <= want + 512


def test_bwd_workspace_size_formula():
    B, H, N, d = 1, 12, 32760, 128
    nqb, nkb = 256, 512
    npad = nqb * 128  # per-row side values (D, lse2) padded to whole query blocks
    want = 2 * B * H * npad * 4 + B * H * (nkb // 32) * nqb * 4 + B * H * nkb * nqb * 4 \
        + B * H * nkb * 4 \
        + B * H * N * d * 2 + B * H * nkb * 4 \
        + B * H * nkb * 4 \
        + 10 * 4  # fp16 copy of dO, dO flag per key block, dK/dV dispatch order and work queues
    got = spa.bwd_workspace_bytes((B, H, N, d), 128, 64)
    assert want <= got <= want + 1024


def test_fwd_workspace_size_formula():
    B, H, N, d = 2, 3, 1000, 128
    nkb = -(-N // 64)
    al = lambda x: -(-x // 256) * 256
    want = al(B * H * N * d * 2) + al(B * H * nkb * 4)  # fp16 copy of V, flag per key block
    assert spa.fwd_workspace_bytes((B, H, N, d), 128, 64) == want


@pytest.mark.parametrize("dims,code", [
    (dict(B=0), -2), (dict(N=0), -2), (dict(d=96), -4), (dict(bq=32), -4), (dict(bk=128), -4),
    (dict(N=64 * 2049), -4), (dict(B=1, H=64, N=300000, d=128), -2),
])
def test_bad_dims_rejected(dims, code):
    lib = spa.load_library()
    d = _dims(**dims)
    assert lib.spa_mask_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.spa_bwd_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.spa_fwd_workspace_bytes(ctypes.byref(d)) == 0
    rc = lib.spa_build_mask(ctypes.byref(d), FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE, None,
                            FAKE, 1 << 40, None)
    assert rc == code
    rc = lib.spa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, None,
                                 FAKE, None, 0, None)
    assert rc == code


def test_null_pointers_rejected():
    lib = spa.load_library()
    d = _dims()
    assert lib.spa_build_mask(None, FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE, None, FAKE, 1 << 40,
                              None) == -1
    assert lib.spa_build_mask(ctypes.byref(d), None, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE, None, FAKE,
                              1 << 40, None) == -1
    assert lib.spa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, None,
                                   None, None, 0, None) == -1
    # the residual output needs the workspace
    assert lib.spa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE,
                                   FAKE, None, 1 << 40, None) == -1
    assert lib.spa_sparse_attn_bwd(ctypes.byref(d), *([FAKE] * 5), None, FAKE, FAKE, FAKE,
                                   0.0, FAKE, FAKE, None, 0, FAKE, 1 << 40, None) == -1


@pytest.mark.parametrize("k,p", [(-0.1, 0.9), (1.5, 0.9), (0.05, -1.0), (0.05, 1.01),
                                 (float("nan"), 0.9), (0.05, float("nan"))])
def test_bad_fractions_rejected(k, p):
    lib = spa.load_library()
    d = _dims()
    rc = lib.spa_build_mask(ctypes.byref(d), FAKE, FAKE, k, p, 0.0, FAKE, FAKE, None, FAKE,
                            1 << 40, None)
    assert rc == -3


def test_bad_scales_and_grad_dtype_rejected():
    lib = spa.load_library()
    d = _dims()
    assert lib.spa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, float("inf"),
                                   FAKE, None, FAKE, None, 0, None) == -3
    assert lib.spa_build_mask(ctypes.byref(d), FAKE, FAKE, 0.05, 0.9, float("nan"), FAKE, FAKE,
                              None, FAKE, 1 << 40, None) == -3
    assert lib.spa_sparse_attn_bwd(ctypes.byref(d), *([FAKE] * 9), 0.0, FAKE, FAKE, FAKE, 2, FAKE,
                                   1 << 40, None) == -3


@pytest.mark.parametrize("stages", [0, 4, 8, 0xFFFFFFFF])
def test_bad_stage_masks_rejected(stages):
    lib = spa.load_library()
    d = _dims()
    assert lib.spa_sparse_attn_fwd_stages(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE,
                                          None, FAKE, None, 0, stages, None) == -3
    assert lib.spa_build_mask_stages(ctypes.byref(d), FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE,
                                     None, FAKE, 1 << 40, stages, None) == -3
    if stages != 4:  # 4 is SPA_BWD_DKDV
        assert lib.spa_sparse_attn_bwd_stages(ctypes.byref(d), *([FAKE] * 9), 0.0, FAKE, FAKE,
                                              FAKE, 0, FAKE, 1 << 40, stages, None) == -3


def test_small_workspace_rejected():
    lib = spa.load_library()
    d = _dims()
    need = lib.spa_mask_workspace_bytes(ctypes.byref(d))
    assert lib.spa_build_mask(ctypes.byref(d), FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE, None, FAKE,
                              need - 1, None) == -5
    need = lib.spa_bwd_workspace_bytes(ctypes.byref(d))
    assert lib.spa_sparse_attn_bwd(ctypes.byref(d), *([FAKE] * 9), 0.0, FAKE, FAKE, FAKE, 0, FAKE,
                                   need - 1, None) == -5
    need = lib.spa_fwd_workspace_bytes(ctypes.byref(d))
    assert lib.spa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE,
                                   FAKE, FAKE, need - 1, None) == -5


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        spa.build_mask(q, q, 64, 64)


def test_c_program_is_built_and_links():
    """build() also produces tests/c/abi_smoke, a plain-C user of the ABI; its shared-library
    dependencies (libspa.so through the run path, the HIP runtime) must resolve."""
    import subprocess
    binp = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_smoke")
    assert os.path.exists(binp), "run __graft_entry__.build() first"
    r = subprocess.run(["ldd", binp], capture_output=True, text=True, timeout=30)
    assert r.returncode == 0, r.stderr
    assert "not found" not in r.stdout, r.stdout
    assert "libspa.so" in r.stdout


def test_noalloc_mask_validates_before_any_device_call():
    """spa_build_mask_noalloc: the usual argument checks, and a problem whose mask workspace
    exceeds the fixed scratch returns SPA_E_SCRATCH, all before any HIP call."""
    lib = spa.load_library()
    d = _dims()
    assert lib.spa_build_mask_noalloc(None, FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE, None,
                                      None) == -1
    assert lib.spa_build_mask_noalloc(ctypes.byref(d), FAKE, None, 0.05, 0.9, 0.0, FAKE, FAKE,
                                      None, None) == -1
    assert lib.spa_build_mask_noalloc(ctypes.byref(d), FAKE, FAKE, 1.5, 0.9, 0.0, FAKE, FAKE,
                                      None, None) == -3
    assert lib.spa_build_mask_noalloc(ctypes.byref(_dims(d=96)), FAKE, FAKE, 0.05, 0.9, 0.0,
                                      FAKE, FAKE, None, None) == -4
    # a valid shape (B*H*N*d < 2^31) whose fp64 pooled means need 189 MB, beyond 96 MiB
    big = _dims(B=1, H=120, N=131072, d=64)
    need = lib.spa_mask_workspace_bytes(ctypes.byref(big))
    assert need > spa.NOALLOC_SCRATCH_BYTES
    assert lib.spa_build_mask_noalloc(ctypes.byref(big), FAKE, FAKE, 0.05, 0.9, 0.0, FAKE, FAKE,
                                      None, None) == -7
    assert "scratch" in spa.status_string(-7)

"""The C ABI from plain C: `tests/c/abi_smoke` (built by build(); no Python, no PyTorch)
runs mask, forward and backward on a seeded ragged problem (B=1, H=2, N=1000, d=64, blocks
64 x 64, k=10 %, p=0.9) and checks the documented error returns.  Its results must equal,
bit for bit, those of the Python binding on the same inputs (same library, deterministic
kernels), and its mask must match the oracle's.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from oracle import spa_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "abi_smoke")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _read(path):
    raw = open(path, "rb").read()
    B, H, N, d, bq, bk = np.frombuffer(raw[:24], dtype=np.int32)
    nqb, nkb = -(-N // bq), -(-N // bk)
    nel, nrow, nl = B * H * N * d, B * H * N, B * H * nqb
    out, off = {"dims": (int(B), int(H), int(N), int(d), int(bq), int(bk))}, 24
    for name, dt, count, shape in (
            ("q", np.uint16, nel, (B, H, N, d)), ("k", np.uint16, nel, (B, H, N, d)),
            ("v", np.uint16, nel, (B, H, N, d)), ("do", np.uint16, nel, (B, H, N, d)),
            ("kv_cnt", np.int32, nl, (B, H, nqb)), ("kv_idx", np.int32, nl * nkb, (B, H, nqb, nkb)),
            ("o", np.uint16, nel, (B, H, N, d)), ("o_lo", np.uint16, nel, (B, H, N, d)),
            ("lse", np.float32, nrow, (B, H, N)), ("dq", np.float32, nel, (B, H, N, d)),
            ("dk", np.float32, nel, (B, H, N, d)), ("dv", np.float32, nel, (B, H, N, d))):
        n = count * np.dtype(dt).itemsize
        out[name] = np.frombuffer(raw[off:off + n], dtype=dt).reshape(shape)
        off += n
    assert off == len(raw)
    return out


def test_c_program_matches_binding(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    if not os.path.exists(BIN):
        pytest.fail("tests/c/abi_smoke is missing: run __graft_entry__.build() first")
    path = str(tmp_path / "abi_smoke.bin")
    log(f"[c abi] running {BIN}")
    r = subprocess.run([BIN, path], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    c = _read(path)
    B, H, N, d, bq, bk = c["dims"]
    dev = {n: torch.from_numpy(c[n].view(np.int16).copy()).view(torch.bfloat16).cuda()
           for n in ("q", "k", "v", "do")}
    kv_idx, kv_cnt = spa.build_mask(dev["q"], dev["k"], bq, bk, 0.1, 0.9)
    o, lse, o_lo = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, bq, bk,
                                       with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, kv_idx,
                                     kv_cnt, bq, bk, o_lo=o_lo)
    torch.cuda.synchronize()
    cnt, idx = kv_cnt.cpu().numpy(), kv_idx.cpu().numpy()
    assert np.array_equal(cnt, c["kv_cnt"])
    for (b, h, i), n in np.ndenumerate(cnt):
        assert np.array_equal(idx[b, h, i, :n], c["kv_idx"][b, h, i, :n]), (b, h, i)
    for name, got in (("o", o), ("o_lo", o_lo)):
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), c[name]), name
    for name, got in (("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(got.cpu().numpy(), c[name]), name
    # the C program's mask against the oracle
    f = {n: O.widen_bf16(c[n]) for n in ("q", "k")}
    mask = O.build_mask(f["q"], f["k"], bq, bk, 0.1, 0.9)
    n, exempt, fails = parity.compare_mask_rows(c["kv_idx"], c["kv_cnt"], mask["rows"], 0.9)
    log(f"  mask: {n} rows, {len(exempt)} exempt; mean list length {c['kv_cnt'].mean():.1f}")
    assert not fails, fails[:5]
    assert c["kv_cnt"].mean() < 0.5 * (-(-N // bk))  # a real selection, not everything kept

"""spa_build_mask_noalloc, the mask entry point that allocates nothing (its pooled means
live in the library's fixed device scratch), through the C ABI: its lists, counts and rule
lengths must equal spa_build_mask's bit for bit on two calls in a row, the second on a
smaller problem (the scratch keeps the first call's contents), then the first problem
again.  The first call on the device sets up the scratch (the runtime places the array
when its address is first queried); the calls after it must leave the device's free memory
unchanged."""
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from block_sparse_attention_pooled_amd import synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    synth.Workload("noalloc_a", 2, 3, 1000, 128, 128, 64, 0.1, 0.9, kind="video",
                   grid=(2, 20, 25), alpha=synth.ALPHA_480P, n_sinks=2, seed=21),
    synth.Workload("noalloc_b", 1, 2, 700, 64, 64, 64, 0.05, 0.9, kind="video",
                   grid=(2, 14, 25), alpha=synth.ALPHA_480P, n_sinks=2, seed=22),
]


def _check_equal(torch, w, got, want):
    idx_g, cnt_g, rl_g = (t.cpu().numpy() for t in got)
    idx_w, cnt_w, rl_w = (t.cpu().numpy() for t in want)
    assert np.array_equal(cnt_g, cnt_w)
    assert np.array_equal(rl_g, rl_w)
    for (b, h, i), c in np.ndenumerate(cnt_w):  # the defined prefix of each list
        assert np.array_equal(idx_g[b, h, i, :c], idx_w[b, h, i, :c]), (w.name, b, h, i)


def test_noalloc_mask_equals_the_workspace_form():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    spa.load_library()
    inputs = []
    for w in CASES:
        g = synth.generate(w, with_do=False)
        q, k = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda()
                for n in ("q", "k"))
        B, H, N, d = w.shape()
        nqb, nkb = -(-N // w.blk_q), -(-N // w.blk_k)
        outs = [(torch.full((B, H, nqb, nkb), -1, dtype=torch.int32, device="cuda"),
                 torch.full((B, H, nqb), -1, dtype=torch.int32, device="cuda"),
                 torch.full((B, H, nqb, 2), -1, dtype=torch.int32, device="cuda"))
                for _ in range(2)]
        want = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p, rule_len=True)
        inputs.append((w, q, k, outs, want))
    torch.cuda.synchronize()
    free0 = None
    for call, x in enumerate([0, 1, 0]):
        w, q, k, outs, want = inputs[x]
        got = outs[call // 2]
        log(f"[noalloc] call {call}: {w.name} shape={w.shape()} blk=({w.blk_q},{w.blk_k})")
        spa.build_mask_noalloc(q, k, got[0], got[1], w.blk_q, w.blk_k, w.k_frac, w.p,
                               rule_len=got[2])
        torch.cuda.synchronize()
        _check_equal(torch, w, got, want)
        if free0 is None:  # after the set-up of the first call
            free0, _ = torch.cuda.mem_get_info()
    free1, _ = torch.cuda.mem_get_info()
    log(f"[noalloc] device free memory before {free0} after {free1}")
    assert free1 == free0

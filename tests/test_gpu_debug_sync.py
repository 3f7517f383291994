"""The library's debug mode: with PISA_SYNC_LAUNCHES=1 in the environment every launch waits for its
stream, so a kernel's asynchronous error is returned by the entry point that launched it.  A child
process with the variable set runs the pyramid, the selection, the attention (two passes and the
token-order kernels) and a decode step on the 4096-token workload; every call must succeed and give
the same bits as the same calls in this process, which runs without the variable.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gpu_harness as H
from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_calls() -> dict:
    """Pyramid, selection, attention and one decode step of the first sequence; host copies."""
    w = W.WORKLOADS["prefill_n4096"].with_(batch=1, top_k=8)           # decode holds G * 2K <= 256 on chip
    q, k, v = W.prefill_inputs(w, bits=True)
    qd, kd, vd = H.to_device(q, w), H.to_device(k, w), H.to_device(v, w)
    B, N, Hq, d = qd.shape
    n0 = N - 1                                              # decode appends the last token
    pyr = binding.build_pyramid(kd, n=n0, capacity=N)
    pyr_full = binding.build_pyramid(kd)
    sel = binding.select_blocks(qd, kd, pyr_full, w.top_k)
    o = binding.sparse_attn_fwd(qd, kd, vd, sel, out_dtype=torch.float32)
    kc, vc = kd.clone(), vd.clone()
    od = torch.empty((B, Hq, d), dtype=torch.float32, device=qd.device)
    sel_d = torch.empty((B, w.n_kv_heads, w.top_k), dtype=torch.int32, device=qd.device)
    binding.decode_step(qd[:, n0], kd[:, n0], vd[:, n0], kc, vc, pyr, n0, w.top_k, out=od, sel_out=sel_d)
    torch.cuda.synchronize()
    return {"sel": sel.cpu().numpy(), "o": o.cpu().numpy(), "pyr": pyr.cpu().numpy(),
            "decode_o": od.cpu().numpy(), "decode_sel": sel_d.cpu().numpy()}


def child(path: str) -> None:
    np.savez(path, **run_calls())


def test_sync_launches_give_the_same_bits(tmp_path):
    here = run_calls()
    out = str(tmp_path / "sync.npz")
    env = dict(os.environ, PISA_SYNC_LAUNCHES="1")
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]; "
            f"import test_gpu_debug_sync as m; m.child({out!r})")
    H.log("[debug sync] child process with PISA_SYNC_LAUNCHES=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    there = np.load(out)
    for name, want in here.items():
        assert np.array_equal(there[name], want, equal_nan=True), name

"""The allocation-free forward attention (fixed device array inside the library) against the
entry point that takes a caller workspace: two calls in a row, the second on a smaller input, each
compared bit for bit (same kernels, same order of sums) for float32 and bfloat16 outputs, with the
row LSE; plus the host-side refusal of a workload whose workspace exceeds the array."""
import numpy as np
import pytest
import torch

from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W

import gpu_harness as H

pytestmark = pytest.mark.gpu


def _case(n, batch, hq, hkv, d, K, seed):
    w = W.WORKLOADS["prefill_n4096"].with_(name="noalloc", seq_len=n, batch=batch, n_q_heads=hq, n_kv_heads=hkv,
                                           head_dim=d, top_k=K, seed=seed)
    q, k, v = W.prefill_inputs(w, bits=True)
    sel = np.stack([np.stack([W.random_selection(w, K, b, h) for h in range(hkv)]) for b in range(batch)])
    return w, H.to_device(q, w), H.to_device(k, w), H.to_device(v, w), torch.from_numpy(sel).to(H.DEV)


def test_noalloc_forward_matches_workspace_forward_twice():
    for n, batch, hq, hkv, d, K, seed in [(20000, 1, 16, 1, 128, 16, 61), (3000, 2, 8, 2, 64, 8, 62)]:
        H.log(f"[noalloc] N={n} B={batch} Hq={hq} Hkv={hkv} d={d} K={K}")
        w, q, k, v, sel = _case(n, batch, hq, hkv, d, K, seed)
        for out_dtype in (torch.float32, torch.bfloat16):
            ref, ref_lse = binding.sparse_attn_fwd(q, k, v, sel, return_lse=True, out_dtype=out_dtype)
            out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=H.DEV)
            lse = torch.full((batch, hq, n), float("nan"), dtype=torch.float32, device=H.DEV)
            binding.sparse_attn_fwd_noalloc(q, k, v, sel, out, lse)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (n, out_dtype)
            assert torch.equal(lse, ref_lse), (n, out_dtype)
    H.log("[noalloc] both calls bit-identical to the workspace entry point")


def test_noalloc_forward_refuses_a_workspace_beyond_the_array():
    w = W.WORKLOADS["prefill_n262144"]
    cfg = binding.make_cfg(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.top_k, torch.bfloat16)
    assert binding.attn_workspace_bytes(cfg) > binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, w.seq_len, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=H.DEV)
    k = torch.zeros((1, w.seq_len, 1, w.head_dim), dtype=torch.bfloat16, device=H.DEV)
    sel = torch.full((1, 1, w.seq_len, w.top_k), -1, dtype=torch.int32, device=H.DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=H.DEV)
    with pytest.raises(RuntimeError, match="workspace"):
        binding.sparse_attn_fwd_noalloc(q, k, k, sel, out)

"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/pisa.h declares, sizes pyramids and workspaces, and rejects invalid
arguments before launching anything (no kernel runs in these tests)."""
import ctypes

import pytest

from hierarchical_top_selection_amd import binding
from oracle import pisa as oracle


@pytest.fixture(scope="module")
def lib():
    return binding.lib()


def test_exports_every_declared_symbol(lib):
    declared = binding.header_symbols()
    assert len(declared) == 17
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.pisa_abi_version() == 7


def test_noalloc_forward_refuses_oversized_workloads_before_touching_the_device(lib):
    """The allocation-free forward attention checks its workspace need against the fixed array first:
    the 256K workload (168 MB of packed K/V and softmax state) exceeds 128 MiB."""
    cfg = _cfg(seq_len=262144)
    assert lib.pisa_attn_workspace_bytes(ctypes.byref(cfg)) > binding.NOALLOC_SCRATCH_BYTES
    good = binding.PisaTensor(4096, 0, 128, 128)
    assert lib.pisa_sparse_attn_fwd_noalloc(ctypes.byref(cfg), good, good, good, ctypes.c_void_p(4096), good, 0,
                                            None, None) == 3
    assert lib.pisa_sparse_attn_fwd_noalloc(ctypes.byref(_cfg(top_k=0)), good, good, good, ctypes.c_void_p(4096),
                                            good, 0, None, None) == 1


def test_stage_events_validation(lib):
    """The timing hook rejects a negative count and null handles; count 0 clears it."""
    assert lib.pisa_stage_events(None, -1) == 1
    assert lib.pisa_stage_events(None, 2) == 1
    arr = (ctypes.c_void_p * 2)(16, None)
    assert lib.pisa_stage_events(ctypes.cast(arr, ctypes.c_void_p), 2) == 1
    assert lib.pisa_stage_events(None, 0) == 0


def test_status_strings(lib):
    assert lib.pisa_status_string(0).decode() == "ok"
    assert "unsupported" in lib.pisa_status_string(2).decode()
    assert lib.pisa_status_string(99).decode() == "unknown status"
    assert lib.pisa_status_string(-1).decode() == "unknown status"


@pytest.mark.parametrize("cap", [1, 63, 64, 65, 1024, 4096, 131072, 131328, 262144])
def test_pyramid_nodes_match_level_sizes(lib, cap):
    assert lib.pisa_pyramid_nodes(cap) == sum(oracle.level_sizes(cap))


def test_pyramid_nodes_rejects_empty(lib):
    assert lib.pisa_pyramid_nodes(0) == 0


def _cfg(**kw):
    base = dict(batch=1, seq_len=4096, n_q_heads=16, n_kv_heads=1, head_dim=128, top_k=16, dtype=None)
    base.update(kw)
    import torch
    return binding.make_cfg(base["batch"], base["seq_len"], base["n_q_heads"], base["n_kv_heads"],
                            base["head_dim"], base["top_k"], base["dtype"] or torch.bfloat16)


def test_workspace_and_pyramid_bytes(lib):
    cfg = _cfg(batch=2, seq_len=32768, n_q_heads=32, n_kv_heads=2, top_k=32)
    slots = 2 * 2 * 32768 * 64
    ws = lib.pisa_select_workspace_bytes(ctypes.byref(cfg))
    assert ws >= 3 * slots * 4
    assert lib.pisa_pyramid_bytes(ctypes.byref(cfg), 32768) == 2 * 2 * sum(oracle.level_sizes(32768)) * 128 * 4


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, 2), ("top_k", 33, 2), ("top_k", 0, 1), ("n_kv_heads", 5, 1), ("n_q_heads", 24, 2),
    ("block", 32, 2), ("fanout", 4, 2), ("seq_len", 0, 1), ("batch", 0, 1), ("dtype", 7, 1), ("dtype", -1, 1),
    ("score", 3, 1), ("score", -5, 1),
])
def test_invalid_configs_are_rejected_before_launch(lib, field, value, status):
    cfg = _cfg()
    setattr(cfg, field, value)
    t = binding.PisaTensor(16, 0, 128, 128)
    got = lib.pisa_build_pyramid(ctypes.byref(cfg), t, 16, 16, ctypes.c_void_p(16), None)
    assert got == status
    assert lib.pisa_select_workspace_bytes(ctypes.byref(cfg)) == 0


def test_invalid_tensors_are_rejected_before_launch(lib):
    cfg = _cfg()
    good = binding.PisaTensor(4096, 0, 128, 128)
    assert lib.pisa_build_pyramid(ctypes.byref(cfg), binding.PisaTensor(None, 0, 128, 128), 16, 16,
                                  ctypes.c_void_p(4096), None) == 1          # null
    assert lib.pisa_build_pyramid(ctypes.byref(cfg), binding.PisaTensor(4100, 0, 128, 128), 16, 16,
                                  ctypes.c_void_p(4096), None) == 1          # misaligned
    assert lib.pisa_build_pyramid(ctypes.byref(cfg), binding.PisaTensor(4096, 0, 130, 128), 16, 16,
                                  ctypes.c_void_p(4096), None) == 1          # stride not a multiple of 8
    assert lib.pisa_build_pyramid(ctypes.byref(cfg), good, 17, 16, ctypes.c_void_p(4096), None) == 1   # n > capacity
    # workspace too small
    assert lib.pisa_select_blocks(ctypes.byref(cfg), good, good, ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                                  None, ctypes.c_void_p(4096), 16, None) == 3
    # decode: position beyond capacity, and the on-chip limit G * 2K <= 256
    o = binding.PisaTensor(4096, 0, 0, 128)
    assert lib.pisa_decode_step(ctypes.byref(cfg), 4096, good, good, good, good, good, ctypes.c_void_p(4096),
                                None, o, 1, None) == 1
    big = _cfg(top_k=16, n_q_heads=16)
    assert lib.pisa_decode_step(ctypes.byref(big), 10, good, good, good, good, good, ctypes.c_void_p(4096),
                                None, o, 1, None) == 2
    # output element type must be float32 or bfloat16
    assert lib.pisa_sparse_attn_fwd(ctypes.byref(cfg), good, good, good, ctypes.c_void_p(4096), good, 5,
                                    None, ctypes.c_void_p(4096), 1 << 30, None) == 1
    # bf16 attention needs its workspace: packed K and V blocks, the (m, l) pair of every
    # (token, query head) carried between the two passes of a float32-output call, then the token
    # order of the passes (block counts, key counts per chunk of 4096 tokens and key totals, two
    # 64-bit statistics, the tokens' keys and their positions, two passes each), each array rounded
    # up to 256 bytes
    up = lambda x: -(-x // 256) * 256
    m1 = 4096 // 64
    want = (2 * 4096 * 128 * 2 + 16 * 4096 * 2 * 4 + up(m1 * 4) + 2 * up(2 * (m1 + 1) * 4) + 256
            + 2 * up(2 * 4096 * 4))
    assert lib.pisa_attn_workspace_bytes(ctypes.byref(cfg)) == want
    assert lib.pisa_sparse_attn_fwd(ctypes.byref(cfg), good, good, good, ctypes.c_void_p(4096), good, 0,
                                    None, None, 0, None) == 3


def test_flat_selection_validation_and_workspace(lib):
    """The flat baseline keeps at most 16 leaves and needs its two packed buffers."""
    cfg = _cfg()
    good = binding.PisaTensor(4096, 0, 128, 128)
    groups, tiles = -(-cfg.seq_len // 16), -(-(-(-cfg.seq_len // 64)) // 16)
    want = (-(-groups * 16 * cfg.head_dim * 4 // 256) + -(-tiles * 16 * cfg.head_dim * 4 // 256)) * 256
    assert lib.pisa_flat_workspace_bytes(ctypes.byref(cfg)) == want
    assert lib.pisa_select_flat(ctypes.byref(cfg), good, ctypes.c_void_p(4096), ctypes.c_void_p(4096), None,
                                ctypes.c_void_p(4096), 16, None) == 3                      # workspace too small
    assert lib.pisa_select_flat(ctypes.byref(cfg), good, ctypes.c_void_p(4096), None, None,
                                ctypes.c_void_p(4096), 1 << 30, None) == 1                 # no output
    wide = _cfg(top_k=17)
    assert lib.pisa_select_flat(ctypes.byref(wide), good, ctypes.c_void_p(4096), ctypes.c_void_p(4096), None,
                                ctypes.c_void_p(4096), 1 << 30, None) == 2                 # K > 16


def test_backward_validation_and_workspace(lib):
    """The backward takes bf16 inputs, at most 8192 leaves, a float32 or bfloat16 gradient type
    and its full workspace; everything is checked before any launch."""
    import torch

    cfg = _cfg(batch=1, seq_len=4096, n_q_heads=16, n_kv_heads=1, top_k=16)
    ws = lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(cfg))
    m1, slots = 64, 4096 * 16
    max_items = slots // 512 + m1
    assert ws >= 2 * m1 * 64 * 128 * 2 + 4096 * 8320 + 2 * slots * 4 + max_items * 2 * 64 * 128 * 4
    assert lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(_cfg(dtype=torch.float32))) == 0
    assert lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(_cfg(seq_len=8192 * 64 + 1))) == 0
    assert lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(_cfg(seq_len=8192 * 64))) > 0
    good = binding.PisaTensor(4096, 0, 128, 128)
    bad = binding.PisaTensor(4100, 0, 128, 128)
    lse = ctypes.c_void_p(4096)

    def call(c=cfg, gd=0, q=good, dq=good, w=ctypes.c_void_p(4096), wlen=1 << 40, lse_ptr=lse):
        return lib.pisa_sparse_attn_bwd(ctypes.byref(c), q, good, good, ctypes.c_void_p(4096), good, good, gd,
                                        lse_ptr, dq, good, good, w, wlen, None)

    assert call(c=_cfg(dtype=torch.float32)) == 2            # fp32 inputs unsupported
    assert call(wlen=16) == 3                                 # workspace too small
    assert call(w=ctypes.c_void_p(4096 + 16)) == 3            # workspace not 256-byte aligned
    assert call(gd=5) == 1                                    # gradient type
    assert call(q=bad) == 1 and call(dq=bad) == 1             # misaligned tensors
    assert call(lse_ptr=None) == 1                            # row LSE required


def test_binding_rejects_mismatched_tensors_before_any_call():
    """The Python binding checks dtype and shape agreement, output overlap and workspace size in
    bytes before it reaches the library (CPU tensors: nothing is launched)."""
    import torch

    B, N, Hq, Hkv, d, K = 1, 256, 4, 1, 64, 2
    q = torch.zeros((B, N, Hq, d), dtype=torch.bfloat16)
    k = torch.zeros((B, N, Hkv, d), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    sel = torch.zeros((B, Hkv, N, K), dtype=torch.int32)
    with pytest.raises(ValueError, match="dtype"):            # a float32 q with bfloat16 K/V
        binding.sparse_attn_fwd(q.float(), k, v, sel)
    with pytest.raises(ValueError, match="shape"):            # v of another length
        binding.sparse_attn_fwd(q, k, v[:, :128], sel)
    with pytest.raises(ValueError, match="shape"):            # undersized output
        binding.sparse_attn_fwd(q, k, v, sel, out=torch.empty((B, N - 1, Hq, d), dtype=torch.float32))
    with pytest.raises(ValueError, match="overlap"):          # output aliasing q
        binding.sparse_attn_fwd(q, k, v, sel, out=q)
    packed = torch.zeros((B, N, Hq + 2 * Hkv, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="overlap"):          # output aliasing a view of a packed QKV buffer
        binding.sparse_attn_fwd(packed[:, :, :Hq], packed[:, :, Hq:Hq + 1], packed[:, :, Hq + 1:], sel,
                                out=packed[:, :, :Hq])
    assert not binding._overlap(packed[:, :, :Hq], q)
    pyr = torch.zeros((B, Hkv, binding.pyramid_nodes(N), d), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):            # pyramid of another capacity
        binding.select_blocks(q, k, pyr[:, :, 1:], K)
    with pytest.raises(ValueError, match="dtype"):
        binding.select_blocks(q, k.float(), pyr, K)
    kc = torch.zeros((2, 300, Hkv, d), dtype=torch.bfloat16)
    dpyr = torch.zeros((2, Hkv, binding.pyramid_nodes(300), d), dtype=torch.float32)
    qn = torch.zeros((2, Hq, d), dtype=torch.bfloat16)
    kn = torch.zeros((2, Hkv, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):            # float32 query against bfloat16 caches
        binding.decode_step(qn.float(), kn, kn, kc, kc.clone(), dpyr, 10, K)
    with pytest.raises(ValueError, match="shape"):            # pyramid sized for another capacity
        binding.decode_step(qn, kn, kn, kc, kc.clone(), dpyr[:, :, :-1], 10, K)
    assert binding._ws_bytes(torch.empty(10, dtype=torch.float32)) == 40

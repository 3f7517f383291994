"""Seeded synthetic workloads for PISA prefill and decode.

This module only draws inputs: it holds no part of the method's arithmetic
(no pooling, scoring, selection or attention).  The GPU path and the CPU
oracle both consume the arrays it returns, so the two always see identical
bytes.

Shapes and value distributions follow the five workloads the path is
measured on (tiny fp32 prefill, 4K / 32K / 256K bf16 prefill, and a
64-sequence decode over a 131072-token context), plus three 64K input
regimes of the selection-quality study (diffuse, isolated strong blocks, and
strong blocks in runs of adjacent leaves).  The pages that describe
PISA measure selection on real model activations, which are not available
here; these planted Gaussian inputs stand in for them.

Recipe (every draw is ``numpy.random.default_rng([seed, tensor_id, ...])``):

* ``u``  = unit vector, ``rng([seed, 99]).standard_normal(d)`` normalised.
* ``Q[b, :, h, :]``   = ``rng([seed, 0, b, h]).standard_normal((N, d))`` + alpha_q * u
* ``K[b, :, kvh, :]`` = ``rng([seed, 1, b, kvh]).standard_normal((N, d))``, plus
  alpha_k * u on every key of ``n_plant`` leaf blocks chosen by
  ``rng([seed, 98, b, kvh]).choice(M1, n_plant, replace=False)``; with
  ``plant_run`` = r > 1 the same stream instead picks ceil(n_plant / r) of the
  aligned runs of r adjacent leaves.
* ``V[b, :, kvh, :]`` = ``rng([seed, 2, b, kvh]).standard_normal((N, d))``
* decode tokens: ``rng([seed, 10|11|12, b, head]).standard_normal((steps, d))``
  for q / k_new / v_new.

All draws are float32; shifts are added in float32, then the bf16
workloads round to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses

import numpy as np

LEAF = 64      # C: raw keys per leaf block
FANOUT = 2     # g: children per pyramid node above the leaves


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    seq_len: int          # prefill length N, or the prebuilt context length for decode
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    top_k: int
    dtype: str            # "f32" or "bf16"
    plant_blocks: int     # leaf blocks per (b, kvh) whose keys get alpha_k * u (0: none)
    alpha_k: float
    alpha_q: float
    decode_steps: int = 0
    block: int = LEAF
    fanout: int = FANOUT
    plant_run: int = 1    # planted blocks come in runs of this many adjacent leaves

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_leaves(self) -> int:
        return -(-self.seq_len // self.block)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _plant_count(frac: float, n_leaves: int) -> int:
    return max(1, int(round(frac * n_leaves)))


# The five workloads: tiny fp32 prefill, three bf16 prefills and the decode run.
WORKLOADS = {
    "tiny_f32_n1024": Workload("tiny_f32_n1024", seed=0, batch=1, seq_len=1024, head_dim=64,
                               n_q_heads=4, n_kv_heads=1, top_k=4, dtype="f32",
                               plant_blocks=2, alpha_k=3.0, alpha_q=1.5),
    "prefill_n4096": Workload("prefill_n4096", seed=1, batch=1, seq_len=4096, head_dim=128,
                              n_q_heads=16, n_kv_heads=1, top_k=16, dtype="bf16",
                              plant_blocks=_plant_count(0.02, 64), alpha_k=2.0, alpha_q=1.0),
    "prefill_n32768": Workload("prefill_n32768", seed=2, batch=2, seq_len=32768, head_dim=128,
                               n_q_heads=32, n_kv_heads=2, top_k=32, dtype="bf16",
                               plant_blocks=_plant_count(0.02, 512), alpha_k=2.0, alpha_q=1.0),
    "prefill_n262144": Workload("prefill_n262144", seed=3, batch=1, seq_len=262144, head_dim=128,
                                n_q_heads=16, n_kv_heads=1, top_k=16, dtype="bf16",
                                plant_blocks=_plant_count(0.005, 4096), alpha_k=2.5, alpha_q=1.0),
    # input regimes of the selection-quality study (64K tokens, one KV group, K = 8)
    "quality_diffuse_n65536": Workload("quality_diffuse_n65536", seed=21, batch=1, seq_len=65536, head_dim=128,
                                       n_q_heads=16, n_kv_heads=1, top_k=8, dtype="bf16",
                                       plant_blocks=_plant_count(0.005, 1024), alpha_k=2.5, alpha_q=1.0),
    "quality_needles_n65536": Workload("quality_needles_n65536", seed=22, batch=1, seq_len=65536, head_dim=128,
                                       n_q_heads=16, n_kv_heads=1, top_k=8, dtype="bf16",
                                       plant_blocks=_plant_count(0.01, 1024), alpha_k=12.0, alpha_q=2.0),
    "quality_runs_n65536": Workload("quality_runs_n65536", seed=23, batch=1, seq_len=65536, head_dim=128,
                                    n_q_heads=16, n_kv_heads=1, top_k=8, dtype="bf16",
                                    plant_blocks=_plant_count(0.01, 1024), alpha_k=12.0, alpha_q=2.0, plant_run=8),
    "decode_b64_ctx131072": Workload("decode_b64_ctx131072", seed=4, batch=64, seq_len=131072,
                                     head_dim=128, n_q_heads=32, n_kv_heads=8, top_k=16,
                                     dtype="bf16", plant_blocks=0, alpha_k=0.0, alpha_q=0.0,
                                     decode_steps=256),
}


# ----------------------------------------------------------------------------- bf16 helpers
def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantise(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the workload's storage type, returned as float32."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return bf16_bits_to_f32(round_bf16_bits(x))


# ----------------------------------------------------------------------------- draws
def _rng(*ids: int) -> np.random.Generator:
    return np.random.default_rng([int(i) for i in ids])


def planted_direction(w: Workload) -> np.ndarray:
    u = _rng(w.seed, 99).standard_normal(w.head_dim)
    return (u / np.linalg.norm(u)).astype(np.float32)


def planted_blocks(w: Workload, b: int, kvh: int, n_leaves: int | None = None) -> np.ndarray:
    m1 = w.n_leaves if n_leaves is None else n_leaves
    if w.plant_blocks <= 0:
        return np.zeros(0, dtype=np.int64)
    if w.plant_run <= 1:
        return np.sort(_rng(w.seed, 98, b, kvh).choice(m1, min(w.plant_blocks, m1), replace=False))
    runs = m1 // w.plant_run                    # run r covers leaves [r * run, (r + 1) * run)
    pick = _rng(w.seed, 98, b, kvh).choice(runs, min(-(-w.plant_blocks // w.plant_run), runs), replace=False)
    return np.sort((pick[:, None] * w.plant_run + np.arange(w.plant_run)[None, :]).ravel())


def _draw_q(w: Workload, b: int, h: int, n: int) -> np.ndarray:
    x = _rng(w.seed, 0, b, h).standard_normal((n, w.head_dim), dtype=np.float32)
    if w.alpha_q:
        x += np.float32(w.alpha_q) * planted_direction(w)
    return x


def _draw_k(w: Workload, b: int, kvh: int, n: int) -> np.ndarray:
    x = _rng(w.seed, 1, b, kvh).standard_normal((n, w.head_dim), dtype=np.float32)
    if w.plant_blocks:
        shift = np.float32(w.alpha_k) * planted_direction(w)
        for j in planted_blocks(w, b, kvh, -(-n // w.block)):
            x[j * w.block:(j + 1) * w.block] += shift
    return x


def _draw_v(w: Workload, b: int, kvh: int, n: int) -> np.ndarray:
    return _rng(w.seed, 2, b, kvh).standard_normal((n, w.head_dim), dtype=np.float32)


def _draw_do(w: Workload, b: int, h: int, n: int) -> np.ndarray:
    return _rng(w.seed, 3, b, h).standard_normal((n, w.head_dim), dtype=np.float32)


_DRAW = {"q": _draw_q, "k": _draw_k, "v": _draw_v, "do": _draw_do}


def draw(w: Workload, which: str, b: int, h: int, n: int | None = None, bits: bool = False) -> np.ndarray:
    """One [n, d] slice of Q ('q', head h), K / V ('k' / 'v', KV head h) or the upstream
    gradient of the attention output ('do', head h) of sequence b.

    Returns float32 values rounded to the workload dtype, or with ``bits`` the
    storage form (float32 for fp32 workloads, uint16 bfloat16 patterns otherwise).
    """
    x = _DRAW[which](w, b, h, w.seq_len if n is None else n)
    return to_storage(x, w.dtype) if bits else quantise(x, w.dtype)


def q_slice(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    """Q[b, :n, h, :] as float32 values already rounded to the workload dtype."""
    return draw(w, "q", b, h, n)


def k_slice(w: Workload, b: int, kvh: int, n: int | None = None) -> np.ndarray:
    return draw(w, "k", b, kvh, n)


def v_slice(w: Workload, b: int, kvh: int, n: int | None = None) -> np.ndarray:
    return draw(w, "v", b, kvh, n)


def device_prefill_inputs(w: Workload, n: int, seed: int = 7, with_v: bool = False):
    """Q and K (and V) of n tokens drawn on the GPU, for lengths whose host draw would take minutes.

    The recipe of the host draw with torch's generator instead of NumPy's streams (so the values
    differ from ``prefill_inputs``): u = a normalised N(0,1) vector, Q = N(0,1) + alpha_q u,
    K = N(0,1) with alpha_k u added to every key of round(frac * M1) leaf blocks chosen by a
    random permutation (frac = the workload's planted fraction), V = N(0,1); all drawn in float32
    from one generator seeded with ``seed``, in that order, then rounded to bf16.
    """
    import torch

    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(seed)
    d = w.head_dim
    u = torch.randn(d, generator=gen, device="cuda:0")
    u = u / u.norm()
    q = torch.randn((w.batch, n, w.n_q_heads, d), generator=gen, device="cuda:0") + w.alpha_q * u
    k = torch.randn((w.batch, n, w.n_kv_heads, d), generator=gen, device="cuda:0")
    m1 = -(-n // w.block)
    n_plant = max(1, round(w.plant_blocks / w.n_leaves * m1))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            for j in torch.randperm(m1, generator=gen, device="cuda:0")[:n_plant].tolist():
                k[b, w.block * j:w.block * (j + 1), h] += w.alpha_k * u
    out = [q.to(torch.bfloat16), k.to(torch.bfloat16)]
    del q, k
    if with_v:
        out.append(torch.randn((w.batch, n, w.n_kv_heads, d), generator=gen, device="cuda:0").to(torch.bfloat16))
    return tuple(out)


def decode_tokens(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """New per-step vectors [steps, d] for 'q', 'k' or 'v' of sequence b, head h."""
    tid = {"q": 10, "k": 11, "v": 12}[which]
    x = _rng(w.seed, tid, b, h).standard_normal((w.decode_steps, w.head_dim), dtype=np.float32)
    return quantise(x, w.dtype)


def prefill_inputs(w: Workload, batches=None, n: int | None = None, bits: bool = False, threads: int = 8,
                   with_q: bool = True):
    """Q [B, n, Hq, d], K and V [B, n, Hkv, d] for the given sequences (default: all).

    float32 values in the workload dtype, or storage arrays with ``bits``
    (uint16 bfloat16 patterns for bf16 workloads).  Slices are drawn in a
    thread pool; every slice comes from its own seeded stream, so the result
    does not depend on the pool.
    """
    import concurrent.futures

    batches = list(range(w.batch)) if batches is None else list(batches)
    n = w.seq_len if n is None else n
    dt = (np.uint16 if w.dtype == "bf16" else np.float32) if bits else np.float32
    q = np.empty((len(batches), n, w.n_q_heads if with_q else 0, w.head_dim), dtype=dt)
    k = np.empty((len(batches), n, w.n_kv_heads, w.head_dim), dtype=dt)
    v = np.empty_like(k)
    jobs = [(q, "q", bi, b, h) for bi, b in enumerate(batches) for h in range(q.shape[2])]
    jobs += [(arr, name, bi, b, h) for bi, b in enumerate(batches) for h in range(w.n_kv_heads)
             for arr, name in ((k, "k"), (v, "v"))]

    def run(job):
        arr, name, bi, b, h = job
        arr[bi, :, h] = draw(w, name, b, h, n, bits=bits)

    with concurrent.futures.ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, jobs))
    return q, k, v


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array for the device: float32 as is, bf16 as uint16 bit patterns."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16_bits(x)


def grad_output(w: Workload, batches=None, n: int | None = None) -> np.ndarray:
    """Upstream gradient dO [B, n, Hq, d] of the attention output: N(0,1), rounded to the workload dtype
    (float32 values)."""
    import concurrent.futures

    batches = list(range(w.batch)) if batches is None else list(batches)
    n = w.seq_len if n is None else n
    out = np.empty((len(batches), n, w.n_q_heads, w.head_dim), dtype=np.float32)

    def fill(job):
        bi, b, h = job
        out[bi, :, h] = draw(w, "do", b, h, n)

    jobs = [(bi, b, h) for bi, b in enumerate(batches) for h in range(w.n_q_heads)]
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, jobs))
    return out


def random_selection(w: Workload, K: int, b: int, kvh: int, n: int | None = None) -> np.ndarray:
    """A valid block selection [n, K] int32 for (b, kvh): row t lists min(K, t // 64 + 1) distinct
    blocks j <= t // 64, ascending, padded with -1; rows with more candidates than K take K of them
    uniformly.  Drawn from ``rng([seed, 20, b, kvh])``; used as a fixed input of the attention
    gradients, independent of any scoring."""
    n = w.seq_len if n is None else n
    rng = _rng(w.seed, 20, b, kvh)
    m = np.arange(n) // w.block + 1                            # candidate blocks of each row
    out = np.full((n, K), -1, dtype=np.int32)
    small = m <= K
    for c in np.unique(m[small]):
        out[m == c, :c] = np.arange(c, dtype=np.int32)
    rows = np.nonzero(~small)[0]
    if rows.size:
        keys = rng.random((rows.size, 4 * K))
        cand = np.floor(keys * m[rows, None]).astype(np.int64)
        for r, row in enumerate(rows):
            picked = np.unique(cand[r])
            while picked.size < K:                             # rare: fewer than K distinct draws
                extra = np.floor(rng.random(4 * K) * m[row]).astype(np.int64)
                picked = np.unique(np.concatenate([picked, extra]))
            chosen = rng.permutation(picked)[:K]
            out[row] = np.sort(chosen)
    return out

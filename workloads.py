"""Seeded synthetic inputs for the paged-attention decode workloads.

This module is the ONLY code shared by the GPU path's tests/bench and the oracle: it draws
random values and describes the allocator operations of each workload as plain data.  It
holds none of the method's arithmetic (no slot computation, no gather, no softmax, no
quantization); each side runs the operation script with its own allocator and its own
write/attention code.

Recipe (the pages use no dataset; these stand in for a model's activations):

* Values: ``numpy.random.Generator(PCG64)`` seeded from ``SeedSequence(408_000 + k)`` for
  workload k, one spawned child per tensor; float32 standard normals times the workload's
  standard deviation, rounded once to the storage type (bfloat16: round to nearest even,
  done by torch's conversion).  Large workloads can draw on the device instead, with a
  ``torch.Generator`` seeded from the same sequence (``device_normal``).
* Physical block order: the allocator's initial free queue is a seeded permutation of all
  blocks, so logically adjacent blocks are scattered.
* Ragged lengths: ``round(lognormal(ln 300, 1.0))`` clipped to 16..8192 for every request;
  the first ``n_shared`` requests instead hold a ``prefix``-token shared prefix plus a
  private suffix equal to their draw clipped to 16..(8192 - prefix).
* fp8 scales: per KV head, max |x| over that head's stored bfloat16 values / 448, as float32.

A workload is decoded at its step: every request appends one token (the new token's K/V are
written first), so the decode length L_b includes the new token and L_b - 1 tokens were
cached before the step.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------- shapes

@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    bs: int
    fmt: str            # cache storage: 'f32' | 'bf16' | 'fp8'
    q_fmt: str          # q / out storage: 'f32' | 'bf16'
    std: float
    seq_lens: np.ndarray            # decode lengths L_b (including the step token)
    num_blocks: int
    free_order: np.ndarray          # initial free queue (permutation of num_blocks)
    ops: list = field(default_factory=list)  # prefill script: ('add', s) | ('append', s, n) | ('fork', p, c) | ('free', s)
    layers: int = 1
    seed_index: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def in_fmt(self) -> str:
        """Storage of the K/V rows handed to the write (fp8 and mxfp4 caches are fed bf16 rows)."""
        return "bf16" if self.fmt in ("fp8", "mxfp4") else self.fmt

    @property
    def prefill_tokens(self) -> int:
        return int(sum(op[2] for op in self.ops if op[0] == "append"))

    @property
    def max_blocks(self) -> int:
        return int(-(-int(self.seq_lens.max()) // self.bs)) if len(self.seq_lens) else 0


def _seq(k: int, n: int = 8):
    return np.random.SeedSequence(408_000 + k).spawn(n)


_CHILD = {"perm": 0, "lens": 1, "q": 2, "k_pre": 3, "v_pre": 4, "k_new": 5, "v_new": 6, "misc": 7}


def rng(w: Workload, what: str, layer: int = 0) -> np.random.Generator:
    child = _seq(w.seed_index)[_CHILD[what]]
    if layer:
        child = child.spawn(layer + 1)[layer]
    return np.random.Generator(np.random.PCG64(child))


def _simple_ops(seq_lens):
    ops = []
    for b, L in enumerate(seq_lens):
        ops.append(("add", b))
        if L - 1 > 0:
            ops.append(("append", b, int(L) - 1))
    return ops


def _blocks_for(seq_lens, bs):
    return int(sum(-(-int(L) // bs) for L in seq_lens))


def _perm(w_seed: int, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_seq(w_seed)[_CHILD["perm"]]))
    return g.permutation(n).astype(np.int32)


# --------------------------------------------------------------------------- workloads

def tiny_mha_f32() -> Workload:
    """1 layer, batch 4, 8 q heads = 8 kv heads, head_dim 64, fp32, block 16,
    lengths {17, 50, 128, 200}, pool of 64 blocks in seeded order, N(0,1) values."""
    lens = np.array([17, 50, 128, 200], dtype=np.int64)
    return Workload("tiny_mha_f32", B=4, Hq=8, Hkv=8, d=64, bs=16, fmt="f32", q_fmt="f32",
                    std=1.0, seq_lens=lens, num_blocks=64, free_order=_perm(1, 64),
                    ops=_simple_ops(lens), layers=1, seed_index=1)


def gqa_uniform(B=16, L=4096, Hq=32, Hkv=8, d=128, bs=16, fmt="bf16", layers=32,
                spare_blocks=None, seed_index=2, name="llama3_8b_gqa_decode") -> Workload:
    """Llama-3-8B-shaped GQA decode: 32 q / 8 kv heads, d 128, bf16, block 16, batch 16,
    every length 4096, 32 per-layer caches sharing one seeded block order, N(0,1)*0.5."""
    lens = np.full(B, L, dtype=np.int64)
    need = _blocks_for(lens, bs)
    spare = B * 4 if spare_blocks is None else spare_blocks
    n = need + spare
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, bs=bs, fmt=fmt, q_fmt="bf16", std=0.5,
                    seq_lens=lens, num_blocks=n, free_order=_perm(seed_index, n),
                    ops=_simple_ops(lens), layers=layers, seed_index=seed_index)


def long_context(B=2, L=131072, Hq=64, Hkv=8, d=128, bs=16, spare_blocks=None,
                 seed_index=4, name="long_context_70b_layer") -> Workload:
    """70B-shaped layer at 128k: 64 q / 8 kv heads, d 128, bf16, block 16, batch 2,
    length 131072 each, N(0,1)*0.5, split-K partitions of 512 tokens."""
    return gqa_uniform(B=B, L=L, Hq=Hq, Hkv=Hkv, d=d, bs=bs, fmt="bf16", layers=1,
                       spare_blocks=B * 4 if spare_blocks is None else spare_blocks,
                       seed_index=seed_index, name=name)


def ragged_lengths(seed_index: int, B=256, n_shared=64, prefix=1024, median=300.0,
                   sigma=1.0, lo=16, hi=8192):
    g = np.random.Generator(np.random.PCG64(_seq(seed_index)[_CHILD["lens"]]))
    x = np.round(g.lognormal(mean=np.log(median), sigma=sigma, size=B)).astype(np.int64)
    lens = np.clip(x, lo, hi)
    suffix = np.clip(x[:n_shared], lo, hi - prefix)
    lens[:n_shared] = prefix + suffix
    return lens, suffix


def ragged_prefix(bs=16, fmt="bf16", B=256, n_shared=64, prefix=1024, spare_blocks=256,
                  seed_index=3, name=None) -> Workload:
    """Ragged serving batch: 256 requests, GQA 32/8, d 128, block 16; lognormal lengths
    (median 300, sigma 1, clip 16..8192); requests 0..n_shared-1 share one prefix-token
    system prefix (prefix/bs shared blocks, each referenced n_shared times) plus private
    suffixes.  The prefix is written once through a holder sequence that is forked into
    every sharer and then released."""
    lens, suffix = ragged_lengths(seed_index, B=B, n_shared=n_shared, prefix=prefix)
    holder = B                                   # sequence id of the prefix holder
    ops = []
    if n_shared:
        ops += [("add", holder), ("append", holder, prefix)]
        ops += [("fork", holder, b) for b in range(n_shared)]
        ops += [("free", holder)]
        ops += [("append", b, int(suffix[b]) - 1) for b in range(n_shared) if suffix[b] > 1]
    for b in range(n_shared, B):
        ops.append(("add", b))
        if lens[b] > 1:
            ops.append(("append", b, int(lens[b]) - 1))
    shared_blocks = -(-prefix // bs) if n_shared else 0
    private = sum(-(-int(L) // bs) for L in lens[n_shared:])
    private += sum(-(-int(prefix + s) // bs) - prefix // bs for s in suffix) if n_shared else 0
    n = int(shared_blocks + private + spare_blocks)
    nm = name or f"ragged_prefix_bs{bs}_{fmt}"
    return Workload(nm, B=B, Hq=32, Hkv=8, d=128, bs=bs, fmt=fmt, q_fmt="bf16", std=0.5,
                    seq_lens=lens, num_blocks=n, free_order=_perm(seed_index, n), ops=ops,
                    layers=1, seed_index=seed_index)


def sweep_settings():
    """Block-size x KV-dtype sweep on the ragged prefix batch."""
    return [(bs, fmt) for fmt in ("bf16", "fp8") for bs in (8, 16, 32, 128)]


# --------------------------------------------------------------------------- values

def _round_storage(x32: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return x32.astype(np.float32)
    if fmt == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(fmt)


def normal_storage(g: np.random.Generator, shape, std: float, fmt: str) -> np.ndarray:
    """float32 standard normals * std rounded to the storage type ('f32' float32,
    'bf16' uint16 bit patterns)."""
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return _round_storage(x, fmt)


def host_values(w: Workload, layer: int = 0) -> dict:
    """All values of one layer of a workload on the host, as stored bits/values:
    q [B,Hq,d], prefill rows k_pre/v_pre [T,Hkv,d] in operation order, step rows
    k_new/v_new [B,Hkv,d], and fp8 scales when the cache is fp8."""
    T = w.prefill_tokens
    vals = {
        "q": normal_storage(rng(w, "q", layer), (w.B, w.Hq, w.d), w.std, w.q_fmt),
        "k_pre": normal_storage(rng(w, "k_pre", layer), (T, w.Hkv, w.d), w.std, w.in_fmt),
        "v_pre": normal_storage(rng(w, "v_pre", layer), (T, w.Hkv, w.d), w.std, w.in_fmt),
        "k_new": normal_storage(rng(w, "k_new", layer), (w.B, w.Hkv, w.d), w.std, w.in_fmt),
        "v_new": normal_storage(rng(w, "v_new", layer), (w.B, w.Hkv, w.d), w.std, w.in_fmt),
    }
    if w.fmt == "fp8":
        vals["k_scale"] = _amax_scale(vals["k_pre"], vals["k_new"])
        vals["v_scale"] = _amax_scale(vals["v_pre"], vals["v_new"])
    return vals


def _bf16_abs_max_per_head(bits: np.ndarray) -> np.ndarray:
    # exponent/mantissa bits order like the magnitude, so the max pattern is the max value
    mag = (bits & np.uint16(0x7FFF)).reshape(-1, bits.shape[-2], bits.shape[-1])
    m = mag.max(axis=(0, 2)).astype(np.uint32) << np.uint32(16)
    return m.view(np.float32).astype(np.float64)


def _amax_scale(pre: np.ndarray, new: np.ndarray) -> np.ndarray:
    a = np.maximum(_bf16_abs_max_per_head(pre) if pre.size else 0.0, _bf16_abs_max_per_head(new))
    return (np.maximum(a, 1e-30) / 448.0).astype(np.float32)


def device_normal(w: Workload, what: str, shape, layer: int = 0, device="cuda"):
    """Same recipe drawn on the device with a seeded torch.Generator (for workloads too big
    to draw on the host).  Returns a torch tensor in the storage dtype."""
    import torch
    seed = int(rng(w, what, layer).integers(0, 2**62))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * w.std
    fmt = w.q_fmt if what == "q" else w.in_fmt
    return x if fmt == "f32" else x.to(torch.bfloat16)


# --------------------------------------------------------------------------- prompts

@dataclass
class PromptWorkload:
    """Requests arriving with token-id prompts, some starting with one of a few shared
    system prompts, for prefix caching.  `finished` requests are released right after
    their prompt is in (their blocks stay registered while free)."""
    name: str
    Hq: int
    Hkv: int
    d: int
    bs: int
    std: float
    prompts: list          # token ids per request
    finished: list         # requests released after their prompt is in
    step_tokens: list      # the decode token of each request
    num_blocks: int
    free_order: np.ndarray
    seed_index: int = 0


def prompt_workload(n_req=16, systems=(80, 160, 48), suffix_max=60, Hq=32, Hkv=8, d=128, bs=16,
                    finished_every=4, seed_index=7, name=None) -> PromptWorkload:
    """Request i starts with system prompt i % len(systems) and adds a private suffix of
    0..suffix_max tokens; token ids uniform in [0, 1000).  Every `finished_every`-th request
    is released after its prompt.  The pool holds every request's blocks without sharing
    (so a run without the cache fits too), in a seeded order."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(408_000 + seed_index)))
    sys_toks = [[int(x) for x in g.integers(0, 1000, size=n)] for n in systems]
    prompts, step = [], []
    for i in range(n_req):
        suffix = [int(x) for x in g.integers(0, 1000, size=int(g.integers(0, suffix_max + 1)))]
        prompts.append(sys_toks[i % len(sys_toks)] + suffix)
        step.append(int(g.integers(0, 1000)))
    finished = [i for i in range(n_req) if finished_every and i % finished_every == finished_every - 1]
    n = sum(-(-(len(p) + 1) // bs) for p in prompts) + 4
    return PromptWorkload(name or f"prompts{n_req}_bs{bs}_d{d}", Hq=Hq, Hkv=Hkv, d=d, bs=bs, std=0.5,
                          prompts=prompts, finished=finished, step_tokens=step, num_blocks=n,
                          free_order=_perm(seed_index, n), seed_index=seed_index)


def prefix_kv(token_ids, Hkv: int, d: int, std: float, seed_index: int, fmt: str = "bf16"):
    """K and V rows [n, Hkv, d] for a token sequence, each row a function of the whole
    token prefix through it (as a model's K/V are): row j is drawn from a generator seeded
    by the seed index and a 64-bit FNV-1a digest of token_ids[:j+1].  Equal prefixes give
    equal rows, different prefixes different ones."""
    h = 14695981039346656037
    ks, vs = [], []
    for t in token_ids:
        for i in range(4):
            h ^= (int(t) >> (8 * i)) & 0xFF
            h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
        g = np.random.Generator(np.random.PCG64([408_000 + seed_index, h]))
        x = g.standard_normal(size=(2, Hkv, d), dtype=np.float32) * np.float32(std)
        ks.append(x[0])
        vs.append(x[1])
    if not ks:
        z = np.zeros((0, Hkv, d), np.float32)
        return _round_storage(z, fmt), _round_storage(z, fmt)
    return _round_storage(np.stack(ks), fmt), _round_storage(np.stack(vs), fmt)

"""Slot-mapped KV write, block-table gather and decode attention (oracle; test
infrastructure only).

What is computed ("PagedAttention: Optimizing KV Cache Utilization in Large Language
Models", "The Math: Block Attention Calculation"): for the query q of the newest token,
the key vectors are found through the request's page table, and the attention weights are
the softmax of q.K^T / sqrt(d_k).  Readings where that section is silent or loose:

* It writes the softmax per block b.  The reading taken: ONE softmax over all of the
  request's keys, of which block b's weights are a slice.  A per-block softmax would make
  the output depend on block size and block boundaries, which contradicts paging being a
  transparent page table ("KV Cache Optimization and PagedAttention", prose on paging).
* It omits V.  The output is the weighted sum of the value vectors, o = A.V.
* Decode has query length 1; the new token's K/V are written before the attention, so
  ``seq_lens[b]`` counts the cached tokens including the new one and the query sees
  logical positions 0..L_b-1 (a new token's attention covers all earlier tokens: "KV Cache
  Optimization and PagedAttention", first paragraph; "KV Cache Management", "Why Does This
  Exist?").  No other mask.
* ``scale`` is taken as given (1/sqrt(d) in the workloads), widened to float64.
* Grouped-query attention: query head h reads KV head h // (Hq/Hkv).
* L_b = 0 gives o = 0 (the empty sum).

Cache layout (the pages fix none): ``cache[num_blocks, Hkv, block_size, d]``; slot s lives
at block s // block_size, row s % block_size.  Slots < 0 are padding and are skipped.

Storage formats: 'f32' (float32 values), 'bf16' (uint16 bit patterns), 'fp8' (uint8
E4M3FN codes with a float32 scale per KV head), 'mxfp4' (OCP MXFP4: per (block, head) tile
of bytes holding the 4-bit codes [block_size, d/2] and then the E8M0 scales of every 32 dims
[block_size, d/32]; see codecs).  The oracle reads the exact stored values in float64 and
computes the plain definition in float64.
"""

from __future__ import annotations

import math

import numpy as np

from . import codecs


# ----------------------------------------------------------------------------- KV write

def kv_write(k, v, slot_mapping, k_cache, v_cache, block_size: int, fmt: str,
             k_scale=None, v_scale=None) -> None:
    """Scatter new tokens' K/V rows into the caches, in place.

    k, v: [T, Hkv, d] stored inputs ('f32' float32 or 'bf16' uint16 bits).
    fmt: cache format.  For 'fp8' the inputs are bf16 bits or float32 values and every value
    of head h is quantized with that head's scale; otherwise the cache format equals the input
    format and rows are copied bit for bit.  Token t goes to block slot//block_size, row
    slot%block_size, for every KV head; slots < 0 are skipped.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots >= 0
    s = slots[live]
    assert len(np.unique(s)) == len(s), "duplicate slots in one write"
    assert np.all(s < k_cache.shape[0] * block_size), "slot beyond the cache"
    blk, row = s // block_size, s % block_size
    kr, vr = k[live], v[live]
    if fmt == "mxfp4":
        for src, cache in ((kr, k_cache), (vr, v_cache)):
            d = src.shape[-1]
            codes, scales = codecs.mxfp4_quantize(codecs.bf16_bits_to_f64(src))   # [T, Hkv, d], [T, Hkv, d/32]
            base = mx_tile_view(cache, block_size, d)
            base["codes"][blk, :, row] = codecs.pack_nibbles(codes)
            base["scales"][blk, :, row] = scales
        return
    if fmt == "fp8":
        ks = np.asarray(k_scale, dtype=np.float32)[None, :, None]
        vs = np.asarray(v_scale, dtype=np.float32)[None, :, None]
        exact = (lambda a: a.astype(np.float64)) if kr.dtype == np.float32 else codecs.bf16_bits_to_f64
        kr = codecs.e4m3_quantize(exact(kr), ks)
        vr = codecs.e4m3_quantize(exact(vr), vs)
    k_cache[blk, :, row] = kr
    v_cache[blk, :, row] = vr


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """Whole-block copies src -> dst (the copy-on-write step: "KV Cache Optimization and
    PagedAttention", prose on shared prefix blocks), in place, K and V, every head, row and
    dim.  A pair naming a block outside the pool is skipped, as the library's contract for
    its block copy states."""
    n = k_cache.shape[0]
    for src, dst in pairs:
        if 0 <= src < n and 0 <= dst < n:
            k_cache[dst] = k_cache[src]
            v_cache[dst] = v_cache[src]


def mx_tile_view(cache, block_size: int, d: int):
    """The two parts of an MXFP4 cache [num_blocks, Hkv, block_size * (d/2 + d/32)] bytes: per
    (block, head) the codes [block_size, d/2] (two per byte, even dim in the low nibble) and
    then the E8M0 scales [block_size, d/32], as writable views."""
    n, h, tb = cache.shape
    cb = block_size * d // 2
    assert tb == cb + block_size * d // 32
    return {"codes": cache[:, :, :cb].reshape(n, h, block_size, d // 2),
            "scales": cache[:, :, cb:].reshape(n, h, block_size, d // 32)}


# ----------------------------------------------------------------------------- gather

def gather(cache, table_row, L: int, kv_head: int, block_size: int, fmt: str, scale=None, head_dim=None):
    """K (or V) rows of logical tokens 0..L-1 of one request and head, float64 [L, d]."""
    j = np.arange(L, dtype=np.int64)                       # logical token positions
    blk = np.asarray(table_row, dtype=np.int64)[j // block_size]   # page-table lookup
    assert np.all(blk >= 0), "block table entry -1 inside the sequence"
    if fmt == "mxfp4":                                     # the tile does not carry head_dim
        t = mx_tile_view(cache, block_size, int(head_dim))
        codes = codecs.unpack_nibbles(t["codes"][blk, kv_head, j % block_size])
        return codecs.mxfp4_dequantize(codes, t["scales"][blk, kv_head, j % block_size])
    out = codecs.storage_to_f64(cache[blk, kv_head, j % block_size], fmt)
    if fmt == "fp8":
        out *= np.float64(np.float32(scale[kv_head]))
    return out


# ----------------------------------------------------------------------------- attention

def attend(q_row, K, V, scale: float):
    """softmax(scale * q.K^T) . V for one query row, float64.  K, V: [L, d]."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = np.float64(scale) * (K @ np.asarray(q_row, dtype=np.float64))
    m = np.max(s)
    e = np.exp(s - m)
    p = e / np.sum(e)
    return p @ V


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float, block_size: int,
           fmt: str, q_fmt: str, k_scale=None, v_scale=None):
    """Decode attention for every request and query head.  Returns float64 [B, Hq, d].

    q: [B, Hq, d] stored ('f32' float32 or 'bf16' bits).  block_tables: [B, max_blocks].
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    qf = codecs.storage_to_f64(q, q_fmt)
    scale = float(np.float32(scale))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(Hkv):
            K = gather(k_cache, block_tables[b], L, g, block_size, fmt, k_scale, d)
            V = gather(v_cache, block_tables[b], L, g, block_size, fmt, v_scale, d)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend(qf[b, h], K, V, scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, scale: float, block_size: int,
            fmt: str, q_fmt: str, k_scale=None, v_scale=None):
    """Attention of several new tokens per request through the block table, causal.
    Returns float64 [T, Hq, d].

    The pages' step before decode: a prompt's K/V are computed once and stored ("KV Cache
    Management", "Why Does This Exist?": the first 1,000 tokens' keys and values are saved
    as they are calculated), and a token's attention covers all tokens before it ("KV Cache
    Optimization and PagedAttention", first paragraph).  Readings: the new tokens' K/V are
    written into the cache first (as for decode), so request b's L_b = seq_lens[b] cached
    tokens include its n_b = query_start[b+1] - query_start[b] new ones, which are its last
    n_b tokens; new token i sits at logical position L_b - n_b + i and sees positions
    0..L_b - n_b + i (itself included), through one softmax.  Earlier tokens of the request
    (a cached prefix or earlier chunks) are read from the cache like the new ones.

    q: [T, Hq, d] stored, request b's rows query_start[b]..query_start[b+1]-1.
    """
    T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    qf = codecs.storage_to_f64(q, q_fmt)
    scale = float(np.float32(scale))
    out = np.zeros((T, Hq, d), dtype=np.float64)
    B = len(seq_lens)
    for b in range(B):
        L = int(seq_lens[b])
        q0, q1 = int(query_start[b]), int(query_start[b + 1])
        n = q1 - q0
        assert 0 <= n <= L
        for g in range(Hkv):
            K = gather(k_cache, block_tables[b], L, g, block_size, fmt, k_scale, d)
            V = gather(v_cache, block_tables[b], L, g, block_size, fmt, v_scale, d)
            for i in range(n):
                pos = L - n + i                                # logical position of new token i
                for h in range(g * G, (g + 1) * G):
                    out[q0 + i, h] = attend(qf[q0 + i, h], K[: pos + 1], V[: pos + 1], scale)
    return out


def decode_splitk(q, k_cache, v_cache, block_tables, seq_lens, scale: float, block_size: int,
                  fmt: str, q_fmt: str, k_scale=None, v_scale=None, partition_tokens: int = 512):
    """The same result through partitions [P*p, min(P*(p+1), L)) of each request's tokens:
    each partition keeps its running maximum m_p, its sum l_p = sum exp(s - m_p) and its
    unnormalised accumulator acc_p = sum exp(s - m_p) v; the partitions are then merged by
    rescaling to the global maximum M:  o = sum_p e^(m_p-M) acc_p / sum_p e^(m_p-M) l_p.
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qf = codecs.storage_to_f64(q, q_fmt)
    scale = float(np.float32(scale))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for g in range(Hkv):
            K = gather(k_cache, block_tables[b], L, g, block_size, fmt, k_scale, d)
            V = gather(v_cache, block_tables[b], L, g, block_size, fmt, v_scale, d)
            for h in range(g * G, (g + 1) * G):
                parts = []
                for start in range(0, L, partition_tokens):
                    stop = min(start + partition_tokens, L)
                    s = scale * (K[start:stop] @ qf[b, h])
                    m = np.max(s)
                    e = np.exp(s - m)
                    parts.append((m, np.sum(e), e @ V[start:stop]))
                M = max(p[0] for p in parts)
                num = sum(math.exp(m - M) * acc for m, _, acc in parts)
                den = sum(math.exp(m - M) * l for m, l, _ in parts)
                out[b, h] = num / den
    return out


def decode_bruteforce(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                      block_size: int, fmt: str, q_fmt: str, k_scale=None, v_scale=None):
    """Pure-Python loops with math.exp over the stored values; tiny inputs only.
    Returns nested lists [B][Hq][d]."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qf = codecs.storage_to_f64(q, q_fmt).tolist()
    kc = codecs.storage_to_f64(k_cache, fmt).tolist()
    vc = codecs.storage_to_f64(v_cache, fmt).tolist()
    ks = [float(np.float32(x)) for x in k_scale] if fmt == "fp8" else [1.0] * Hkv
    vs = [float(np.float32(x)) for x in v_scale] if fmt == "fp8" else [1.0] * Hkv
    scale = float(np.float32(scale))
    out = []
    for b in range(B):
        L = int(seq_lens[b])
        rows = []
        for h in range(Hq):
            g = h // G
            scores = []
            for j in range(L):
                blk = int(block_tables[b][j // block_size])
                krow = kc[blk][g][j % block_size]
                dot = 0.0
                for i in range(d):
                    dot += qf[b][h][i] * (krow[i] * ks[g])
                scores.append(scale * dot)
            o = [0.0] * d
            if L:
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                for j in range(L):
                    blk = int(block_tables[b][j // block_size])
                    vrow = vc[blk][g][j % block_size]
                    for i in range(d):
                        o[i] += (w[j] / z) * (vrow[i] * vs[g])
            rows.append(o)
        out.append(rows)
    return out

"""Pins of the oracle's causal prefill (CPU only): torch's float64 scaled dot-product
attention with the causal mask written out, decode as the one-token special case,
causality, chunked = whole, and a pure-Python brute force on tiny inputs."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import codecs as C
from oracle.allocator import Allocator


def _case(rng, lens, n_new, Hq, Hkv, d, bs, perm_seed=5):
    """Requests with lens[b] cached tokens, of which the last n_new[b] are the queries;
    K/V rows written through the oracle's allocator and write in a permuted pool."""
    K_rows = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    V_rows = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    N = sum(-(-L // bs) for L in lens) + 2
    al = Allocator(N, bs, np.random.default_rng(perm_seed).permutation(N))
    slots = []
    for b, L in enumerate(lens):
        al.add(b)
        s, _ = al.append(b, L)
        slots += s
    kc = np.zeros((N, Hkv, bs, d), np.float32)
    vc = np.zeros_like(kc)
    A.kv_write(np.concatenate(K_rows), np.concatenate(V_rows), np.array(slots), kc, vc, bs, "f32")
    tables, seq_lens = al.block_table(range(len(lens)), max(-(-L // bs) for L in lens))
    qs = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), Hq, d)).astype(np.float32)
    return dict(q=q, kc=kc, vc=vc, tables=np.array(tables), lens=np.array(seq_lens), qs=qs, K=K_rows, V=V_rows)


def _run(c, scale, bs):
    return A.prefill(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], c["qs"], scale, bs, "f32", "f32")


@pytest.mark.parametrize("G", [1, 4])
def test_matches_torch_sdpa_with_causal_mask(G):
    """Each request's gathered K/V (heads repeated G times) through torch's float64 SDPA with
    the mask "new token i sees positions <= L - n + i" written out as a boolean matrix."""
    rng = np.random.default_rng(70 + G)
    Hkv, d, bs = 2, 16, 8
    Hq = Hkv * G
    lens, n_new = [5, 40, 33, 17], [5, 13, 1, 0]
    c = _case(rng, lens, n_new, Hq, Hkv, d, bs)
    scale = np.float32(1 / math.sqrt(d))
    got = _run(c, scale, bs)
    for b, (L, n) in enumerate(zip(lens, n_new)):
        if n == 0:
            continue
        Kb = torch.from_numpy(c["K"][b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        Vb = torch.from_numpy(c["V"][b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        qb = torch.from_numpy(c["q"][c["qs"][b]: c["qs"][b + 1]].astype(np.float64)).permute(1, 0, 2).contiguous()
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]        # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, Kb, Vb, attn_mask=mask, scale=float(scale))
        np.testing.assert_allclose(got[c["qs"][b]: c["qs"][b + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)


def test_single_new_token_is_decode():
    rng = np.random.default_rng(80)
    lens = [1, 7, 64, 100]
    c = _case(rng, lens, [1] * 4, 8, 2, 32, 16)
    scale = np.float32(0.2)
    got = _run(c, scale, 16)
    ref = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, 16, "f32", "f32")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_causal_later_tokens_do_not_matter():
    """Changing the K/V of positions after a new token leaves that token's output unchanged,
    and changes a later token's."""
    rng = np.random.default_rng(81)
    c = _case(rng, [30], [12], 4, 2, 8, 4)
    base = _run(c, np.float32(0.3), 4)
    blk, row = c["tables"][0][25 // 4], 25 % 4                  # position 25 = new token 7
    c["kc"][blk, :, row] += 1.0
    c["vc"][blk, :, row] -= 2.0
    moved = _run(c, np.float32(0.3), 4)
    assert np.array_equal(base[:7], moved[:7])                  # positions 18..24 do not see 25
    assert not np.allclose(base[7:], moved[7:])


def test_chunked_equals_whole():
    """A prompt prefilled in one call, or in two chunks where the second sees the first
    through the cache, gives the same outputs."""
    rng = np.random.default_rng(82)
    L, n1 = 45, 19
    c = _case(rng, [L], [L], 8, 2, 16, 8)
    whole = _run(c, np.float32(0.25), 8)
    c1 = dict(c, lens=np.array([n1]), qs=np.array([0, n1]), q=c["q"][:n1])
    c2 = dict(c, lens=np.array([L]), qs=np.array([0, L - n1]), q=c["q"][n1:])
    parts = np.concatenate([_run(c1, np.float32(0.25), 8), _run(c2, np.float32(0.25), 8)])
    np.testing.assert_array_equal(parts, whole)


def test_bruteforce_pure_python():
    """Explicit loops, math.exp, no numpy in the arithmetic."""
    rng = np.random.default_rng(83)
    lens, n_new = [6, 11], [3, 11]
    c = _case(rng, lens, n_new, 4, 2, 5, 3)
    scale = 0.37
    got = _run(c, np.float32(scale), 3)
    s32 = float(np.float32(scale))
    for b, (L, n) in enumerate(zip(lens, n_new)):
        for i in range(n):
            t = int(c["qs"][b]) + i
            for h in range(4):
                g = h // 2
                K = [[float(x) for x in c["K"][b][j, g]] for j in range(L - n + i + 1)]
                V = [[float(x) for x in c["V"][b][j, g]] for j in range(L - n + i + 1)]
                q = [float(x) for x in c["q"][t, h]]
                s = [s32 * sum(a * k for a, k in zip(q, krow)) for krow in K]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                o = [sum(e[j] * V[j][k] for j in range(len(V))) / z for k in range(5)]
                np.testing.assert_allclose(got[t, h], o, rtol=0, atol=1e-12)


def test_bf16_storage_read_exactly():
    """bf16 caches and queries are read as their exact values."""
    rng = np.random.default_rng(84)
    c = _case(rng, [20], [8], 4, 1, 8, 4)
    qb = C.f32_to_bf16_bits(c["q"])
    kb, vb = C.f32_to_bf16_bits(c["kc"]), C.f32_to_bf16_bits(c["vc"])
    got = A.prefill(qb, kb, vb, c["tables"], c["lens"], c["qs"], np.float32(0.3), 4, "bf16", "bf16")
    ref = A.prefill(C.storage_to_f64(qb, "bf16").astype(np.float32), C.storage_to_f64(kb, "bf16").astype(np.float32),
                    C.storage_to_f64(vb, "bf16").astype(np.float32), c["tables"], c["lens"], c["qs"],
                    np.float32(0.3), 4, "f32", "f32")
    np.testing.assert_array_equal(got, ref)

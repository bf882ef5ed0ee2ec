"""Pins of the float64 oracle to things other than itself (CPU only).

Each test names what it pins: a worked example the pages print (tests/golden/), a closed
form, an invariant of paging, a library routine, or brute force.  A plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand, a per-block
instead of per-request softmax) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import codecs as C
from oracle import measures as M
from oracle.allocator import Allocator

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("=")
        parts = lhs.split()
        rows.append((parts[0], [int(x) for x in parts[1:]], float(rhs)))
    return rows


# --------------------------------------------------------------------------- worked examples

def test_pages_worked_examples():
    """Every worked example printed by the pages (golden file, each line cited there)."""
    seen = set()
    for name, args, want in _golden():
        seen.add(name)
        if name == "footprint_gb_1dp":
            gb = M.footprint_bytes(*args) / 1e9
            assert f"{gb:.1f}" == f"{want:.1f}"
        elif name == "reserved_unused":
            tokens, reserve = args
            assert M.unused_slots(tokens, reserve=reserve) == want
        elif name == "blocks_unused":
            tokens, bs = args
            assert M.unused_slots(tokens, block_size=bs) == want
        elif name == "blocks_unused_max":
            bs = args[0]
            assert max(M.unused_slots(L, block_size=bs) for L in range(1, 5000)) == want
        elif name == "default_block_size":
            assert want == 16
        else:
            raise AssertionError(f"unknown golden entry {name}")
    assert {"footprint_gb_1dp", "reserved_unused", "blocks_unused", "blocks_unused_max"} <= seen


def test_footprint_exact_and_decode_bytes_agree():
    """The listing's product is 2*32*8*128*4096*16*2; the per-layer KV term of the
    algorithmic byte model times 32 layers must equal it."""
    assert M.footprint_bytes(32, 8, 128, 4096, 16, 2) == 8_589_934_592
    per_layer = M.decode_bytes([4096] * 16, 32, 8, 128, 16, kv_bytes=2, q_bytes=2, out_bytes=2)
    kv = 2 * 8 * 4096 * 128 * 2 * 16
    assert per_layer == kv + 16 * 32 * 128 * 4 + 16 * 256 * 4 + 16 * 4
    assert 32 * kv == M.footprint_bytes(32, 8, 128, 4096, 16, 2)


def test_footprint_counts_each_vector_once():
    """Each factor enters once: doubling any one of layers, heads, dims, tokens, requests or
    bytes doubles the footprint, and one layer of one head for one token of one request holds
    one K and one V vector."""
    base = (3, 5, 7, 11, 13, 2)
    f0 = M.footprint_bytes(*base)
    for i in range(6):
        args = list(base)
        args[i] *= 2
        assert M.footprint_bytes(*args) == 2 * f0
    assert M.footprint_bytes(1, 1, 128, 1, 1, 2) == 2 * 128 * 2


@pytest.mark.parametrize("bs", [8, 16, 32, 128])
def test_paged_unused_bound_bruteforce(bs):
    """Paged waste never exceeds block-1 and is zero exactly on block multiples; held slots
    are the fewest whole blocks that cover the request (brute force over block counts)."""
    for L in range(1, 20001):
        held, filled = M.slot_budget(L, block_size=bs)
        assert filled == L and held % bs == 0
        assert held >= L and held - bs < L
        w = M.unused_slots(L, block_size=bs)
        assert 0 <= w <= bs - 1
        assert (w == 0) == (L % bs == 0)


def test_slot_budget_rejects_ambiguous_or_short_placements():
    with pytest.raises(ValueError):
        M.slot_budget(10)
    with pytest.raises(ValueError):
        M.slot_budget(10, reserve=16, block_size=16)
    with pytest.raises(ValueError):
        M.slot_budget(20, reserve=16)


def test_copy_blocks_hand_worked():
    """The copy-on-write copy, by hand: two (src, dst) pairs move whole blocks, K and V both,
    from src to dst (not the other way), every head, row and dim; other blocks are untouched;
    a pair naming a block outside the pool is skipped (the library's stated contract for
    pa_copy_blocks)."""
    N, H, bs, d = 5, 2, 3, 2
    k = np.arange(N * H * bs * d, dtype=np.float32).reshape(N, H, bs, d)
    v = -k - 1
    k0, v0 = k.copy(), v.copy()
    A.copy_blocks(k, v, [(0, 3), (4, 1), (2, 5), (-1, 2)])
    # block 3 now holds block 0's K and V; block 1 holds block 4's
    assert k[3, 1, 2, 1] == 0 * 12 + 1 * 6 + 2 * 2 + 1 == k0[0, 1, 2, 1]
    assert v[3, 0, 0, 0] == -1.0
    assert k[1, 0, 1, 0] == 4 * 12 + 0 * 6 + 1 * 2 + 0 == 50
    assert v[1, 1, 2, 1] == -(4 * 12 + 1 * 6 + 2 * 2 + 1) - 1 == -60
    assert np.array_equal(k[3], k0[0]) and np.array_equal(v[3], v0[0])
    assert np.array_equal(k[1], k0[4]) and np.array_equal(v[1], v0[4])
    # sources and every other block unchanged; the out-of-range pairs wrote nothing
    for blk in (0, 2, 4):
        assert np.array_equal(k[blk], k0[blk]) and np.array_equal(v[blk], v0[blk])


def test_copy_on_write_keeps_every_sequence_readable():
    """Copy-on-write through the oracle's allocator, write and copy: a parent and a forked
    child share a partly filled block; appending to the child moves it to a fresh block, whose
    (old, new) pair copy_blocks copies before the write.  Read through their tables, both
    sequences then hold exactly their own rows (the parent's prefix in both, each one's own
    new row in its own position), and the shared block still holds only the parent's rows."""
    rng = np.random.default_rng(3)
    N, H, bs, d = 8, 2, 4, 3
    al = Allocator(N, bs, list(rng.permutation(N)))
    k = np.full((N, H, bs, d), np.nan, np.float32)
    v = np.full_like(k, np.nan)
    al.add(0)
    rows_k = rng.standard_normal((6, H, d)).astype(np.float32)
    rows_v = rng.standard_normal((6, H, d)).astype(np.float32)
    slots, cow = al.append(0, 6)
    assert not cow
    A.kv_write(rows_k, rows_v, np.array(slots), k, v, bs, "f32")
    al.fork(0, 1)
    child_k = rng.standard_normal((1, H, d)).astype(np.float32)
    child_v = rng.standard_normal((1, H, d)).astype(np.float32)
    s_child, cow = al.append(1, 1)
    assert len(cow) == 1
    A.copy_blocks(k, v, cow)
    A.kv_write(child_k, child_v, np.array(s_child), k, v, bs, "f32")
    tab, lens = al.block_table([0, 1], 4)
    for h in range(H):
        pk = A.gather(k, tab[0], lens[0], h, bs, "f32")
        ck = A.gather(k, tab[1], lens[1], h, bs, "f32")
        cv = A.gather(v, tab[1], lens[1], h, bs, "f32")
        assert np.array_equal(pk, rows_k[:, h].astype(np.float64))
        assert np.array_equal(ck[:6], rows_k[:, h].astype(np.float64))
        assert np.array_equal(ck[6], child_k[0, h].astype(np.float64))
        assert np.array_equal(cv[6], child_v[0, h].astype(np.float64))
    src, dst = cow[0]
    assert tab[0][1] == src and tab[1][1] == dst
    assert np.isnan(k[src, :, 2:]).all()       # the shared block's unfilled rows stay unwritten


# --------------------------------------------------------------------------- helpers

def _scatter_case(rng, B, Hq, Hkv, d, bs, lens, fmt="f32", permute=True, spare=3, perm_seed=99):
    """Logical K/V rows per request, written into a paged cache through the oracle's own
    allocator and write; returns everything needed for decode and for direct attention.
    Values come from rng; the physical block order from its own seed, so the same values
    can be placed in different orders."""
    K_rows, V_rows = [], []
    for L in lens:
        for rows in (K_rows, V_rows):
            x = rng.standard_normal((L, Hkv, d)).astype(np.float32)
            rows.append(C.f32_to_bf16_bits(x) if fmt == "bf16" else x)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    need = sum(-(-L // bs) for L in lens)
    N = need + spare
    order = np.random.default_rng(perm_seed).permutation(N) if permute else np.arange(N)
    al = Allocator(N, bs, order)
    slots = []
    for b, L in enumerate(lens):
        al.add(b)
        s, cow = al.append(b, L)
        assert cow == []
        slots += s
    dt = np.uint16 if fmt == "bf16" else np.float32
    kc = np.zeros((N, Hkv, bs, d), dtype=dt)
    vc = np.zeros((N, Hkv, bs, d), dtype=dt)
    A.kv_write(np.concatenate(K_rows), np.concatenate(V_rows), np.array(slots), kc, vc, bs, fmt)
    tables, seq_lens = al.block_table(range(len(lens)), max(-(-L // bs) for L in lens))
    return dict(q=q, kc=kc, vc=vc, tables=np.array(tables), lens=np.array(seq_lens),
                K=K_rows, V=V_rows)


def _direct(q, K_rows, V_rows, Hq, Hkv, scale, fmt="f32"):
    """Attention over each request's rows in logical order, with no cache and no table."""
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        for h in range(Hq):
            Kb = C.storage_to_f64(K_rows[b][:, h // G], fmt)
            Vb = C.storage_to_f64(V_rows[b][:, h // G], fmt)
            out[b, h] = A.attend(q[b, h].astype(np.float64), Kb, Vb, scale)
    return out


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("bs", [1, 3, 8, 16])
def test_paging_transparency(bs):
    """Paged decode under a random physical block order equals attention over the same
    tokens held contiguously, and equals the identity order (the page-table analogy)."""
    rng = np.random.default_rng(11 + bs)
    lens = [1, 5, 17, 33, 40]
    B, Hq, Hkv, d = len(lens), 4, 2, 8
    scale = np.float32(1 / math.sqrt(d))
    c = _scatter_case(rng, B, Hq, Hkv, d, bs, lens, permute=True)
    got = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, bs, "f32", "f32")
    want = _direct(c["q"], c["K"], c["V"], Hq, Hkv, float(scale))
    np.testing.assert_array_equal(got, want)
    # identity order: the same rows, different physical placement
    rng2 = np.random.default_rng(11 + bs)
    c2 = _scatter_case(rng2, B, Hq, Hkv, d, bs, lens, permute=False)
    assert not np.array_equal(c2["tables"], c["tables"]) or bs >= 40
    got2 = A.decode(c2["q"], c2["kc"], c2["vc"], c2["tables"], c2["lens"], scale, bs, "f32", "f32")
    np.testing.assert_array_equal(got, got2)


def test_block_size_does_not_change_attention():
    """One softmax per request: the same tokens in blocks of 1, 2, 3, 8 and 16 give the
    same output (a per-block softmax would not)."""
    outs = []
    for bs in (1, 2, 3, 8, 16):
        rng = np.random.default_rng(5)
        c = _scatter_case(rng, 3, 2, 2, 8, bs, [19, 7, 33])
        outs.append(A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"],
                             np.float32(0.3), bs, "f32", "f32"))
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=1e-13)


def test_shared_prefix_equals_private_copies():
    """Requests whose table rows point at one shared set of prefix blocks give exactly the
    outputs of the same requests holding private copies of the prefix."""
    rng = np.random.default_rng(3)
    bs, Hkv, Hq, d, P = 4, 2, 4, 8, 12
    pre_k = rng.standard_normal((P, Hkv, d)).astype(np.float32)
    pre_v = rng.standard_normal((P, Hkv, d)).astype(np.float32)
    suf = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in (3, 6, 1)]
    sufv = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in (3, 6, 1)]
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    scale = np.float32(0.35)
    N = 40
    # shared: holder writes the prefix once, forks into 3 sharers, is released
    al = Allocator(N, bs, rng.permutation(N))
    kc = np.full((N, Hkv, bs, d), np.nan, np.float32)
    vc = np.full((N, Hkv, bs, d), np.nan, np.float32)
    al.add(99)
    s, _ = al.append(99, P)
    A.kv_write(pre_k, pre_v, np.array(s), kc, vc, bs, "f32")
    for b in range(3):
        al.fork(99, b)
    al.release(99)
    assert all(r == 3 for r in [al.refcount[x] for x in al.seqs[0].blocks])
    for b in range(3):
        s, cow = al.append(b, len(suf[b]))
        assert cow == []                       # the prefix fills whole blocks
        A.kv_write(suf[b], sufv[b], np.array(s), kc, vc, bs, "f32")
    t, L = al.block_table(range(3), 8)
    shared = A.decode(q, kc, vc, np.array(t), np.array(L), scale, bs, "f32", "f32")
    # private: each request writes its own prefix copy
    al2 = Allocator(N, bs, rng.permutation(N))
    kc2 = np.full((N, Hkv, bs, d), np.nan, np.float32)
    vc2 = np.full((N, Hkv, bs, d), np.nan, np.float32)
    for b in range(3):
        al2.add(b)
        s, _ = al2.append(b, P + len(suf[b]))
        A.kv_write(np.concatenate([pre_k, suf[b]]), np.concatenate([pre_v, sufv[b]]),
                   np.array(s), kc2, vc2, bs, "f32")
    t2, L2 = al2.block_table(range(3), 8)
    private = A.decode(q, kc2, vc2, np.array(t2), np.array(L2), scale, bs, "f32", "f32")
    np.testing.assert_array_equal(shared, private)


def test_stale_slots_do_not_leak():
    """NaN in the unused tail of the last block and in unused blocks does not reach the
    output (positions >= L are never read)."""
    rng = np.random.default_rng(8)
    c = _scatter_case(rng, 2, 2, 1, 8, 16, [5, 21])
    kc, vc = c["kc"].copy(), c["vc"].copy()
    used = {(int(row[j // 16]), j % 16) for row, L in zip(c["tables"], c["lens"]) for j in range(L)}
    for blk in range(kc.shape[0]):
        for r in range(16):
            if (blk, r) not in used:
                kc[blk, :, r] = np.nan
                vc[blk, :, r] = np.inf
    got = A.decode(c["q"], kc, vc, c["tables"], c["lens"], np.float32(0.3), 16, "f32", "f32")
    assert np.isfinite(got).all()
    want = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], np.float32(0.3), 16, "f32", "f32")
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------- closed forms

def test_closed_form_two_tokens():
    """Two keys with scores a and b: o = (e^a v0 + e^b v1) / (e^a + e^b)."""
    q = np.array([0.7, -1.3, 0.2])
    K = np.array([[1.0, 0.5, -2.0], [-0.3, 0.8, 1.1]])
    V = np.array([[1.0, 2.0, 3.0], [-4.0, 5.0, 0.5]])
    scale = 0.6
    a = scale * (0.7 * 1.0 - 1.3 * 0.5 + 0.2 * -2.0)
    b = scale * (0.7 * -0.3 - 1.3 * 0.8 + 0.2 * 1.1)
    want = [(math.exp(a) * V[0, i] + math.exp(b) * V[1, i]) / (math.exp(a) + math.exp(b))
            for i in range(3)]
    np.testing.assert_allclose(A.attend(q, K, V, scale), want, rtol=1e-14, atol=1e-15)


def test_closed_forms():
    rng = np.random.default_rng(1)
    d = 16
    V = rng.standard_normal((37, d))
    K = rng.standard_normal((37, d))
    q = rng.standard_normal(d)
    # one token: the output is that token's value row
    np.testing.assert_array_equal(A.attend(q, K[:1], V[:1], 0.25), V[0])
    # all keys equal, or q = 0: uniform weights, the output is the mean of V
    Ke = np.tile(K[:1], (37, 1))
    np.testing.assert_allclose(A.attend(q, Ke, V, 0.25), V.mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(A.attend(np.zeros(d), K, V, 0.25), V.mean(0), rtol=0, atol=1e-14)
    # one score dominant by a wide margin: the output is that value row
    Kd = K * 0.01
    Kd[23] = q * 50.0
    np.testing.assert_allclose(A.attend(q, Kd, V, 1.0), V[23], rtol=0, atol=1e-12)
    # no keys: the empty sum
    assert np.all(A.attend(q, K[:0], V[:0], 1.0) == 0)


# --------------------------------------------------------------------------- library routine

@pytest.mark.parametrize("G", [1, 4])
def test_matches_torch_sdpa_float64(G):
    """Gathered contiguous K/V (heads repeated G times) through torch's scaled dot-product
    attention in float64 on the CPU agrees with the oracle."""
    rng = np.random.default_rng(21 + G)
    Hkv, d, bs = 2, 16, 8
    Hq = Hkv * G
    lens = [1, 9, 64, 77]
    c = _scatter_case(rng, len(lens), Hq, Hkv, d, bs, lens)
    scale = np.float32(1 / math.sqrt(d))
    got = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, bs, "f32", "f32")
    for b, L in enumerate(lens):
        Kb = torch.from_numpy(c["K"][b].astype(np.float64)).permute(1, 0, 2)   # [Hkv, L, d]
        Vb = torch.from_numpy(c["V"][b].astype(np.float64)).permute(1, 0, 2)
        Kb = Kb.repeat_interleave(G, dim=0).contiguous()
        Vb = Vb.repeat_interleave(G, dim=0).contiguous()
        qb = torch.from_numpy(c["q"][b].astype(np.float64))[:, None, :]      # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, Kb, Vb, scale=float(scale))
        np.testing.assert_allclose(got[b], ref[:, 0].numpy(), rtol=0, atol=1e-10)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("bs", [1, 2, 3, 16])
def test_bruteforce_pure_python(bs):
    rng = np.random.default_rng(40 + bs)
    lens = list(rng.integers(1, 41, size=3))
    c = _scatter_case(rng, 3, 4, 2, 6, bs, lens)
    scale = np.float32(0.41)
    got = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, bs, "f32", "f32")
    ref = A.decode_bruteforce(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, bs, "f32", "f32")
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-12)


def test_bruteforce_tiny_mha_workload():
    """The tiny MHA fp32 workload shape (4 requests, 8 heads, d 64, block 16)."""
    import workloads
    w = workloads.tiny_mha_f32()
    vals = workloads.host_values(w)
    al = Allocator(w.num_blocks, w.bs, w.free_order)
    slots = []
    for op in w.ops:
        if op[0] == "add":
            al.add(op[1])
        elif op[0] == "append":
            slots += al.append(op[1], op[2])[0]
    kc = np.zeros((w.num_blocks, w.Hkv, w.bs, w.d), np.float32)
    vc = np.zeros_like(kc)
    A.kv_write(vals["k_pre"], vals["v_pre"], np.array(slots), kc, vc, w.bs, "f32")
    step = [al.append(b, 1)[0][0] for b in range(w.B)]
    A.kv_write(vals["k_new"], vals["v_new"], np.array(step), kc, vc, w.bs, "f32")
    t, L = al.block_table(range(w.B), w.max_blocks)
    assert L == list(w.seq_lens)
    scale = np.float32(1 / math.sqrt(w.d))
    got = A.decode(vals["q"], kc, vc, np.array(t), np.array(L), scale, w.bs, "f32", "f32")
    ref = A.decode_bruteforce(vals["q"], kc, vc, np.array(t), np.array(L), scale, w.bs, "f32", "f32")
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- split-K algebra

@pytest.mark.parametrize("ptok", [16, 64, 512])
def test_splitk_merge_equals_single_pass(ptok):
    rng = np.random.default_rng(ptok)
    lens = [1, 15, 16, 17, 511, 513, 1300]
    c = _scatter_case(rng, len(lens), 4, 2, 8, 16, lens)
    scale = np.float32(0.33)
    a = A.decode(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, 16, "f32", "f32")
    b = A.decode_splitk(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], scale, 16, "f32", "f32",
                        partition_tokens=ptok)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- codecs

def test_fp8_write_float32_input_equals_bf16_input():
    """The oracle's fp8 write from float32 inputs gives, for values that bf16 holds exactly,
    the same codes as its write from the bf16 bit patterns of those values (same scales);
    float32 inputs between bf16 neighbours land on one of the two neighbours' codes or between
    them (the encoder is monotone)."""
    rng = np.random.default_rng(17)
    T, H, d, bs = 40, 2, 16, 8
    x32 = (rng.standard_normal((T, H, d)) * 40).astype(np.float32)
    xb = C.f32_to_bf16_bits(x32)
    x_exact = C.bf16_bits_to_f64(xb).astype(np.float32)        # the bf16 values, as float32
    scales = np.float32([0.37, 1.9])
    slots = np.arange(T)
    kb, vb = np.zeros((T // bs, H, bs, d), np.uint8), np.zeros((T // bs, H, bs, d), np.uint8)
    kf, vf = kb.copy(), vb.copy()
    A.kv_write(xb, xb, slots, kb, vb, bs, "fp8", scales, scales)
    A.kv_write(x_exact, x_exact, slots, kf, vf, bs, "fp8", scales, scales)
    assert np.array_equal(kb, kf) and np.array_equal(vb, vf)
    # unrounded float32 inputs: codes are monotone in the value, per head
    kr = np.zeros_like(kb)
    A.kv_write(x32, x32, slots, kr, kr.copy(), bs, "fp8", scales, scales)
    vals = C.e4m3_bits_to_f64(kr).transpose(0, 2, 1, 3).reshape(T, H, d)
    for h in range(H):
        order = np.argsort(x32[:, h].ravel(), kind="stable")
        assert np.all(np.diff(vals[:, h].ravel()[order]) >= 0)


def test_e4m3_decode_table_from_format():
    D = C.E4M3_DECODE
    assert D[0x00] == 0.0 and D[0x01] == 2.0 ** -9 and D[0x07] == 7 * 2.0 ** -9
    assert D[0x08] == 2.0 ** -6 and D[0x38] == 1.0 and D[0x7E] == 448.0
    assert np.isnan(D[0x7F]) and np.isnan(D[0xFF])
    assert D[0x80] == 0.0 and np.signbit(D[0x80]) and D[0xB8] == -1.0 and D[0xFE] == -448.0
    finite = D[:0x7F]
    assert np.all(np.diff(finite) > 0)          # codes 0..126 strictly increase
    # library routine: torch's float8_e4m3fn interpretation of every code
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(D))
    np.testing.assert_array_equal(t[~np.isnan(t)], D[~np.isnan(D)])


def test_e4m3_encode_vs_torch_in_range():
    """Library routine: torch's float32 -> float8_e4m3fn (round to nearest even) on a dense
    sweep of in-range values, every code midpoint and its float32 neighbours."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 2_000_000).astype(np.float32),
        (rng.standard_normal(2_000_000) * 2.0 ** rng.integers(-12, 9, 2_000_000)).astype(np.float32),
    ])
    D = C.E4M3_DECODE[:0x7F]
    mids = ((D[1:] + D[:-1]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    x = np.concatenate([x, mids, -mids, D.astype(np.float32), -D.astype(np.float32)])
    x = x[np.abs(x) <= 448]
    got = C.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_vs_exhaustive_search():
    """Brute force over all 256 codes: the nearest finite value, ties to the even code,
    saturation beyond 448, sign kept; on random values of every magnitude."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 12, 20000)).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 448, 449, 463.9, 464, 465, 1e9, np.inf, -np.inf, 2.0 ** -10, 2.0 ** -10 * 3])])
    got = C.e4m3_encode(x)
    D = C.E4M3_DECODE
    for xi, gi in zip(x, got):
        a = min(abs(float(xi)), 448.0)
        best = None
        for code in range(0x7F):
            err = abs(D[code] - a)
            if best is None or err < best[0] or (err == best[0] and code % 2 == 0):
                best = (err, code)
        want = best[1] | (0x80 if np.signbit(xi) else 0)
        assert gi == want, (xi, gi, want)
    assert C.e4m3_encode(np.float32([np.nan]))[0] & 0x7F == 0x7F


def test_e4m3_quantize_division_is_correctly_rounded():
    """float32(float64(x)/float64(s)) equals the correctly rounded float32 quotient,
    checked against exact rational arithmetic."""
    from fractions import Fraction
    rng = np.random.default_rng(2)
    xs = C.bf16_bits_to_f64(C.f32_to_bf16_bits(rng.standard_normal(3000).astype(np.float32)))
    ss = rng.uniform(1e-3, 2.0, 3000).astype(np.float32)
    for x, s in zip(xs, ss):
        q32 = np.float32(np.float64(x) / np.float64(s))
        exact = Fraction(float(x)) / Fraction(float(s))
        lo = np.nextafter(q32, np.float32(-np.inf))
        hi = np.nextafter(q32, np.float32(np.inf))
        e = abs(Fraction(float(q32)) - exact)
        assert e <= abs(Fraction(float(lo)) - exact) and e <= abs(Fraction(float(hi)) - exact)


def test_bf16_codec_vs_torch():
    """Library routine: torch's float32 -> bfloat16 (round to nearest even) on every
    exponent, random mantissas, and the tie patterns; decode is exact."""
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, 100000, dtype=np.uint64).astype(np.uint32) << 16) | np.uint32(0x8000)
    u = np.concatenate([u, ties, ties ^ np.uint32(1)])
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    got = C.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    back = C.bf16_bits_to_f64(got)
    ref_back = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(back, ref_back)
    nan_bits = C.f32_to_bf16_bits(np.float32([np.nan, -np.nan]))
    assert np.isnan(C.bf16_bits_to_f64(nan_bits)).all()


def test_fp8_decode_path_matches_dequantize():
    """fp8 cache: gather applies the per-head scale to the decoded codes."""
    rng = np.random.default_rng(4)
    bs, Hkv, d = 4, 2, 8
    N = 6
    k = C.f32_to_bf16_bits(rng.standard_normal((10, Hkv, d)).astype(np.float32))
    v = C.f32_to_bf16_bits(rng.standard_normal((10, Hkv, d)).astype(np.float32))
    ks = np.float32([0.01, 0.02])
    vs = np.float32([0.015, 0.005])
    kc = np.zeros((N, Hkv, bs, d), np.uint8)
    vc = np.zeros((N, Hkv, bs, d), np.uint8)
    slots = np.array([4, 5, 6, 7, 0, 1, 2, 3, 12, 13])    # logical order through table [1, 0, 3]
    A.kv_write(k, v, slots, kc, vc, bs, "fp8", ks, vs)
    table = [1, 0, 3]
    Kg = A.gather(kc, table, 10, 1, bs, "fp8", ks)
    kf = C.bf16_bits_to_f64(k[:, 1])
    # every row decodes to within half a code step (relative 2^-4) of the input
    np.testing.assert_allclose(Kg, kf, rtol=2.0 ** -4, atol=float(ks[1]) * 2.0 ** -10)
    assert np.array_equal(kc[1, 1, 1], C.e4m3_quantize(kf[1], ks[1]))

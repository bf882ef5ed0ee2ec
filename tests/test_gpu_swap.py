"""GPU parity of preemption by swapping: sequences are swapped out to a pinned host pool,
their freed device blocks are reused, and they are swapped back in.  Compared with the
oracle (its allocator model and numpy block copies from the same stored inputs): the pairs,
the whole host pool and the whole device cache bit for bit; and the decode of every request
after the round trip is bit-identical to its decode before (decode does not depend on
where the blocks are), and within tolerance of the oracle's attention."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_408_amd as pk
import workloads
from tests.gpu_common import (DEV, NP_DT, SENTINEL, GpuSide, OracleSide, bits, check_close, out_f64,
                              to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.name}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _pinned_sentinel(n, w):
    a = np.full((n, w.Hkv, w.bs, w.d), SENTINEL[w.fmt], dtype=NP_DT[w.fmt])
    t = torch.from_numpy(a.view(np.int16) if w.fmt == "bf16" else a).pin_memory()
    return (t.view(torch.bfloat16) if w.fmt == "bf16" else t), a.copy()


def _host_bits(t, fmt):
    return bits(t.view(torch.int16).numpy().view(np.uint16) if fmt == "bf16" else t.numpy())


def _pairs_arg(pairs, where):
    t = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2))
    return t.pin_memory() if where == "pinned" else t.to(DEV)


def swap_round_trip(w, out_ids, pairs_in="device", sample_rows=(0,)):
    vals = workloads.host_values(w)
    g, o = GpuSide(w, vals), OracleSide(w, vals)
    before = g.decode()
    nh = sum(-(-int(L) // w.bs) for L in w.seq_lens) + 3
    g.alloc.set_host_blocks(nh)
    o.alloc.set_host_blocks(nh)
    hk, ohk = _pinned_sentinel(nh, w)
    hv, ohv = _pinned_sentinel(nh, w)

    # swap out: pairs, then the host pool bit for bit (untouched host blocks keep the sentinel)
    pairs = g.alloc.swap_out(out_ids)
    opairs = o.alloc.swap_out(out_ids)
    assert [tuple(map(int, p)) for p in pairs] == opairs
    pk.pa_swap_blocks(hk, hv, g.kc, g.vc, _pairs_arg(pairs, pairs_in))
    torch.cuda.synchronize()
    for d, h in opairs:
        ohk[h], ohv[h] = o.kc[d], o.vc[d]
    assert np.array_equal(_host_bits(hk, w.fmt), bits(ohk)), "host K pool differs"
    assert np.array_equal(_host_bits(hv, w.fmt), bits(ohv)), "host V pool differs"

    # the freed device blocks are reused by someone else: overwrite them on both sides
    ref, free = g.alloc.dump()
    assert list(map(int, free)) == o.alloc.dump()[1]
    freed = [int(b) for b in free]
    if freed:
        idx = torch.tensor(freed, device=DEV)
        junk = torch.arange(len(freed) * w.Hkv * w.bs * w.d, device=DEV, dtype=torch.int32) % 97
        junk = junk.reshape(len(freed), w.Hkv, w.bs, w.d)
        g.kc[idx] = junk.to(g.kc.dtype)
        g.vc[idx] = (junk + 1).to(g.vc.dtype)
        o.kc[freed] = to_host(g.kc[idx], w.fmt)
        o.vc[freed] = to_host(g.vc[idx], w.fmt)

    # swap in: pairs, then the whole device cache bit for bit
    pairs = g.alloc.swap_in(out_ids)
    opairs = o.alloc.swap_in(out_ids)
    assert [tuple(map(int, p)) for p in pairs] == opairs
    pk.pa_swap_blocks(g.kc, g.vc, hk, hv, _pairs_arg(pairs, pairs_in))
    torch.cuda.synchronize()
    for h, d in opairs:
        o.kc[d], o.vc[d] = ohk[h], ohv[h]
    assert np.array_equal(bits(to_host(g.kc, w.fmt)), bits(o.kc)), "device K cache differs"
    assert np.array_equal(bits(to_host(g.vc, w.fmt)), bits(o.vc)), "device V cache differs"

    # every request decodes exactly as before the round trip, through its new table
    tab, lens = g.alloc.block_tables(list(range(w.B)), max(w.max_blocks, 1))
    otab, olens = o.alloc.block_table(range(w.B), max(w.max_blocks, 1))
    assert tab.tolist() == otab and lens.tolist() == olens
    after = g.decode(tables=torch.from_numpy(tab).to(DEV))
    assert torch.equal(after.view(torch.int16) if after.dtype == torch.bfloat16 else after.view(torch.int32),
                       before.view(torch.int16) if before.dtype == torch.bfloat16 else before.view(torch.int32))
    o.tables = np.array(otab, dtype=np.int64)
    rows = list(sample_rows)
    ref = o.decode(rows=rows)
    print(check_close(out_f64(after)[rows], ref[rows], w.fmt, f"{w.name} after swap"), flush=True)
    return g, o


def small_ragged(bs=16, fmt="bf16"):
    return workloads.ragged_prefix(bs=bs, fmt=fmt, B=24, n_shared=8, prefix=128, spare_blocks=16,
                                   name=f"ragged24_bs{bs}_{fmt}")


@pytest.mark.parametrize("bs,fmt", [(16, "bf16"), (8, "fp8"), (32, "bf16"), (128, "fp8")])
def test_swap_partial_sharers_and_private(bs, fmt):
    """Swap out three of the eight prefix sharers (the prefix blocks stay on the device for
    the other five and are copied) and four private requests."""
    w = small_ragged(bs, fmt)
    swap_round_trip(w, [0, 3, 5, 9, 12, 17, 23], sample_rows=(0, 12))


def test_swap_all_sharers_maps_prefix_once():
    """Swap out all eight sharers: each prefix block goes to one host block holding all eight
    references, and the device blocks are freed."""
    w = small_ragged(16, "bf16")
    g, o = swap_round_trip(w, list(range(8)), pairs_in="pinned", sample_rows=(1,))
    ref, _ = g.alloc.dump()
    tab, _ = g.alloc.block_tables(list(range(8)), w.max_blocks)
    prefix_blocks = tab[0, : 128 // 16]
    assert (tab[:8, : 128 // 16] == prefix_blocks).all()
    assert all(int(ref[b]) == 8 for b in prefix_blocks)


def test_swap_f32_mha():
    w = workloads.tiny_mha_f32()
    swap_round_trip(w, [1, 3], sample_rows=(1, 3))


def test_swap_d64_gqa():
    w = workloads.gqa_uniform(B=3, L=300, Hq=16, Hkv=2, d=64, bs=16, fmt="bf16", layers=1, name="d64_swap")
    swap_round_trip(w, [0, 2], sample_rows=(2,))


def test_swap_blocks_checks_pointers():
    """Pageable host memory and ranges past an allocation are refused before any launch; the
    library leaves no error behind for the next call."""
    lib = pk.load()
    dev_pool = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    pinned = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16).pin_memory()
    pageable = np.zeros((4, 2, 16, 64), dtype=np.uint16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int64, device=DEV)
    P = ctypes.c_void_p
    args = lambda dst, n_dst: (P(dst), P(dst), P(dev_pool.data_ptr()), P(dev_pool.data_ptr()), P(pairs.data_ptr()),
                               1, 4, n_dst, 2, 64, 16, pk.PA_DTYPE_BF16, None)
    rc = lib.pa_swap_blocks(*args(pageable.ctypes.data, 4))
    assert rc == -1, rc
    print(lib.pa_last_error().decode(), flush=True)
    rc = lib.pa_swap_blocks(*args(pinned.data_ptr(), 1 << 24))      # 64 GiB: past the 16 KiB tensor
    assert rc == -1, rc
    print(lib.pa_last_error().decode(), flush=True)
    assert lib.pa_swap_blocks(*args(pinned.data_ptr(), 0)) == -1     # bad size
    with pytest.raises(ValueError):
        pk.pa_swap_blocks(torch.from_numpy(pageable).view(torch.bfloat16), pinned, dev_pool, dev_pool, pairs)
    # a valid call right after the refusals
    dev_pool[0] = 1.5
    pk.pa_swap_blocks(pinned, pinned, dev_pool, dev_pool, pairs)
    torch.cuda.synchronize()
    assert (pinned[1] == 1.5).all() and (pinned[0] == 0).all()
    pk.pa_swap_blocks(pinned, pinned, dev_pool, dev_pool, pairs[:0])   # no pairs: nothing to do

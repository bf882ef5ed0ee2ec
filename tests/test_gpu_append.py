"""pa_decode_append (each request's new token written through its table inside the decode
launch) against the two calls it replaces, pa_kv_write of the step's slots followed by
pa_decode, on the same inputs: the whole K and V caches byte for byte and every output bit for
bit, for every cache type, head dim, block size and group size, on the uniform grid and on the
compact item list; plus the float64 oracle on the result."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_408_amd as pk
import workloads
from oracle import attention as OA
from tests.gpu_common import DEV, OracleSide, check_close, out_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.name}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _caches(w):
    """Caches filled with a NaN pattern (stale slots must not matter)."""
    if w.fmt == "mxfp4":
        kc = pk.mxfp4_cache(w.num_blocks, w.Hkv, w.bs, w.d, DEV)
        kc.fill_(0xFF)
        return kc, kc.clone()
    if w.fmt == "fp8":
        kc = torch.full((w.num_blocks, w.Hkv, w.bs, w.d), 0x7F, dtype=torch.uint8, device=DEV)
        return kc, kc.clone()
    kc = torch.full((w.num_blocks, w.Hkv, w.bs, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    return kc, kc.clone()


def run_both(w, partition_tokens=0, edit=None):
    vals = workloads.host_values(w)
    alloc = pk.Allocator(w.num_blocks, w.bs, w.free_order)
    slots = []
    for op in w.ops:
        if op[0] == "add":
            alloc.add(op[1])
        elif op[0] == "append":
            slots.append(alloc.append(op[1], op[2])[0])
        elif op[0] == "fork":
            alloc.fork(op[1], op[2])
        elif op[0] == "free":
            alloc.free(op[1])
    kc, vc = _caches(w)
    ks = vs = None
    if w.fmt == "fp8":
        ks, vs = torch.from_numpy(vals["k_scale"]).to(DEV), torch.from_numpy(vals["v_scale"]).to(DEV)
    if slots:
        pk.pa_kv_write(to_dev(vals["k_pre"], "bf16"), to_dev(vals["v_pre"], "bf16"),
                       torch.from_numpy(np.concatenate(slots)).to(DEV), kc, vc, k_scale=ks, v_scale=vs)
    step, cow = alloc.batch_append(list(range(w.B)), [1] * w.B)
    assert not cow
    tab, lens = alloc.block_tables(list(range(w.B)), w.max_blocks)
    if edit is not None:          # the test's changes to the tables, lengths and slots
        edit(tab, lens, step)
    tables, lens_d = torch.from_numpy(tab).to(DEV), torch.from_numpy(lens).to(DEV)
    kn, vn = to_dev(vals["k_new"], "bf16"), to_dev(vals["v_new"], "bf16")
    q = to_dev(vals["q"], "bf16")
    scale = 1.0 / math.sqrt(w.d)
    maxL = int(lens.max())
    # two calls
    kA, vA = kc.clone(), vc.clone()
    pk.pa_kv_write(kn, vn, torch.from_numpy(step).to(DEV), kA, vA, k_scale=ks, v_scale=vs)
    outA = torch.empty_like(q)
    pk.pa_decode(outA, q, kA, vA, tables, lens_d, scale, w.bs, max_seq_len=maxL, k_scale=ks, v_scale=vs,
                 partition_tokens=partition_tokens)
    # one call
    kB, vB = kc.clone(), vc.clone()
    outB = torch.empty_like(q)
    pk.pa_decode_append(outB, q, kn, vn, kB, vB, tables, lens_d, scale, w.bs, max_seq_len=maxL, k_scale=ks,
                        v_scale=vs, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert torch.equal(kA.view(torch.uint8), kB.view(torch.uint8)), "K cache differs from pa_kv_write's"
    assert torch.equal(vA.view(torch.uint8), vB.view(torch.uint8)), "V cache differs from pa_kv_write's"
    assert torch.equal(outA.view(torch.int16), outB.view(torch.int16)), "output differs from pa_decode's"
    return w, vals, outB


def _small(fmt, d, bs, G, B=6, Hkv=2, name="append"):
    lens = np.array([1, bs, bs + 1, 300, 777, 1200][:B])
    n = int(sum(-(-int(L) // bs) for L in lens)) + 3
    ops = []
    for b, L in enumerate(lens):
        ops += [("add", b)] + ([("append", b, int(L) - 1)] if L > 1 else [])
    return workloads.Workload(f"{name}_{fmt}_d{d}_bs{bs}_G{G}", B=len(lens), Hq=Hkv * G, Hkv=Hkv, d=d, bs=bs,
                              fmt=fmt, q_fmt="bf16", std=0.5, seq_lens=lens, num_blocks=n,
                              free_order=np.random.default_rng(bs * G + d).permutation(n).astype(np.int32),
                              ops=ops, seed_index=62)


@pytest.mark.parametrize("fmt,d,bs,G", [
    (f, d, bs, G) for f in ("bf16", "fp8", "mxfp4") for d in (64, 128) for bs in (8, 16, 32, 128) for G in (1, 4, 8)
])
def test_append_equals_write_then_decode(fmt, d, bs, G):
    """Small ragged batch on the uniform grid, 128-token partitions (the new token sits in a
    request's last partition, whose work-group writes it)."""
    run_both(_small(fmt, d, bs, G), partition_tokens=128)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("bs", [8, 16, 128])
def test_append_item_list(fmt, bs):
    """100 requests with a shared prefix: more items than resident work-groups, so the compact
    item list (two-wave work-groups, automatic 512-token partitions) runs the appends."""
    run_both(workloads.ragged_prefix(bs=bs, fmt=fmt, B=100, n_shared=10, seed_index=63, name=f"append_list_{fmt}_{bs}"))


def test_append_llama_layer_against_oracle():
    """One Llama-3-8B-shaped layer at 4096 tokens, automatic partitions (2 per request and KV
    head), the benchmark's fused step: identical to the two calls, and within the bf16
    tolerance of the oracle on sampled requests."""
    w, vals, out = run_both(workloads.gqa_uniform(B=16, L=4096, layers=1, seed_index=64, name="append_llama"))
    o = OracleSide(w, vals)
    rows = [0, 7, 15]
    print(check_close(out_f64(out)[rows], o.decode(rows)[rows], "bf16", w.name), flush=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_append_empty_request_and_out_of_pool_entry(fmt):
    """Request 0 has length 0 (no new token: its slot is -1 for the write), and request 2's
    table entry at its new token's position lies outside the pool (its slot too, which the
    write skips).  The caches equal pa_kv_write's and the outputs pa_decode's, bit for bit;
    request 0's output is zeros, request 2's NaN, and the others are finite."""
    w = _small(fmt, 128, 16, 4)

    def edit(tab, lens, step):
        lens[0] = 0
        step[0] = -1
        e = (int(lens[2]) - 1) // w.bs
        tab[2, e] = w.num_blocks + 5
        step[2] = int(tab[2, e]) * w.bs + (int(lens[2]) - 1) % w.bs     # outside the pool: skipped

    w, vals, out = run_both(w, partition_tokens=128, edit=edit)
    o = out.float().cpu()
    assert torch.all(o[0] == 0.0), "an empty request decodes to zeros"
    assert torch.all(torch.isnan(o[2])), "an out-of-pool entry in the live range gives NaN"
    assert torch.all(torch.isfinite(o[[1, 3, 4, 5]]))


def test_append_refuses_float32_and_null_rows():
    lib = pk.load()
    assert lib.pa_decode_append(None, None, None, None, None, None, None, None, 1.0, 16, 1, 8, 8, 64, 10, 4, 64,
                                pk.PA_DTYPE_F32, pk.PA_DTYPE_F32, None, None, None, 0, 0, None) == pk._lib.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_append(None, None, None, None, None, None, None, None, 1.0, 16, 1, 8, 8, 64, 10, 4, 64,
                                pk.PA_DTYPE_BF16, pk.PA_DTYPE_BF16, None, None, None, 0, 0, None) == pk._lib.PA_ERR_INVALID

"""Decode steps replayed from HIP graphs.

The per-layer K/V writes and decodes of one generation step are captured once (prepared
launchers on a capture stream) and replayed for several steps on the same buffers, whose
contents -- block tables, lengths, slots, the new tokens' K/V and q -- the host refreshes
between replays, as a serving loop does.  Every replay is checked against:
 - the same step launched eagerly on a second pair of caches: outputs and caches bit for bit;
 - the float64 oracle (its allocator, numpy writes and attention): outputs within the bf16
   tolerance, caches bit for bit.
Covers the bf16 path (direct-to-LDS stages) and the fp8 and 4-bit ones (widened tiles)."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_408_amd as pk
import workloads
from oracle import attention as OA
from oracle.allocator import Allocator as OAlloc
from tests.gpu_common import BF16_ATOL, BF16_RTOL, DEV, NP_DT, SENTINEL, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.name}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


B, HQ, HKV, D, BS, LAYERS, STEPS = 3, 8, 2, 128, 16, 2, 4
L0 = [37, 200, 515]                 # cached tokens per request before the first step


def _caches(fmt, nb):
    if fmt == "mxfp4":
        return (pk.mxfp4_cache(nb, HKV, BS, D, DEV), pk.mxfp4_cache(nb, HKV, BS, D, DEV),
                np.zeros((nb, HKV, BS * pk.mx_row_bytes(D)), np.uint8), np.zeros((nb, HKV, BS * pk.mx_row_bytes(D)), np.uint8))
    o = np.full((nb, HKV, BS, D), SENTINEL[fmt], NP_DT[fmt])
    return to_dev(o, fmt), to_dev(o, fmt), o.copy(), o.copy()


def _host_cache(t, fmt, like):
    return t.cpu().numpy().reshape(like.shape) if fmt == "mxfp4" else to_host(t, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_graph_replay_matches_eager_and_oracle(fmt):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([408_700, ["bf16", "fp8", "mxfp4"].index(fmt)])))
    nb = sum(-(-(L + STEPS) // BS) for L in L0) + 8
    free_order = g.permutation(nb).astype(np.int32)
    T0 = sum(L0)
    # every K/V row the run writes, per layer: the prefix, then one token per request per step
    kpre = [workloads.normal_storage(g, (T0, HKV, D), 0.5, "bf16") for _ in range(LAYERS)]
    vpre = [workloads.normal_storage(g, (T0, HKV, D), 0.5, "bf16") for _ in range(LAYERS)]
    knew = [[workloads.normal_storage(g, (B, HKV, D), 0.5, "bf16") for _ in range(LAYERS)] for _ in range(STEPS)]
    vnew = [[workloads.normal_storage(g, (B, HKV, D), 0.5, "bf16") for _ in range(LAYERS)] for _ in range(STEPS)]
    qs = [[workloads.normal_storage(g, (B, HQ, D), 0.5, "bf16") for _ in range(LAYERS)] for _ in range(STEPS)]
    scales = [[None, None] for _ in range(LAYERS)]
    if fmt == "fp8":                     # per head: max |x| over everything written / 448
        for l in range(LAYERS):
            for j, (pre, new) in enumerate(((kpre[l], [s[l] for s in knew]), (vpre[l], [s[l] for s in vnew]))):
                allv = np.concatenate([pre] + new).view(np.uint16).astype(np.uint32) << 16
                amax = np.abs(allv.view(np.float32)).max(axis=(0, 2))
                scales[l][j] = (amax / np.float32(448.0)).astype(np.float32)
    sc_dev = [[None if s is None else torch.from_numpy(s).to(DEV) for s in pair] for pair in scales]

    # allocators: the library's and the oracle's take the same decisions
    al, oal = pk.Allocator(nb, BS, free_order), OAlloc(nb, BS, free_order)
    pre_slots = []
    for b in range(B):
        al.add(b)
        oal.add(b)
        s, cow = al.append(b, L0[b])
        os_, ocow = oal.append(b, L0[b])
        assert list(s) == os_ and not cow and not ocow
        pre_slots += os_
    pre_slots = np.asarray(pre_slots, np.int64)
    caches = [_caches(fmt, nb) for _ in range(LAYERS)]          # (graph k, graph v, oracle k, oracle v)
    eager = [_caches(fmt, nb)[:2] for _ in range(LAYERS)]
    for l in range(LAYERS):
        kp, vp = to_dev(kpre[l], "bf16"), to_dev(vpre[l], "bf16")
        sl = torch.from_numpy(pre_slots).to(DEV)
        for kc, vc in (caches[l][:2], eager[l]):
            pk.pa_kv_write(kp, vp, sl, kc, vc, k_scale=sc_dev[l][0], v_scale=sc_dev[l][1])
        OA.kv_write(kpre[l], vpre[l], pre_slots, caches[l][2], caches[l][3], BS, fmt, scales[l][0], scales[l][1])

    # the buffers the graph holds
    max_blocks = -(-(max(L0) + STEPS) // BS)
    max_seq = max_blocks * BS
    tables_d = torch.full((B, max_blocks), -1, dtype=torch.int32, device=DEV)
    lens_d = torch.zeros((B,), dtype=torch.int32, device=DEV)
    slot_d = torch.zeros((B,), dtype=torch.int64, device=DEV)
    kn = [torch.empty((B, HKV, D), dtype=torch.bfloat16, device=DEV) for _ in range(LAYERS)]
    vn = [torch.empty_like(kn[0]) for _ in range(LAYERS)]
    q = [torch.empty((B, HQ, D), dtype=torch.bfloat16, device=DEV) for _ in range(LAYERS)]
    out = [torch.empty_like(q[0]) for _ in range(LAYERS)]
    out_e = [torch.empty_like(q[0]) for _ in range(LAYERS)]
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(max(pk.pa_decode_workspace_bytes(B, HQ, HKV, D, max_seq, 0, BS, caches[0][0]), 256),
                     dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws)
    pk.pa_decode_workspace_init(ws)
    pk.pa_decode_workspace_init(ws_e)
    torch.cuda.synchronize()

    cap = torch.cuda.Stream()
    wr = [pk.PreparedKVWrite(kn[l], vn[l], slot_d, caches[l][0], caches[l][1], k_scale=sc_dev[l][0],
                             v_scale=sc_dev[l][1], stream=cap) for l in range(LAYERS)]
    dec = [pk.PreparedDecode(out[l], q[l], caches[l][0], caches[l][1], tables_d, lens_d, scale, BS,
                             max_seq_len=max_seq, workspace=ws, k_scale=sc_dev[l][0], v_scale=sc_dev[l][1],
                             stream=cap) for l in range(LAYERS)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap, capture_error_mode="thread_local"):
        for l in range(LAYERS):
            wr[l]()
        for l in range(LAYERS):
            dec[l]()
    torch.cuda.synchronize()

    for st in range(STEPS):
        slots = al.batch_append(list(range(B)), [1] * B)
        oslots = [oal.append(b, 1)[0][0] for b in range(B)]
        assert list(slots[0]) == oslots and not slots[1]
        tab, lens = al.block_tables(list(range(B)), max_blocks)
        otab, olens = oal.block_table(range(B), max_blocks)
        assert np.array_equal(tab, np.array(otab)) and list(lens) == olens
        # the host's own work between replays: new contents for every captured buffer
        tables_d.copy_(torch.from_numpy(tab))
        lens_d.copy_(torch.from_numpy(lens))
        slot_d.copy_(torch.from_numpy(np.asarray(slots[0], np.int64)))
        for l in range(LAYERS):
            kn[l].copy_(to_dev(knew[st][l], "bf16"))
            vn[l].copy_(to_dev(vnew[st][l], "bf16"))
            q[l].copy_(to_dev(qs[st][l], "bf16"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(LAYERS):          # the same step, launched eagerly on the second caches
            pk.pa_kv_write(kn[l], vn[l], slot_d, eager[l][0], eager[l][1], k_scale=sc_dev[l][0], v_scale=sc_dev[l][1])
            pk.pa_decode(out_e[l], q[l], eager[l][0], eager[l][1], tables_d, lens_d, scale, BS, max_seq_len=max_seq,
                         workspace=ws_e, k_scale=sc_dev[l][0], v_scale=sc_dev[l][1])
        torch.cuda.synchronize()
        for l in range(LAYERS):
            kc, vc, okc, ovc = caches[l]
            OA.kv_write(knew[st][l], vnew[st][l], np.asarray(oslots, np.int64), okc, ovc, BS, fmt,
                        scales[l][0], scales[l][1])
            assert torch.equal(out[l].view(torch.int16), out_e[l].view(torch.int16)), (st, l, "graph vs eager output")
            for a, e, o in ((kc, eager[l][0], okc), (vc, eager[l][1], ovc)):
                ha = _host_cache(a, fmt, o)
                assert np.array_equal(ha, _host_cache(e, fmt, o)), (st, l, "graph vs eager cache")
                assert np.array_equal(ha, o), (st, l, "cache vs oracle")
            ref = OA.decode(qs[st][l], okc, ovc, np.array(otab), np.array(olens), np.float32(scale), BS, fmt, "bf16",
                            scales[l][0], scales[l][1])
            got = out[l].float().cpu().numpy().astype(np.float64)
            err = np.abs(got - ref)
            bad = int((err > BF16_ATOL + BF16_RTOL * np.abs(ref)).sum())
            print(f"  step {st} layer {l} ({fmt}): lengths {list(lens)}, {bad} of {got.size} outside tolerance, "
                  f"max abs err {err.max():.3e}", flush=True)
            assert bad == 0

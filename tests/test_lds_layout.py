"""Bank-conflict check of the kernels' LDS tile layouts (CPU only).

The slot tables come from the kernels' own functions (pa_layout.h), printed by a host program
built with hipcc; the access patterns below are the kernels' LDS instructions, lane by lane.
The phase model is the one measured on gfx950 with the LDS bank-conflict counter (a probe of
lane pairs, then of full-wave patterns, among them every pattern checked here, whose counts the
model reproduced exactly):
  - 8-byte reads (ds_read_b64_tr_b16): lanes 0-31, then 32-63; 64 banks of 4 bytes;
  - 16-byte reads (ds_read_b128): 16 lanes at a time -- in each 32-lane half, the lane quads
    whose index (lane / 4) % 8 has even bit parity, then the odd ones; 64 banks;
  - 16-byte writes (ds_write_b128): 8 consecutive lanes at a time, colliding on chunks equal
    modulo 128 bytes.
Two lanes of one phase collide when they touch one bank at different words."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def tables(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("lds") / "lds_layout_dump")
    subprocess.run([HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O1", "-o", exe,
                    os.path.join(HERE, "lds_layout_dump.cpp")], check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    t = {"vt": {}, "dm": {}, "pf": {}}
    for line in out.splitlines():
        f = line.split()
        D, r = int(f[1]), int(f[2])
        t[f[0]][(D, r)] = [int(x) for x in f[3:]] if f[0] != "pf" else int(f[3])
    return t


def _phases(kind):
    if kind == "read8":
        return [list(range(0, 32)), list(range(32, 64))], 256
    if kind == "read16":
        ph = []
        for half in (0, 32):
            for par in (0, 1):
                ph.append([half + l for l in range(32) if bin((l >> 2) & 7).count("1") % 2 == par])
        return ph, 256
    assert kind == "write16"
    return [list(range(s, s + 8)) for s in range(0, 64, 8)], 128


def conflicts(addrs, kind):
    """Phases of one instruction (64 lane addresses) in which two lanes touch one bank at
    different words."""
    nbytes = 8 if kind == "read8" else 16
    phases, window = _phases(kind)
    bad = []
    for ph in phases:
        banks = {}
        for l in ph:
            for word in range(addrs[l] // 4, (addrs[l] + nbytes) // 4):
                banks.setdefault(word % (window // 4), set()).add(word)
        if any(len(words) > 1 for words in banks.values()):
            bad.append(ph[0])
    return bad


# ---- the kernels' access patterns (rowb = bytes per bf16 tile row; slot(row, chunk))
def decode_transpose_reads(D, slot):
    """V^T operand of the 16x16x16 products: lane l reads 8 bytes of row 4 (l / 16) + (l % 16) / 4,
    chunk 2 t + (l % 4) / 2, one instruction per 16 dims."""
    rowb = 2 * D
    return [[(4 * (l // 16) + (l % 16) // 4) * rowb + 16 * slot(4 * (l // 16) + (l % 16) // 4, 2 * t + ((l & 3) >> 1))
             + 8 * (l & 1) for l in range(64)] for t in range(D // 16)]


def decode_mx_writes(D, slot):
    """4-bit tile widened into LDS: lane l converts 8 dims per instruction wi into row l / 4,
    chunk NW (l % 4) + wi (NW = D / 32)."""
    rowb, nw = 2 * D, D // 32
    return [[(l >> 2) * rowb + 16 * slot(l >> 2, nw * (l & 3) + wi) for l in range(64)] for wi in range(nw)]


def decode_fp8_writes(D, slot):
    """fp8 tile widened into LDS: 16 fp8 bytes per lane (row ci / CPR, fp8 chunk ci % CPR,
    ci = 64 r + l) become bf16 chunks 2 c and 2 c + 1, one instruction each."""
    rowb, cpr = 2 * D, D // 16
    out = []
    for r in range(16 * cpr // 64):
        for h in range(2):
            out.append([((64 * r + l) // cpr) * rowb + 16 * slot((64 * r + l) // cpr, 2 * ((64 * r + l) % cpr) + h)
                        for l in range(64)])
    return out


def decode_k_reads(D, slot):
    """K operand read from the bf16 stage: lane l reads 16 bytes of row l % 16, chunk 4 j + l / 16."""
    rowb = 2 * D
    return [[(l % 16) * rowb + 16 * slot(l % 16, 4 * j + l // 16) for l in range(64)] for j in range(D // 32)]


@pytest.mark.parametrize("D", [64, 128])
def test_decode_v_tile(tables, D):
    vt = tables["vt"]
    slot = lambda r, c: vt[(D, r)][c]
    for r in range(64):                                 # a permutation of the row's chunks
        assert sorted(vt[(D, r)]) == list(range(D // 8))
    for i, a in enumerate(decode_transpose_reads(D, slot)):
        assert conflicts(a, "read8") == [], ("transpose read", i)
    for i, a in enumerate(decode_mx_writes(D, slot)):
        assert conflicts(a, "write16") == [], ("4-bit write", i)
    for i, a in enumerate(decode_fp8_writes(D, slot)):
        assert conflicts(a, "write16") == [], ("fp8 write", i)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_bf16_stage(tables, D):
    dm = tables["dm"]
    slot = lambda r, c: dm[(D, r)][c]
    for r in range(64):                                 # an involution on the row's chunks
        assert sorted(dm[(D, r)]) == list(range(D // 8))
        assert all(slot(r, slot(r, c)) == c for c in range(D // 8))
    for i, a in enumerate(decode_k_reads(D, slot)):
        assert conflicts(a, "read16") == [], ("K read", i)
    for i, a in enumerate(decode_transpose_reads(D, slot)):
        assert conflicts(a, "read8") == [], ("transpose read", i)


def test_model_flags_conflicting_layouts():
    """The layouts these replaced, which the counter showed conflicting: the bf16 stage with mask
    row % 16 (2 extra cycles per transpose read), the widened V tile without the bit-3 flip and
    the prefill widening without the per-lane order (8 extra cycles per 16-byte write)."""
    old_stage = lambda r, c: c ^ (r % 16)
    assert all(len(conflicts(a, "read8")) == 2 for a in decode_transpose_reads(128, old_stage))
    assert all(conflicts(a, "read16") == [] for a in decode_k_reads(128, old_stage))
    # a mask that suits the transpose reads but not the 16-byte read phases
    half = lambda r, c: c ^ (2 * (r & 7) | ((r >> 3) & 1))
    assert all(conflicts(a, "read8") == [] for a in decode_transpose_reads(128, half))
    assert all(len(conflicts(a, "read16")) == 4 for a in decode_k_reads(128, half))
    old_vt = lambda r, c: c ^ ((2 * (r & 7)) ^ ((r ^ (r >> 1)) & 1))
    assert all(len(conflicts(a, "write16")) == 8 for a in decode_mx_writes(128, old_vt))
    assert all(len(conflicts(a, "write16")) == 8 for a in decode_fp8_writes(128, old_vt))
    assert all(conflicts(a, "read8") == [] for a in decode_transpose_reads(128, old_vt))
    swz = lambda r: ((r & 3) << 2) | ((r >> 2) & 3)
    assert all(len(conflicts(a, "write16")) == 8 for a in prefill_widened_writes(128, swz, lambda row, q: row & 1))


def prefill_widened_writes(D, swz, swap):
    """fp8 / 4-bit tiles widened into LDS: lane l of wave w writes row 8 w + l / 8, NC = D / 64
    chunks NC (l % 8) + c; with NC = 2 a lane with swap(row, l % 8) writes its second chunk first."""
    rowb, nc = 2 * D, D // 64
    out = []
    for w in range(8):
        for i in range(nc):
            a = []
            for l in range(64):
                row, q = 8 * w + l // 8, l % 8
                c = (1 - i if swap(row, q) else i) if nc == 2 else i
                a.append(row * rowb + 16 * ((nc * q + c) ^ swz(row)))
            out.append(a)
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_kv_tile(tables, D):
    pf = tables["pf"]
    rowb = 2 * D
    slot = lambda r, c: c ^ pf[(D, r)]
    for r in range(64):
        assert 0 <= pf[(D, r)] < D // 8
    # K operand reads: lane l reads 16 bytes of row 32 sb + l % 32, chunk 2 j + l / 32
    for sb in range(2):
        for j in range(D // 16):
            addrs = [(32 * sb + l % 32) * rowb + 16 * slot(32 * sb + l % 32, 2 * j + l // 32) for l in range(64)]
            assert conflicts(addrs, "read16") == [], ("K read", sb, j)
    # V transpose reads: row 32 sb + 16 h + 4 (l / 32) + (l % 16) / 4 (+ 8), chunk 4 t + 2 ((l / 16) % 2) + (l % 4) / 2
    for sb in range(2):
        for h in range(2):
            for rd in range(2):
                for t in range(D // 32):
                    addrs = []
                    for l in range(64):
                        row = 32 * sb + 16 * h + 4 * (l // 32) + (l % 16) // 4 + 8 * rd
                        c = 4 * t + 2 * ((l >> 4) & 1) + ((l & 3) >> 1)
                        addrs.append(row * rowb + 16 * slot(row, c) + 8 * (l & 1))
                    assert conflicts(addrs, "read8") == [], ("V read", sb, h, rd, t)
    # widened fp8 / 4-bit tiles: the kernel's order (lanes 4..7 of a row, or odd rows, but not
    # both, write their second chunk first)
    for i, a in enumerate(prefill_widened_writes(D, lambda r: pf[(D, r)], lambda row, q: (row ^ (q >> 2)) & 1)):
        assert conflicts(a, "write16") == [], ("widened write", i)

"""Bank-conflict check of the kernels' LDS tile layouts (CPU only).

The slot tables come from the kernels' own functions (pa_layout.h), printed by a host program
built with hipcc; the access patterns below are the kernels' LDS instructions, lane by lane.
LDS has 64 banks of 4 bytes.  An instruction is checked in phases of 8, 16 and 32 lanes (no
phase may touch one bank at two different words; the 32-lane phase only where 32 lanes fit in
one pass of 256 bytes)."""

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
    vt, pf = {}, {}
    for line in out.splitlines():
        f = line.split()
        D, r = int(f[1]), int(f[2])
        if f[0] == "vt":
            vt[(D, r)] = [int(x) for x in f[3:]]
        else:
            pf[(D, r)] = int(f[3])
    return vt, pf


def conflicts(addrs, nbytes, phases):
    """Phases (first lane, width) in which two lanes touch one bank at different words."""
    bad = []
    for ph in phases:
        for p0 in range(0, len(addrs), ph):
            banks = {}
            for a in addrs[p0:p0 + ph]:
                for word in range(a // 4, (a + nbytes) // 4):
                    banks.setdefault(word % 64, set()).add(word)
            if any(len(words) > 1 for words in banks.values()):
                bad.append((p0, ph))
    return bad


@pytest.mark.parametrize("D", [64, 128])
def test_decode_v_tile(tables, D):
    vt, _ = tables
    rowb = 2 * D                                        # bf16 row bytes
    slot = lambda r, c: vt[(D, r)][c]
    for r in range(64):                                 # a permutation of the row's chunks
        assert sorted(vt[(D, r)]) == list(range(D // 8))
    # transpose reads: lane l reads 8 bytes of row 4 (l / 16) + (l % 16) / 4, chunk 2 t + (l % 4) / 2
    for t in range(D // 16):
        addrs = [(4 * (l // 16) + (l % 16) // 4) * rowb + 16 * slot(4 * (l // 16) + (l % 16) // 4, 2 * t + ((l & 3) >> 1))
                 + 8 * (l & 1) for l in range(64)]
        assert conflicts(addrs, 8, (16, 32)) == [], ("transpose read", t)
    # 4-bit tile writes: lane l converts 8 dims per instruction wi into row l / 4, chunk NW (l % 4) + wi
    nw = D // 32
    for wi in range(nw):
        addrs = [(l >> 2) * rowb + 16 * slot(l >> 2, nw * (l & 3) + wi) for l in range(64)]
        assert conflicts(addrs, 16, (8, 16)) == [], ("4-bit write", wi)
    # fp8 tile writes: 16 fp8 bytes per lane (row ci / CPR, fp8 chunk ci % CPR) -> bf16 chunks 2c, 2c + 1
    cpr = D // 16
    for r in range(16 * cpr // 64):
        for h in range(2):
            addrs = []
            for l in range(64):
                ci = 64 * r + l
                addrs.append((ci // cpr) * rowb + 16 * slot(ci // cpr, 2 * (ci % cpr) + h))
            assert conflicts(addrs, 16, (8, 16)) == [], ("fp8 write", r, h)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_kv_tile(tables, D):
    _, pf = tables
    rowb = 2 * D
    cpr = D // 8
    slot = lambda r, c: c ^ pf[(D, r)]
    for r in range(64):
        assert 0 <= pf[(D, r)] < cpr
    # K operand reads: lane l reads 16 bytes of row 32 sb + l % 32, chunk 2 j + l / 32
    for sb in range(2):
        for j in range(D // 16):
            addrs = [(32 * sb + l % 32) * rowb + 16 * slot(32 * sb + l % 32, 2 * j + l // 32) for l in range(64)]
            assert conflicts(addrs, 16, (8, 16)) == [], ("K read", sb, j)
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
                    assert conflicts(addrs, 8, (16, 32)) == [], ("V read", sb, h, rd, t)
    # fp8 / 4-bit tiles widened into LDS: lane l of wave w writes row 8 w + l / 8, NC = D / 64
    # chunks NC (l % 8) + c; with NC = 2 an odd row writes its second chunk first
    nc = D // 64
    for w in range(8):
        for i in range(nc):
            addrs = []
            for l in range(64):
                row, qcf = 8 * w + l // 8, l % 8
                c = (1 - i if row & 1 else i) if nc == 2 else i
                addrs.append(row * rowb + 16 * slot(row, nc * qcf + c))
            assert conflicts(addrs, 16, (8, 16)) == [], ("widened write", w, i)

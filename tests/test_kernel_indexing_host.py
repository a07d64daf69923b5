"""Host-side replay of the forward kernels' index arithmetic (no GPU; nothing is launched).

The kernels in csrc/fa2_fwd.hip stage K and V tiles into LDS with direct global->LDS loads
(16 bytes per lane, chunk index XOR-swizzled by row) and read them back as MFMA operands:
K rows with 16-byte reads, V^T with the transposed 8-byte reads. The ping-pong variant keeps
four tiles in a ring of LDS stages and issues tile j+2 while tile j is computed. This module
restates that arithmetic in numpy and checks, for every kernel geometry in the variant
table, head dimensions with and without padding, and full and ragged tiles:

* every direct load reads inside the (sequence, head) plane it belongs to, inside one row,
  16-byte aligned, and every LDS byte of a stage is written exactly once per tile;
* every K and V^T fragment read stays inside its tile and returns exactly the element the
  MFMA lane layout of v_mfma_f32_32x32x16_bf16 expects at that operand position (the keys of
  the V^T operand positions also match the keys of the P~ entries a lane holds);
* the ping-pong ring's phase schedule never reads a tile before both wave groups have
  waited for its loads, and never refills a stage before the last read of the tile in it.

The layouts checked are the ones the kernel source states in its header comment:
  A[m][k]: m = l % 32, k = 8*(l / 32) + e;  B[k][n]: n = l % 32, k = 8*(l / 32) + e;
  C[m][n]: n = l % 32, m = 8*(r / 4) + 4*(l / 32) + r % 4;
  ds_read_b64_tr_b16: lane j of a 16-lane group receives element j % 4 of the 8-byte rows
  addressed by lanes 4e + (j % 16) / 4, e = 0..3.
"""
from __future__ import annotations

import numpy as np
import pytest

LANES = np.arange(64)

# (D, BC, NW) of every forward kernel geometry in the variant table (ordinary and persistent
# kernels share one block function, so one entry covers both).
GEOMETRIES = [
    (64, 64, 8), (64, 128, 4), (64, 128, 8), (64, 64, 4),
    (128, 64, 8), (128, 64, 4), (128, 32, 4),
    (256, 32, 8), (256, 64, 4), (256, 32, 4),
]
PINGPONG = [(64, 64, 8), (128, 64, 8)]   # four-stage ring, 8 waves


def kswz(D, row):
    row = np.asarray(row)
    return (row & 15) if D >= 128 else ((row >> 1) & 7)


def vswz(D, row):
    row = np.asarray(row)
    return ((row & 3) << 2) if D >= 128 else (((row >> 1) & 1) << 2)


def padded_dims(D):
    """Tensor head dimensions that run on the kernel of width D (multiples of 8)."""
    lo = {64: 8, 128: 72, 256: 136}[D]
    return sorted({D, lo, D - 8, (lo + D) // 2 // 8 * 8})


class Geometry:
    def __init__(self, D, BC, NW):
        self.D, self.BC, self.NW = D, BC, NW
        self.ROWB = 2 * D
        self.TILEB = BC * self.ROWB
        self.STAGEB = 2 * self.TILEB
        assert self.TILEB % (1024 * NW) == 0
        self.DMA = self.TILEB // 1024 // NW
        self.NKB, self.NKC, self.NDB, self.NPC = BC // 32, D // 16, D // 32, BC // 16


def dma_slots(g: Geometry, dg: int):
    """Per (wave, d, lane): tile row, K/V byte offsets into the tile's global rows, and the
    LDS byte offset (inside the K tile; the V tile is the same plus TILEB)."""
    out = []
    for w in range(g.NW):
        for d in range(g.DMA):
            b = w * g.DMA + d
            o = b * 1024 + LANES * 16
            r = o // g.ROWB
            pch = (o % g.ROWB) // 16
            growb = 2 * dg
            koff = r * growb + ((pch ^ kswz(g.D, r)) % (dg // 8)) * 16
            voff = r * growb + ((pch ^ vswz(g.D, r)) % (dg // 8)) * 16
            lds = w * g.DMA * 1024 + d * 1024 + 16 * LANES
            out.append((r, koff, voff, lds, pch))
    return out


def stage_contents(g: Geometry, dg: int, seq_k: int, key0: int, which: str):
    """Simulate one tile's direct loads: returns (row, logical chunk) held by each physical
    16-byte chunk of the K (or V) tile in LDS, as global (key, chunk) pairs, and checks the
    global side of every load."""
    growb = 2 * dg
    nchunk = g.TILEB // 16
    held = np.full((nchunk, 2), -1, dtype=np.int64)
    writes = np.zeros(nchunk, dtype=np.int64)
    full = key0 + g.BC <= seq_k
    last = seq_k - 1 - key0
    for r, koff, voff, lds, pch in dma_slots(g, dg):
        off = koff if which == "K" else voff
        back = 0 if full else (r - np.minimum(r, last)) * growb
        gbyte = key0 * growb + off - back          # byte offset from the plane's first key
        assert np.all(gbyte % 16 == 0)
        assert np.all(gbyte >= 0) and np.all(gbyte + 16 <= seq_k * growb), "load outside the plane"
        key = gbyte // growb
        chunk = (gbyte % growb) // 16
        assert np.all(chunk < dg // 8)
        assert np.all(lds >= 0) and np.all(lds + 16 <= g.TILEB), "LDS write outside the tile"
        idx = lds // 16
        np.add.at(writes, idx, 1)
        held[idx, 0] = key
        held[idx, 1] = chunk
        # the physical chunk of the LDS slot is pch, in row r of the tile
        assert np.all(idx == r * (g.ROWB // 16) + pch)
    assert np.all(writes == 1), "each LDS chunk of a tile is written exactly once"
    return held


def lds_element(g, held, byte_off, key0, dg):
    """Global (key, column) of the bf16 at a byte offset inside the K or V tile in LDS."""
    ch = byte_off // 16
    key = held[ch, 0]
    col = held[ch, 1] * 8 + (byte_off % 16) // 2
    return key - key0, col


def ragged_cases(g):
    # seq_k and key0 of a full tile and of ragged last tiles of several lengths
    yield 4 * g.BC, g.BC
    for rem in (1, 5, g.BC // 2 + 3, g.BC - 1):
        yield 3 * g.BC + rem, 3 * g.BC


@pytest.mark.parametrize("D,BC,NW", GEOMETRIES + PINGPONG)
def test_direct_loads_stay_in_bounds_and_fill_each_stage_once(D, BC, NW):
    g = Geometry(D, BC, NW)
    for dg in padded_dims(D):
        for seq_k, key0 in ragged_cases(g):
            for which in ("K", "V"):
                held = stage_contents(g, dg, seq_k, key0, which)
                # rows past the end of a ragged tile re-read the last valid key
                rows = np.arange(g.BC)
                want = np.minimum(key0 + rows, seq_k - 1)
                keys = held[:, 0].reshape(g.BC, g.ROWB // 16)
                assert np.all(keys == want[:, None])


@pytest.mark.parametrize("D,BC,NW", GEOMETRIES + PINGPONG)
def test_k_fragment_reads_follow_the_mfma_a_layout(D, BC, NW):
    """S^T = K Q^T: the A operand of step kc in key block kb is K[kb*32 + l%32][16kc + 8(l/32) + e]."""
    g = Geometry(D, BC, NW)
    l32, hl = LANES & 31, LANES >> 5
    nka = min(g.NKC, 8)
    kaddr = [l32 * g.ROWB + (((2 * kc + hl) ^ kswz(D, l32)) * 16) for kc in range(nka)]
    for dg in (D, padded_dims(D)[0]):
        seq_k, key0 = 4 * BC, BC
        held = stage_contents(g, dg, seq_k, key0, "K")
        for kb in range(g.NKB):
            for kc in range(g.NKC):
                a = kb * 32 * g.ROWB + (kc >> 3) * 256 + kaddr[kc & 7]
                assert np.all(a % 16 == 0) and np.all(a >= 0) and np.all(a + 16 <= g.TILEB)
                for e in range(8):
                    key, col = lds_element(g, held, a + 2 * e, key0, dg)
                    want_col = 16 * kc + 8 * hl + e
                    assert np.all(key == kb * 32 + l32)
                    live = want_col < dg      # padded columns meet Q's zeros
                    assert np.all(col[live] == want_col[live])


def tr16_read(g, held, key0, dg, addr):
    """Model of ds_read_b64_tr_b16 for a wave: addr[lane] is the lane's 8-byte LDS address.
    Returns (key, column) of the 4 elements each lane receives."""
    keys = np.zeros((64, 4), dtype=np.int64)
    cols = np.zeros((64, 4), dtype=np.int64)
    for j in range(64):
        grp = j // 16 * 16
        for e in range(4):
            src = grp + 4 * e + (j % 16) // 4
            k, c = lds_element(g, held, np.array([addr[src] + 2 * (j % 4)]), key0, dg)
            keys[j, e], cols[j, e] = k[0], c[0]
    return keys, cols


@pytest.mark.parametrize("D,BC,NW", GEOMETRIES + PINGPONG)
def test_vt_fragment_reads_follow_the_mfma_a_layout_and_the_p_keys(D, BC, NW):
    """O^T = V^T P~^T: operand position 8h + 4t + e of step c carries key 16c + 8t + 4h + e and
    column d = 32 db + l%32, and P~ entry u of pw[c] (from S^T register r = 8(c%2) + u of key
    block c/2) belongs to the same key."""
    g = Geometry(D, BC, NW)
    l32, hl = LANES & 31, LANES >> 5
    vr = 4 * hl + ((LANES & 15) >> 2)
    nva = min(g.NDB, 4)
    vaddr = []
    for db in range(nva):
        col = 32 * db + 16 * ((LANES >> 4) & 1) + 4 * (LANES & 3)
        vaddr.append(g.TILEB + vr * g.ROWB + (((col >> 3) ^ vswz(D, vr)) * 16) + (col & 7) * 2)
    # keys of the P~ entries: C layout of the S^T MFMA, register r of key block kb
    def p_key(c, u):
        kb, r = c >> 1, (c & 1) * 8 + u
        return kb * 32 + 8 * (r // 4) + 4 * hl + r % 4

    for dg in (D, padded_dims(D)[0]):
        seq_k, key0 = 4 * BC, BC
        held = stage_contents(g, dg, seq_k, key0, "V")
        for c in range(g.NPC):
            for db in range(g.NDB):
                va = vaddr[db & 3] + (db >> 2) * 256 + 16 * c * g.ROWB - g.TILEB
                for t, a in enumerate((va, va + 8 * g.ROWB)):
                    assert np.all(a >= 0) and np.all(a + 8 <= g.TILEB), "V^T read outside the tile"
                    assert np.all((a % 16) + 8 <= 16), "an 8-byte read crosses a chunk"
                    keys, cols = tr16_read(g, held, key0, dg, a)
                    for e in range(4):
                        assert np.all(keys[:, e] == 16 * c + 8 * t + 4 * hl + e)
                        assert np.all(keys[:, e] == p_key(c, 4 * t + e))
                        live = 32 * db + l32 < dg
                        assert np.all(cols[live, e] == (32 * db + l32)[live])


def pingpong_schedule(nt):
    """Global barrier phases of the ping-pong kernel's two wave groups.

    Barrier k closes phase k. Both groups pass the start-up barrier (phase 1, in which every
    wave loads tiles 0 and 1 and waits for them); group B then passes one extra barrier, so
    iteration j of group g runs its MFMA phase in phase 2 + g + 2j and its VALU phase in the
    next one. An MFMA phase j issues the wave's loads of tile j+2 (if j+2 < nt), runs PV of
    tile j-1 and S of tile j, and ends with a wait that leaves only tile j+2's loads in
    flight (loads complete in issue order), so tile j+1 is complete for that group at the
    end of the phase. Returns per tile the phases of its issue, completion (one per group)
    and reads, and the number of barriers each group passes."""
    ev = {t: {"issue": [], "complete": [], "read": []} for t in range(nt)}
    for grp in (0, 1):
        for t in (0, 1):
            if t < nt:
                ev[t]["issue"].append(1)
                ev[t]["complete"].append(1)
        for j in range(nt + 1):
            ph = 2 + grp + 2 * j
            if j + 2 < nt:
                ev[j + 2]["issue"].append(ph)
            if 1 <= j <= nt - 2:
                ev[j + 1]["complete"].append(ph)
            if j - 1 >= 0:
                ev[j - 1]["read"].append(ph)   # PV(j-1)
            if j < nt:
                ev[j]["read"].append(ph)       # S(j)
    n_barriers = {0: 1 + 2 * (nt + 1) + 1, 1: 1 + 1 + 2 * (nt + 1)}
    return ev, n_barriers


@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5, 8, 13])
def test_pingpong_ring_reads_after_completion_and_refills_after_last_read(nt):
    nstage = 4
    ev, nb = pingpong_schedule(nt)
    assert nb[0] == nb[1], "both groups pass the same number of barriers"
    for t in range(nt):
        e = ev[t]
        assert len(e["issue"]) == 2 and len(e["complete"]) == 2, "each group loads and waits for its share"
        done = max(e["complete"])
        assert min(e["complete"]) >= max(e["issue"])
        assert min(e["read"]) > done, f"tile {t} read in phase {min(e['read'])}, complete only after {done}"
        # the next tile of the same stage is issued only after the last read of this one
        if t + nstage < nt:
            assert min(ev[t + nstage]["issue"]) > max(e["read"])
        # S in phases 2t+2 / 2t+3, PV in 2t+4 / 2t+5 (the last tile's PV in the extra iteration)
        assert sorted(e["read"]) == [2 * t + 2, 2 * t + 3, 2 * t + 4, 2 * t + 5]


@pytest.mark.parametrize("D,BC,NW", PINGPONG)
def test_pingpong_wait_count_is_one_tile_of_loads(D, BC, NW):
    """The partial wait keeps exactly the loads of one tile (K and V share) in flight: the
    kernel waits for vmcnt(2 * DMA_PER_WAVE) with 2 * DMA_PER_WAVE in {2, 4}."""
    g = Geometry(D, BC, NW)
    assert 2 * g.DMA in (2, 4)

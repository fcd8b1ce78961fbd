"""CPU model of the MFMA kernel's LDS tile layouts (attn_mfma_kernel.h).

The kernel stages each wave's K and V d-slices of a 32-key tile in LDS.  This
test restates the index arithmetic of the stores and the reads (the formulas
are retyped here, not imported) and checks, for every slice width the kernel
instantiates (32, 64, 128 d per wave):

  * round trip: what the whole-slice loads store is exactly what the MFMA
    operand reads fetch (K: key 16h + lane%16, d chunk 4s + lane/16;
    V^T via ds_read_b64_tr_b16: lane 4q+r of each 16-lane group receives
    element r of the 8-byte rows addressed by lanes q, q+4, q+8, q+12);
  * bank conflicts: every 16-lane pass of a 16-byte access and every
    32-lane pass of an 8-byte transposing read covers distinct banks
    (64 banks of 4 bytes), except the padded V rows' stores, whose partial
    conflicts are only bounded.

The transposing read's lane semantics were established on the GPU; here they
are a model.
"""
import numpy as np
import pytest

TILE = 32


def geometry(dw):
    nch = dw // 8                 # 16-byte chunks per key slice
    kpi = 64 // nch               # keys per load instruction
    ni = TILE // kpi              # loads per tile
    ksh = {16: 0, 8: 1, 4: 2}[nch]
    krow = dw * 2
    vswz = dw * 2 == 256
    vrow = dw * 2 if vswz else dw * 2 + 32
    return nch, kpi, ni, ksh, krow, vswz, vrow


def kofs(dw, row, chunk):
    nch, _, _, ksh, krow, _, _ = geometry(dw)
    return row * krow + 16 * (chunk ^ ((row >> ksh) & (nch - 1)))


def vofs(dw, row, c8):
    _, _, _, _, _, vswz, vrow = geometry(dw)
    return row * vrow + 8 * ((c8 ^ ((row & 7) << 2)) if vswz else c8)


def banks(addrs, width):
    out = set()
    for a in addrs:
        out |= {(a // 4 + j) % 64 for j in range(width // 4)}
    return out


@pytest.mark.parametrize("dw", [128, 64, 32])
def test_k_and_v_tiles_round_trip_without_conflicts(dw):
    nch, kpi, ni, ksh, krow, vswz, vrow = geometry(dw)
    ks, dt = dw // 32, dw // 16
    K = np.arange(TILE * dw).reshape(TILE, dw)
    V = K + 10 ** 6
    kl = np.full(TILE * krow // 2, -1, np.int64)
    vl = np.full(TILE * vrow // 2, -1, np.int64)
    # stores: load i, lane l holds key i*kpi + l//nch, d chunk l%nch (16 bytes)
    for i in range(ni):
        ka, va = [], []
        for lane in range(64):
            key, sl = i * kpi + lane // nch, lane % nch
            ko, vo = kofs(dw, key, sl), vofs(dw, key, 2 * sl)
            assert ko % 16 == 0 and ko + 16 <= TILE * krow
            assert vo % 16 == 0 and vo + 16 <= TILE * vrow
            kl[ko // 2: ko // 2 + 8] = K[key, 8 * sl: 8 * sl + 8]
            vl[vo // 2: vo // 2 + 8] = V[key, 8 * sl: 8 * sl + 8]
            ka.append(ko)
            va.append(vo)
        for p in range(4):
            assert len(banks(ka[16 * p: 16 * p + 16], 16)) == 64
            assert len(banks(va[16 * p: 16 * p + 16], 16)) >= (64 if vswz else 56)
    assert (kl >= 0).all()
    # K as the MFMA A operand: step s, half h, lane l -> key 16h + l%16, chunk 4s + l//16
    for h in range(2):
        for s in range(ks):
            addrs = []
            for lane in range(64):
                l16, g = lane & 15, lane >> 4
                a = kofs(dw, 16 * h + l16, 4 * s + g)
                addrs.append(a)
                assert list(kl[a // 2: a // 2 + 8]) == list(K[16 * h + l16, 8 * (4 * s + g): 8 * (4 * s + g) + 8])
            for p in range(4):
                assert len(banks(addrs[16 * p: 16 * p + 16], 16)) == 64
    # V^T through transposing reads: d tile c, key half
    for c in range(dt):
        for half in range(2):
            addr = [vofs(dw, 4 * (l >> 4) + ((l & 15) >> 2) + 16 * half, 4 * c + (l & 3)) for l in range(64)]
            for lane in range(64):
                g, l16 = lane >> 4, lane & 15
                q, r = l16 >> 2, l16 & 3
                got = [vl[addr[16 * g + q + 4 * j] // 2 + r] for j in range(4)]
                assert got == [V[16 * half + 4 * g + e, 16 * c + l16] for e in range(4)]
            for p in range(2):
                assert len(banks(addr[32 * p: 32 * p + 32], 8)) == 64


def test_a_planted_swizzle_mistake_is_caught():
    # the same check with the K swizzle dropped must find the 16-way conflict
    dw = 128
    addrs = [row * 256 + 16 * 3 for row in range(16)]
    assert len(banks(addrs, 16)) < 64

"""Decode the intra-chunk kernel's per-(head, chunk) blocks from a copy of
the workspace, following the layout documented in csrc/kda_internal.h:
fragments of 64 lanes x 16 bytes, lane l = 16 grp + n, slot e holding
physical index P(s, grp, e) = 32 s + 16 (e >> 2) + 4 grp + (e & 3)."""

import numpy as np

FRAG = 64 * 16
OFF_WN, OFF_QG, OFF_KGT = 0, 16 * FRAG, 32 * FRAG
OFF_AQK = 48 * FRAG
OFF_U = OFF_AQK + 6 * FRAG
OFF_GAM = OFF_U + 32 * 512
BLOCK = OFF_GAM + 512
LT_PAIRS = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1)]


def _bf16(raw):
    return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _vcol(nt, n):
    """Value column of lane n in value tile nt (kda_internal.h VCOL)."""
    return 32 * (nt >> 1) + 8 * (n >> 2) + 4 * (nt & 1) + (n & 3)


def _perm_index(s, grp, e):
    return 32 * s + 16 * (e >> 2) + 4 * grp + (e & 3)


def _frag(raw, off):
    """[64 lanes, 8 slots] float64 of one fragment."""
    return _bf16(raw[off:off + FRAG]).reshape(64, 8)


def decode_block(raw: np.ndarray) -> dict:
    assert raw.dtype == np.uint8 and raw.size == BLOCK
    W = np.zeros((64, 128))
    QG = np.zeros((64, 128))
    KG = np.zeros((64, 128))
    AQK = np.zeros((64, 64))
    U = np.zeros((64, 128))
    for mt in range(4):
        for s in range(4):
            fw = _frag(raw, OFF_WN + (mt * 4 + s) * FRAG)
            fq = _frag(raw, OFF_QG + (mt * 4 + s) * FRAG)
            for l in range(64):
                n, grp = l & 15, l >> 4
                for e in range(8):
                    W[16 * mt + n, _perm_index(s, grp, e)] = -fw[l, e]
                    QG[16 * mt + n, _perm_index(s, grp, e)] = fq[l, e]
    for mt in range(8):
        for s in range(2):
            fk = _frag(raw, OFF_KGT + (mt * 2 + s) * FRAG)
            for l in range(64):
                n, grp = l & 15, l >> 4
                for e in range(8):
                    KG[_perm_index(s, grp, e), 16 * mt + n] = fk[l, e]
    for x, (mt, s) in enumerate(LT_PAIRS):
        fa = _frag(raw, OFF_AQK + x * FRAG)
        for l in range(64):
            n, grp = l & 15, l >> 4
            for e in range(8):
                AQK[16 * mt + n, _perm_index(s, grp, e)] = fa[l, e]
    for nt in range(8):
        for mp in range(2):
            off = OFF_U + ((nt * 2 + mp) * 64) * 16
            t = _bf16(raw[off:off + 1024]).reshape(64, 8)
            for l in range(64):
                n, grp = l & 15, l >> 4
                for m in range(2):
                    for r in range(4):
                        U[16 * (2 * mp + m) + 4 * grp + r, _vcol(nt, n)] = t[l, 4 * m + r]
    gam = raw[OFF_GAM:OFF_GAM + 512].view(np.float32).astype(np.float64)
    return {"W": W, "qg": QG, "kg": KG, "Aqk": AQK, "U": U, "gamma": gam}

"""Host-side model of chunk_scan's LDS-DMA and staging index arithmetic (no GPU): for every
compiled shape, wave, lane and item, each global read stays inside its row or tile and
each LDS write inside its region.  The formulas restate those of csrc/chunk_scan.hip
(dma_item, the B-tile DMA and store_item); a guard that lets a lane past its data, as a
per-wave guard on the decay rows did for chunk lengths below 256, fails here."""
import itertools

import pytest

LDS_MAX = 160 * 1024
# (Q, P, N) compiled for chunk_scan (SSD_SCAN_SHAPES)
SHAPES = [(32, 32, 64), (32, 64, 64), (32, 64, 128), (64, 16, 16), (64, 16, 32), (64, 16, 64), (64, 16, 128), (64, 32, 32), (64, 32, 64), (64, 32, 128),
          (64, 64, 64), (64, 64, 128), (128, 32, 64), (128, 64, 64), (128, 64, 128), (256, 16, 32),
          (256, 32, 64), (256, 64, 64), (256, 64, 128), (256, 128, 128), (256, 64, 256)]


def layout(e, Q, P, N):
    cum_e = 8 if e == 4 else 4
    NRB = Q // 16
    NW = NRB // 2
    X, ST, CM = Q * P * e, P * N * e, Q * cum_e
    O_ST, O_CM = X, X + ST
    BYTES = O_CM + CM
    DB = 2 * BYTES <= LDS_MAX
    YP, YW = P * e // 16, 32 * P * e
    YS = DB and 2 * BYTES + NW * YW <= LDS_MAX
    LDS = (2 * BYTES if DB else BYTES) + (NW * YW if YS else 0)
    return dict(NW=NW, THREADS=NW * 64, X=X, ST=ST, CM=CM, O_ST=O_ST, O_CM=O_CM,
                BYTES=BYTES, DB=DB, YP=YP, YW=YW, YS=YS, LDS=LDS, XP=P * e // 16, BP=N * e // 16,
                BL=DB and Q * N * e <= LDS - BYTES)


def cases():
    for e in (4, 2):
        for Q, P, N in SHAPES:
            if e == 2 and N % 32:
                continue
            L = layout(e, Q, P, N)
            if L["LDS"] > LDS_MAX or P * e < 32:
                continue                       # not compiled (ScanCfg::OK is false)
            yield e, Q, P, N


@pytest.mark.parametrize("e,Q,P,N", list(cases()))
def test_chunk_scan_dma_and_staging_in_bounds(e, Q, P, N):
    c = layout(e, Q, P, N)
    NW, THREADS, XP, BP = c["NW"], c["THREADS"], c["XP"], c["BP"]
    SP, CP = c["ST"] // 16, c["CM"] // 16
    XK, SK = -(-Q * XP // THREADS), -(-SP // THREADS)
    assert CP <= THREADS
    assert (Q * XP) % 64 == 0 and SP % 64 == 0 and (Q * BP) % 64 == 0   # whole-wave tiles

    def swz(r):
        return (((r >> 1) & 3) << 1) & (XP - 1) if e == 2 else 0
    for Qc, w, lane in itertools.product(sorted({1, Q // 2 + 3, Q}), range(NW), range(64)):
        for k in range(XK):                                     # x tile
            if (k * NW + w) * 64 < Q * XP:
                piece = (k * NW + w) * 64 + lane
                r, qp = divmod(piece, XP)
                q = qp ^ swz(r)
                assert 0 <= min(r, Qc - 1) < Qc and q * 16 + 16 <= P * e
                assert (k * NW + w) * 1024 + lane * 16 + 16 <= c["X"]
        for k in range(SK):                                     # b_in tile
            if (k * NW + w) * 64 < SP:
                pc = (k * NW + w) * 64 + lane
                assert pc * 16 + 16 <= c["ST"]
                assert c["O_ST"] + (k * NW + w) * 1024 + lane * 16 + 16 <= c["O_CM"]
        pc = w * 64 + lane                                      # cum: per-lane guard
        if pc < CP:
            assert pc * 16 + 16 <= c["CM"] and c["O_CM"] + w * 1024 + lane * 16 + 16 <= c["BYTES"]
        if c["BL"]:                                             # B tile beside the first buffer
            for k in range(-(-Q * BP // THREADS)):
                if (k * NW + w) * 64 < Q * BP:
                    j = ((k * NW + w) * 64 + lane) // BP
                    assert j < Q and c["BYTES"] + (k * NW + w) * 1024 + lane * 16 + 16 <= c["LDS"]
        if c["YS"]:                                             # staged output rows of one wave
            YP = c["YP"]
            for k in range(32 * YP // 64):
                row, q = divmod(k * 64 + lane, YP)
                assert row < 32 and (row * YP + (q ^ (row & (min(YP, 8) - 1)))) * 16 + 16 <= c["YW"]


def test_a_per_wave_guard_on_short_decay_rows_would_overrun():
    """The model detects the bug class: with Q = 64 a decay row is 16 pieces, so letting all
    64 lanes of wave 0 copy overruns the 256-byte region (past the end of the head buffer)."""
    c = layout(2, 64, 64, 128)
    CP = c["CM"] // 16
    assert CP < 64
    lanes = range(64)                                           # what a per-wave guard admits
    assert any(c["O_CM"] + lane * 16 + 16 > c["BYTES"] for lane in lanes)

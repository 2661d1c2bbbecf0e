// Host check of the kernels' memory index arithmetic (no GPU): every function called here
// is the one the kernels call (chunked_linear_recurrence_amd/csrc/ssd_index.h), evaluated
// on the CPU for every compiled chunk_scan and chunk_state shape, both activation types,
// every wave, lane and item, and chunk lengths 1, Q/2 + 3 and Q.  For each copy it checks that the source
// lies inside its row or tile, that the LDS destination lies inside its region, and that
// the pieces cover their tile exactly once; for the staged outputs, that the rows read
// back are the ones the fragment stores wrote.  It also checks the state tile order used
// by state_pass.  A guard that lets lanes past their data (as a per-wave guard on the short
// decay rows did for chunks below 256 tokens) is shown to fail here.
//
// Prints one line per failed check and a summary; exits 1 on any failure.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "ssd_index.h"

using namespace ssd;

static long g_checks = 0, g_fail = 0;
static bool g_quiet = false;   // the planted check below fails on purpose: count, don't print

#define CHECK(cond, ...)                                                 \
    do {                                                                 \
        ++g_checks;                                                      \
        if (!(cond)) {                                                   \
            if (g_fail < 40 && !g_quiet) {                               \
                printf("FAIL %s:%d: ", __FILE__, __LINE__);              \
                printf(__VA_ARGS__);                                     \
                printf("\n");                                            \
            }                                                            \
            ++g_fail;                                                    \
        }                                                                \
    } while (0)

typedef DmaPiece (*RowFn)(int wv, int lane, int pieces);

// A row copy (cum or dblk) of `pieces` pieces by the waves wv(w), into an LDS region of
// `region` bytes: in bounds and each piece exactly once.  Returns the number of failures.
static long check_row(const char *what, RowFn fn, int NW, bool down, int pieces, int region, int src_bytes,
                      const char *shape) {
    const long before = g_fail;
    std::vector<int> seen(pieces, 0);
    for (int w = 0; w < NW; ++w)
        for (int lane = 0; lane < 64; ++lane) {
            const DmaPiece d = fn(down ? NW - 1 - w : w, lane, pieces);
            if (!d.on) continue;
            CHECK(d.piece >= 0 && d.piece * 16 + 16 <= src_bytes, "%s %s: piece %d past the row", shape, what, d.piece);
            CHECK(d.lds >= 0 && d.lds + 16 <= region, "%s %s: LDS byte %d past the region of %d", shape, what, d.lds,
                  region);
            if (d.piece >= 0 && d.piece < pieces) ++seen[d.piece];
        }
    for (int q = 0; q < pieces; ++q) CHECK(seen[q] == 1, "%s %s: piece %d copied %d times", shape, what, q, seen[q]);
    return g_fail - before;
}

// The transposed fragment reads of a row-major [rows][W] bf16 tile that a 64-lane x_swz copy
// filled (scan_x_piece): every lane's 8 bytes lie in the tile and hold the 4 columns of the
// row it asks for.  `rows` = Q, `pieces` = W * 2 / 16.
static void check_frag_reads(const char *what, const char *shape, int rows, int W, int nrowblk, int ncolt,
                             int region) {
    const int pieces = W * 2 / 16;
    for (int J = 0; J < nrowblk; ++J)
        for (int ct = 0; ct < ncolt; ++ct)
            for (int lane = 0; lane < 64; ++lane) {
                const FragRead f = tile_frag_read(J, ct, lane, W);
                CHECK(f.row < rows && f.col + 4 <= W, "%s %s: fragment row %d col %d", shape, what, f.row, f.col);
                CHECK(f.off >= 0 && f.off + 8 <= region, "%s %s: fragment byte %d past %d", shape, what, f.off, region);
                // the copy put source piece (pos ^ x_swz(row)) of row `row` at position pos
                const int pos = (f.off - f.row * W * 2) / 16;
                const int src_piece = pos ^ x_swz(f.row, pieces);
                CHECK(src_piece == f.col / 8 && (f.off & 15) == (f.col % 8) * 2, "%s %s: fragment reads the wrong columns",
                      shape, what);
            }
}

template <typename T, int Q, int P, int N>
static void check_scan_shape() {
    using Cfg = ScanCfg<T, Q, P, N>;
    if constexpr (Cfg::OK) {
        char shape[64];
        snprintf(shape, sizeof(shape), "%s Q=%d P=%d N=%d", sizeof(T) == 2 ? "bf16" : "f32", Q, P, N);
        const int NW = Cfg::NW, E = Cfg::E;
        CHECK(Cfg::LDS <= kLdsBytes, "%s: LDS %d", shape, Cfg::LDS);
        CHECK(Cfg::O_ST >= Cfg::X && Cfg::O_CM >= Cfg::O_ST + Cfg::ST && Cfg::O_DL >= Cfg::O_CM + Cfg::CM &&
                  Cfg::HEAD_BYTES >= Cfg::O_DL + Cfg::DL,
              "%s: head buffer regions overlap", shape);
        // x tile: whole tile once, rows < Q, pieces inside a row, LDS inside the x region
        std::vector<int> xsrc(Q * Cfg::XPIECES, 0), xdst(Q * Cfg::XPIECES, 0);
        for (int w = 0; w < NW; ++w)
            for (int lane = 0; lane < 64; ++lane)
                for (int k = 0; k < Cfg::XK; ++k) {
                    const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, Cfg::XPIECES, sizeof(T) == 2);
                    if (!d.on) continue;
                    CHECK(d.row >= 0 && d.row < Q, "%s x: row %d", shape, d.row);
                    CHECK(d.piece >= 0 && d.piece < Cfg::XPIECES, "%s x: piece %d", shape, d.piece);
                    CHECK(d.lds >= 0 && d.lds + 16 <= Cfg::X, "%s x: LDS byte %d", shape, d.lds);
                    if (d.row >= 0 && d.row < Q && d.piece >= 0 && d.piece < Cfg::XPIECES)
                        ++xsrc[d.row * Cfg::XPIECES + d.piece];
                    if (d.lds >= 0 && d.lds + 16 <= Cfg::X) ++xdst[d.lds / 16];
                    // the LDS slot holds source piece d.piece of row d.row: the transposed
                    // fragment reads find it at position piece ^ x_swz(row)
                    if (sizeof(T) == 2)
                        CHECK(d.lds / 16 == d.row * Cfg::XPIECES + (d.piece ^ x_swz(d.row, Cfg::XPIECES)),
                              "%s x: swizzle of row %d", shape, d.row);
                }
        for (int i = 0; i < Q * Cfg::XPIECES; ++i) {
            CHECK(xsrc[i] == 1, "%s x: source piece %d copied %d times", shape, i, xsrc[i]);
            CHECK(xdst[i] == 1, "%s x: LDS slot %d written %d times", shape, i, xdst[i]);
        }
        if (sizeof(T) == 2) check_frag_reads("x", shape, Q, Cfg::PV, Cfg::NRB, Cfg::PT, Cfg::X);
        // within one unit's slice of a chunk of Qc rows: the last byte read (row Qc - 1 after
        // the kernel's clamp) is inside the buffer bound the kernel gives that slice,
        // (Qc - 1) * row_pitch + PV * E, for the tightest row pitch H * P = P
        for (int Qc : {1, Q / 2 + 3, Q}) {
            if (Qc > Q) continue;
            const long pitch = (long)P * E;
            for (int w = 0; w < NW; ++w)
                for (int lane = 0; lane < 64; ++lane)
                    for (int k = 0; k < Cfg::XK; ++k) {
                        const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, Cfg::XPIECES, sizeof(T) == 2);
                        if (!d.on) continue;
                        const long rr = d.row < Qc - 1 ? d.row : Qc - 1;
                        CHECK(rr * pitch + d.piece * 16 + 16 <= (long)(Qc - 1) * pitch + Cfg::PV * E,
                              "%s x: read past the chunk (Qc %d)", shape, Qc);
                    }
        }
        // b(c-1) tile: flat, whole waves; over a head's units, every piece of the head's
        // state once, and each unit's LDS tile holds its p tiles of every n tile in order
        CHECK(Cfg::PS * Cfg::PV == P && Cfg::PS * Cfg::ST == Cfg::STH && Cfg::TP * 16 == 256 * E,
              "%s: channel units", shape);
        std::vector<int> sseen(Cfg::STH / 16, 0);
        for (int half = 0; half < Cfg::PS; ++half)
            for (int w = 0; w < NW; ++w)
                for (int lane = 0; lane < 64; ++lane)
                    for (int kk = 0; kk < Cfg::SK; ++kk) {
                        const DmaPiece d = scan_flat_piece(kk, w, lane, NW, Cfg::SP);
                        if (!d.on) continue;
                        const int src = scan_state_src_piece(d.piece, half, Cfg::PT, Cfg::PTH, Cfg::TP);
                        CHECK(d.piece * 16 + 16 <= Cfg::ST, "%s b_in: piece %d", shape, d.piece);
                        CHECK(src >= 0 && src * 16 + 16 <= Cfg::STH, "%s b_in: source piece %d", shape, src);
                        CHECK(Cfg::O_ST + d.lds + 16 <= Cfg::O_CM, "%s b_in: LDS byte %d", shape, d.lds);
                        // the source tile is (n tile, p tile) = (t / PTH, t % PTH); the LDS tile
                        // the unit's fragment reads index as (nt, pt) = (v / PT, v % PT)
                        const int vt = d.piece / Cfg::TP, st = src / Cfg::TP;
                        CHECK(st / Cfg::PTH == vt / Cfg::PT && st % Cfg::PTH == half * Cfg::PT + vt % Cfg::PT &&
                                  src % Cfg::TP == d.piece % Cfg::TP,
                              "%s b_in: tile of piece %d", shape, d.piece);
                        if (src >= 0 && src * 16 + 16 <= Cfg::STH) ++sseen[src];
                    }
        for (int i = 0; i < Cfg::STH / 16; ++i)
            CHECK(sseen[i] == 1, "%s b_in: piece %d copied %d times", shape, i, sseen[i]);
        // cum (waves from 0 up) and dblk (waves from NW - 1 down) rows
        check_row("cum", scan_row_piece, NW, false, Cfg::CP, Cfg::O_DL - Cfg::O_CM, Cfg::CM, shape);
        check_row("dblk", scan_row_piece, NW, true, Cfg::DP, Cfg::HEAD_BYTES - Cfg::O_DL, Cfg::DL, shape);
        // B tile beside the first head buffer
        if (Cfg::BL) {
            std::vector<int> bseen(Q * Cfg::BPIECES, 0);
            for (int w = 0; w < NW; ++w)
                for (int lane = 0; lane < 64; ++lane)
                    for (int k = 0; k < Cfg::BK; ++k) {
                        const DmaPiece d = scan_b_piece(k, w, lane, NW, Q, Cfg::BPIECES);
                        if (!d.on) continue;
                        CHECK(d.row >= 0 && d.row < Q, "%s B: row %d", shape, d.row);
                        CHECK(d.piece >= 0 && d.piece < Cfg::BPIECES, "%s B: piece %d", shape, d.piece);
                        CHECK(Cfg::HEAD_BYTES + d.lds + 16 <= Cfg::LDS, "%s B: LDS byte %d", shape, d.lds);
                        CHECK(d.lds / 16 == d.row * Cfg::BPIECES + (d.piece ^ (d.row & b_mask(Cfg::BPIECES))),
                              "%s B: swizzle of row %d", shape, d.row);
                        if (d.row >= 0 && d.row < Q && d.piece >= 0 && d.piece < Cfg::BPIECES)
                            ++bseen[d.row * Cfg::BPIECES + d.piece];
                    }
            for (int i = 0; i < Q * Cfg::BPIECES; ++i)
                CHECK(bseen[i] == 1, "%s B: piece %d copied %d times", shape, i, bseen[i]);
        }
        // staged outputs: each (row, piece) read exactly once, from where the fragment
        // stores put it: in the wave's staging area (YS), or in place (IP), inside the
        // wave's own x-copy slots of a head buffer, which no other wave writes
        if (Cfg::STAGED) {
            CHECK(Cfg::IP != Cfg::YS, "%s y: one staging mode", shape);
            for (int w = 0; w < (Cfg::IP ? NW : 1); ++w) {
                // bytes of the area this wave may stage into
                auto own = [&](int byte) {
                    if (!Cfg::IP) return byte >= 0 && byte < Cfg::YW;
                    if (byte < 0 || byte >= Cfg::X) return false;
                    const int slot = byte / 1024;       // x item k of wave w fills slot k * NW + w
                    return slot % NW == w && slot / NW < Cfg::XK;
                };
                std::vector<int> yseen(32 * Cfg::YPIECES, 0);
                std::vector<int> at(Cfg::IP ? Cfg::X : Cfg::YW, 0);
                for (int k = 0; k < Cfg::NSTQ; ++k)
                    for (int lane = 0; lane < 64; ++lane) {
                        const DmaPiece d = scan_y_piece(k, lane, Cfg::YPIECES, Cfg::IP, w, NW);
                        CHECK(d.row >= 0 && d.row < 32 && d.piece >= 0 && d.piece < Cfg::YPIECES,
                              "%s y: row %d piece %d", shape, d.row, d.piece);
                        CHECK(own(d.lds) && own(d.lds + 15), "%s y: wave %d reads LDS byte %d", shape, w, d.lds);
                        CHECK(d.lds == scan_y_stage(d.row, d.piece * 16, Cfg::YPIECES, Cfg::IP, w, NW),
                              "%s y: row %d piece %d misplaced", shape, d.row, d.piece);
                        if (d.row >= 0 && d.row < 32 && d.piece >= 0 && d.piece < Cfg::YPIECES)
                            ++yseen[d.row * Cfg::YPIECES + d.piece];
                    }
                for (int i = 0; i < 32 * Cfg::YPIECES; ++i)
                    CHECK(yseen[i] == 1, "%s y: staged piece %d stored %d times", shape, i, yseen[i]);
                // every fragment store (row, 4 channels at byte offset) lands inside the area,
                // and no two overlap
                for (int row = 0; row < 32; ++row)
                    for (int byte = 0; byte < Cfg::PV * E; byte += 4 * E) {
                        const int o = scan_y_stage(row, byte, Cfg::YPIECES, Cfg::IP, w, NW);
                        const bool in = own(o) && own(o + 4 * E - 1);
                        CHECK(in, "%s y: wave %d stage row %d byte %d at %d", shape, w, row, byte, o);
                        if (in)
                            for (int e = 0; e < 4 * E; ++e) CHECK(++at[o + e] == 1, "%s y: byte %d staged twice", shape, o + e);
                    }
            }
        }
    }
}

template <typename T, int Q, int P, int N>
static void check_state_shape() {
    using Cfg = StateCfg<T, Q, P, N>;
    if constexpr (Cfg::OK) {
        char shape[64];
        snprintf(shape, sizeof(shape), "state %s Q=%d P=%d N=%d", sizeof(T) == 2 ? "bf16" : "f32", Q, P, N);
        const int NW = Cfg::NWS;
        CHECK(Cfg::LDS <= kLdsBytes && 2 * Cfg::HEAD_BYTES <= Cfg::LDS && Cfg::BT <= Cfg::LDS, "%s: LDS", shape);
        // x tile of one head and the B tile of the workgroup: the same 64-lane copy
        for (int which = 0; which < 2; ++which) {
            const int pieces = which == 0 ? Cfg::XPIECES : Cfg::BPIECES;
            const int items = which == 0 ? Cfg::XK : Cfg::BK;
            const int region = which == 0 ? Cfg::X : Cfg::BT;
            std::vector<int> seen(Q * pieces, 0);
            for (int w = 0; w < NW; ++w)
                for (int lane = 0; lane < 64; ++lane)
                    for (int k = 0; k < items; ++k) {
                        const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, pieces, sizeof(T) == 2);
                        if (!d.on) continue;
                        CHECK(d.row < Q && d.piece < pieces, "%s %s: row %d piece %d", shape, which ? "B" : "x", d.row,
                              d.piece);
                        CHECK(d.lds >= 0 && d.lds + 16 <= region, "%s %s: LDS byte %d", shape, which ? "B" : "x", d.lds);
                        if (d.row < Q && d.piece < pieces) ++seen[d.row * pieces + d.piece];
                    }
            for (int i = 0; i < Q * pieces; ++i)
                CHECK(seen[i] == 1, "%s %s: piece %d copied %d times", shape, which ? "B" : "x", i, seen[i]);
        }
        check_row("wend", scan_row_piece, NW, true, Cfg::WP, Cfg::HEAD_BYTES - Cfg::O_W, Cfg::WB, shape);
        // every output tile (n tile, p tile) owned by exactly one wave
        CHECK(Cfg::THREADS <= 1024 && Cfg::NWN * Cfg::NTW == Cfg::NT && Cfg::PS * Cfg::PTW == Cfg::PT,
              "%s: wave split", shape);
        std::vector<int> tseen(Cfg::NT * Cfg::PT, 0);
        for (int w = 0; w < NW; ++w) {
            const StateTiles t = state_wave_tiles(w, Cfg::NWN, Cfg::NTW, Cfg::PTW, Cfg::PS);
            for (int i = 0; i < Cfg::NTW; ++i)
                for (int pt = 0; pt < Cfg::PTW; ++pt) {
                    const int nt = t.nt0 + i, pp = t.pt0 + pt;
                    CHECK(nt >= 0 && nt < Cfg::NT && pp >= 0 && pp < Cfg::PT, "%s: wave %d tile (%d, %d)", shape, w,
                          nt, pp);
                    if (nt >= 0 && nt < Cfg::NT && pp >= 0 && pp < Cfg::PT) ++tseen[nt * Cfg::PT + pp];
                }
        }
        for (int i = 0; i < Cfg::NT * Cfg::PT; ++i)
            CHECK(tseen[i] == 1, "%s: output tile %d owned by %d waves", shape, i, tseen[i]);
        if (sizeof(T) == 2) {
            check_frag_reads("x", shape, Q, P, Cfg::KT, Cfg::PT, Cfg::X);
            check_frag_reads("B", shape, Q, N, Cfg::KT, Cfg::NT, Cfg::BT);
        }
    }
}

#define SSD_CHECK_SHAPE(T, q, pp, nn) check_scan_shape<T, q, pp, nn>();
#define SSD_CHECK_STATE(T, q, pp, nn) check_state_shape<T, q, pp, nn>();

// A per-wave guard on the row copies, the form that once let lanes past a row shorter than
// a wave: the check above must reject it.
static DmaPiece per_wave_guard(int wv, int lane, int pieces) {
    const int pc = wv * 64 + lane;
    return DmaPiece{wv * 64 < pieces, 0, pc, pc * 16};
}

static void check_tile_order() {
    for (int P : {16, 32, 64, 128})
        for (int N : {16, 32, 64, 128, 256}) {
            std::vector<int> seen(P * N, 0);
            for (int e = 0; e < P * N; e += 4) {
                const StateIdx pn = tile_elem(e, P);
                CHECK(pn.p >= 0 && pn.p < P && pn.n0 >= 0 && pn.n0 + 3 < N, "tile order P=%d N=%d e=%d", P, N, e);
                if (pn.p >= 0 && pn.p < P && pn.n0 >= 0 && pn.n0 + 3 < N)
                    for (int r = 0; r < 4; ++r) ++seen[pn.p * N + pn.n0 + r];
            }
            for (int i = 0; i < P * N; ++i) CHECK(seen[i] == 1, "tile order P=%d N=%d: element %d seen %d times", P, N, i,
                                                  seen[i]);
        }
}

int main() {
    SSD_SCAN_SHAPES(SSD_CHECK_SHAPE, bf16)
    SSD_SCAN_SHAPES(SSD_CHECK_SHAPE, float)
    SSD_STATE_SHAPES(SSD_CHECK_STATE, bf16)
    SSD_STATE_SHAPES(SSD_CHECK_STATE, float)
    check_tile_order();
    const long checks = g_checks, fails = g_fail;
    // sensitivity: the per-wave guard on the 16-piece cum row of Q = 64 (bf16) overruns
    g_quiet = true;
    const long f = check_row("cum (per-wave guard)", per_wave_guard, ScanCfg<bf16, 64, 64, 128>::NW, false,
                             ScanCfg<bf16, 64, 64, 128>::CP,
                             ScanCfg<bf16, 64, 64, 128>::O_DL - ScanCfg<bf16, 64, 64, 128>::O_CM,
                             ScanCfg<bf16, 64, 64, 128>::CM, "planted");
    printf("index checks: %ld, failures: %ld; planted per-wave guard detected: %s\n", checks, fails,
           f > 0 ? "yes" : "no");
    return (fails == 0 && f > 0) ? 0 : 1;
}

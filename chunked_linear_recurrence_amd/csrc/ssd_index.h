// Index arithmetic of the libssdscan kernels that touches memory: which lane copies which
// 16-byte piece where, and the LDS layouts those copies fill.  The kernels call these
// functions, and the host program tests/c/index_check.cpp calls the very same ones for
// every compiled shape, wave, lane and item to check that every global read stays inside
// its row or tile and every LDS access inside its region (so an index or guard change
// cannot drift away from what is checked).  Nothing here touches memory.
#pragma once

#include "ssd_common.h"

namespace ssd {

// ---------------------------------------------------------------------------------
// chunk_scan: layout constants
// ---------------------------------------------------------------------------------
template <typename T, int Q, int P, int N>
struct ScanCfg {
    typedef typename CumT<T>::type S;
    static constexpr int E = (int)sizeof(T);
    static constexpr int NRB = Q / 16, NW = NRB / 2, THREADS = NW * 64;
    static constexpr int NSLOT = NRB + 2, NPAIR = NSLOT / 2;
    static constexpr int NTRI = NRB * (NRB + 1) / 2;            // causal tiles per chunk
    // A head whose inputs do not fit in LDS twice (P = 128; fp32 at Q = 256) is taken as
    // PS = 2 units of PV = P/2 channels: a unit is a head of PV channels for the products,
    // the LDS layout and the stores, reading its channels' slice of x, b(c-1) and y.
    static constexpr int CM = Q * (int)sizeof(S), DL = Q * 4;
    static constexpr int HEAD_BYTES_P = Q * P * E + P * N * E + CM + DL;
    static constexpr int PS = (2 * HEAD_BYTES_P > kLdsBytes && (P / 2) % 16 == 0 && (P / 2) * E >= 32) ? 2 : 1;
    static constexpr int PV = P / PS;                           // channels per unit
    static constexpr int PT = PV / 16, NT = N / 16;             // p tiles per unit, n tiles
    static constexpr int PTH = P / 16;                          // p tiles of a whole head
    static constexpr int TP = 16 * E;                           // 16-byte pieces per 16x16 state tile
    static constexpr int STH = P * N * E;                       // a head's b(c-1) in bytes
    // one unit's inputs in LDS (HeadBuf): x tile [Q][PV], b(c-1) tile [PV*N] (the unit's p
    // tiles of every n tile, tile order), the prefix sums cum [Q] and the block decays
    // dblk [Q] (float32)
    static constexpr int X = Q * PV * E, ST = PV * N * E;
    static constexpr int O_ST = X, O_CM = X + ST, O_DL = O_CM + CM;
    static constexpr int HEAD_BYTES = O_DL + DL;
    static constexpr bool DB = 2 * HEAD_BYTES <= kLdsBytes;     // double-buffered head data
    static constexpr int XPIECES = PV * E / 16;                 // 16-byte pieces per x row
    static constexpr int YPIECES = PV * E / 16;                 // 16-byte pieces per output row
    static constexpr int YW = 32 * PV * E;                      // one wave's staged outputs
    // Outputs leave through LDS rows (whole 128-byte output rows per store): a separate
    // staging area when it fits beside the two head buffers (YS), else in place (IP): each
    // wave stages its rows in its own x slots of the finished head buffer (a wave's 32
    // output rows are exactly as many bytes as its share of the x copy).
    static constexpr bool YS = DB && 2 * HEAD_BYTES + NW * YW <= kLdsBytes;
    static constexpr bool IP = DB && !YS;
    static constexpr bool STAGED = YS || IP;
    static constexpr int LDS = (DB ? 2 * HEAD_BYTES : HEAD_BYTES) + (YS ? NW * YW : 0);
    // The chunk's B tile (Q x N) is staged in LDS for the S^T products when it fits beside
    // the first head's buffer; otherwise the B fragments are loaded from L2.
    static constexpr int BPIECES = N * E / 16;                  // 16-byte pieces per B row
    static constexpr bool BL = DB && Q * N * E <= LDS - HEAD_BYTES;
    // memory work per head and wave, in single-instruction items (64 lanes x 16 bytes)
    static constexpr int XK = (Q * XPIECES + THREADS - 1) / THREADS;   // x tile
    static constexpr int SP = ST / 16, SK = (SP + THREADS - 1) / THREADS;  // b(c-1) tile
    static constexpr int CP = CM / 16, DP = DL / 16;                  // cum, dblk rows
    static constexpr int NDMA = XK + SK + 2;
    static constexpr int BK = (Q * BPIECES + THREADS - 1) / THREADS;  // B tile (per workgroup)
    static constexpr int NSTQ = 32 * YPIECES / 64;                    // staged-output stores
    static constexpr bool OK = LDS <= kLdsBytes &&
                               (sizeof(T) == 4 || NT % 2 == 0) && (Q == 32 || Q == 64 || Q == 128 || Q == 256) &&
                               PV * E >= 32 && CP <= THREADS && DP <= THREADS;
};

// Piece v of a unit's b(c-1) tile in LDS (its p tiles of every n tile, in tile order) as a
// piece of the head's whole state (tile order [n tile][p tile], PTH p tiles): unit `half`
// takes p tiles [half PT, (half + 1) PT).  The identity for a single unit (PT = PTH).
__host__ __device__ constexpr int scan_state_src_piece(int v, int half, int PT, int PTH, int TP) {
    return (((v / TP) / PT) * PTH + half * PT + (v / TP) % PT) * TP + v % TP;
}

// Every (Q, P, N) compiled for chunk_scan, for each activation type T (X(T, Q, P, N)).
#define SSD_SCAN_SHAPES(X, T)                                                              \
    X(T, 32, 32, 64) X(T, 32, 64, 64) X(T, 32, 64, 128)                                    \
    X(T, 64, 16, 16) X(T, 64, 16, 32) X(T, 64, 16, 64) X(T, 64, 16, 128)                   \
    X(T, 64, 32, 32) X(T, 64, 32, 64) X(T, 64, 32, 128) X(T, 64, 64, 64) X(T, 64, 64, 128) \
    X(T, 128, 32, 64) X(T, 128, 64, 64) X(T, 128, 64, 128)                                 \
    X(T, 256, 16, 32) X(T, 256, 32, 64) X(T, 256, 64, 64) X(T, 256, 64, 128)               \
    X(T, 256, 128, 128) X(T, 256, 64, 256)

// One lane's part of a 64-lane global -> LDS copy of 16-byte pieces: whether it copies,
// the source row and 16-byte piece within that row (or the piece of a flat tile), and the
// byte offset it fills in its LDS region (the copy writes lane l at base + 16 l).
struct DmaPiece {
    bool on;
    int row, piece, lds;
};

// x tile in LDS: row-major [Q][P] in 16-byte pieces; piece q of row r is stored at position
// q ^ x_swz(r) of that row (bf16), which spreads the 4 rows read by one transpose load over
// different banks.  pieces = XPIECES is a power of two.
__host__ __device__ constexpr int x_swz(int r, int pieces) { return (((r >> 1) & 3) << 1) & (pieces - 1); }

// x tile, item k (< XK) of wave w.  The source row may lie past a short chunk; the kernel
// reads min(row, Qc - 1) instead (those rows only meet zero weights).
__host__ __device__ constexpr DmaPiece scan_x_piece(int k, int w, int lane, int NW, int Q, int xpieces, bool swz) {
    const int blk = (k * NW + w) * 64;
    const int piece = blk + lane;
    const int r = piece / xpieces;
    return DmaPiece{blk < Q * xpieces, r, (piece % xpieces) ^ (swz ? x_swz(r, xpieces) : 0), piece * 16};
}

// Byte offset, inside a row-major [rows][W] bf16 tile stored with x_swz, of the 8 bytes lane
// `lane` reads for the transposed fragment (16-row block J, 16-column tile ct): lane s of a
// 16-lane group g reads columns c..c+3 of row r, with r = 16J + 4g + s / 4 and
// c = 16ct + 4 (s % 4); after the transpose, lane (col, g) holds rows 16J + 4g + e of
// column 16ct + col.
struct FragRead {
    int row, col, off;
};
__host__ __device__ constexpr FragRead tile_frag_read(int J, int ct, int lane, int W) {
    const int s = lane & 15, g = lane >> 4;
    const int r = J * 16 + 4 * g + (s >> 2);
    const int c = ct * 16 + 4 * (s & 3);
    return FragRead{r, c, r * (W * 2) + ((c >> 3) ^ x_swz(r, W * 2 / 16)) * 16 + (c & 7) * 2};
}

// A flat tile of `pieces` pieces (b(c-1) in tile order), item kk (< SK) of wave w; the
// tile is a whole number of waves, so the guard is uniform.
__host__ __device__ constexpr DmaPiece scan_flat_piece(int kk, int w, int lane, int NW, int pieces) {
    const int blk = (kk * NW + w) * 64;
    return DmaPiece{blk < pieces, 0, blk + lane, (blk + lane) * 16};
}

// A short row of `pieces` pieces (cum or dblk of one (head, chunk)) copied by wave wv.  The
// row need not fill whole waves (Q < 256), so the guard is per lane then: no lane reads past
// the row or writes past its LDS region.
__host__ __device__ constexpr DmaPiece scan_row_piece(int wv, int lane, int pieces) {
    const int pc = wv * 64 + lane;
    return DmaPiece{(pieces % 64 == 0) ? (wv * 64 < pieces) : (pc < pieces), 0, pc, pc * 16};
}

// B tile in LDS: row-major [Q][N], piece q of row j at position q ^ (j & bmask), so the 16
// rows read by one fragment load hit different banks.
__host__ __device__ constexpr int b_mask(int bpieces) { return (bpieces < 16 ? bpieces : 16) - 1; }

// B tile, item k (< BK) of wave w (rows past a short chunk: the kernel reads the last row,
// and the fragments it builds from them are zeroed).
__host__ __device__ constexpr DmaPiece scan_b_piece(int k, int w, int lane, int NW, int Q, int bpieces) {
    const int blk = (k * NW + w) * 64;
    const int slot = blk + lane;
    const int j = slot / bpieces;
    return DmaPiece{blk < Q * bpieces, j, (slot % bpieces) ^ (j & b_mask(bpieces)), slot * 16};
}

// Staged outputs of one wave: 32 rows (its two row blocks) of YPIECES 16-byte pieces; piece
// q of row r sits at position q ^ ysw(r), so the fragment writes and the row reads both
// spread over all banks.
__host__ __device__ constexpr int ysw(int r, int ypieces) { return r & ((ypieces < 8 ? ypieces : 8) - 1); }

// Start of staged row r of wave w.  In a separate staging area (inplace false) the wave's
// rows are contiguous (offsets inside the wave's area).  In place, the rows fill the
// wave's own 1 KB x-copy slots of a head buffer, slots k * NW + w for k = 0..XK-1,
// 64 / ypieces rows per slot (offsets inside the buffer).
__host__ __device__ constexpr int scan_y_row_base(int row, int ypieces, bool inplace, int w, int NW) {
    return inplace ? ((row / (64 / ypieces)) * NW + w) * 1024 + (row % (64 / ypieces)) * ypieces * 16
                   : row * ypieces * 16;
}

// Store item k (< NSTQ) of a wave's staged rows: the staging row (0..31; rows 0..15 are
// tokens of row block I0, 16..31 of I1), the 16-byte piece of the output row, and the LDS
// byte offset it is read from.
__host__ __device__ constexpr DmaPiece scan_y_piece(int k, int lane, int ypieces, bool inplace = false, int w = 0,
                                                   int NW = 1) {
    const int pc = k * 64 + lane;
    const int row = pc / ypieces, q = pc % ypieces;
    return DmaPiece{true, row, q, scan_y_row_base(row, ypieces, inplace, w, NW) + (q ^ ysw(row, ypieces)) * 16};
}

// LDS byte offset of the staged output value (row, byte) written by the fragment stores:
// row = ri * 16 + token within the block, byte = channel * sizeof(T).
__host__ __device__ constexpr int scan_y_stage(int row, int byte, int ypieces, bool inplace = false, int w = 0,
                                               int NW = 1) {
    return scan_y_row_base(row, ypieces, inplace, w, NW) + ((byte >> 4) ^ ysw(row, ypieces)) * 16 + (byte & 15);
}

// ---------------------------------------------------------------------------------
// chunk_state: layout constants
// ---------------------------------------------------------------------------------
template <typename T, int Q, int P, int N>
struct StateCfg {
    static constexpr int E = (int)sizeof(T);
    static constexpr int NT = N / 16, PT = P / 16, KT = Q / 16;
    // one head's inputs in LDS: x tile [Q][P] (row-major, x_swz pieces for bf16) and the
    // chunk-end decays wend [Q] (float32); double-buffered across heads
    static constexpr int X = Q * P * E, WB = Q * 4;
    static constexpr int O_W = X, HEAD_BYTES = X + WB;
    // the chunk's B tile [Q][N] (row-major, x_swz pieces), read once per workgroup into
    // fragments, occupies the head buffers before the first head's inputs arrive
    static constexpr int BT = Q * N * E;
    static constexpr int LDS = 2 * HEAD_BYTES > BT ? 2 * HEAD_BYTES : BT;
    // Waves: N/32 along n, each owning NTW n tiles.  When the LDS leaves room for only one
    // workgroup per CU (so each SIMD has the registers of two waves) and that makes at most
    // 8 waves, a second wave per n range takes half of the p tiles: each wave then holds
    // half the accumulators, which keeps the large tiles (P = 128, fp32 at Q = 256) in
    // registers.
    static constexpr int NWN = N >= 32 ? N / 32 : 1;           // waves along n
    static constexpr int NTW = NT / NWN;                        // n tiles per wave
    static constexpr int PS = (LDS > kLdsBytes / 2 && NWN <= 4 && PT % 2 == 0) ? 2 : 1;
    static constexpr int PTW = PT / PS;                         // p tiles per wave
    static constexpr int NWS = NWN * PS;                        // waves
    static constexpr int THREADS = NWS * 64;
    static constexpr int MINB = PS == 2 ? 1 : 2;                // workgroups per CU (launch bound)
    static constexpr int XPIECES = P * E / 16, BPIECES = N * E / 16;
    static constexpr int XK = (Q * XPIECES + THREADS - 1) / THREADS;   // x items per head and wave
    static constexpr int WP = WB / 16;                                 // wend pieces
    static constexpr int NDMA = XK + 1;
    static constexpr int BK = (Q * BPIECES + THREADS - 1) / THREADS;   // B items per workgroup and wave
    static constexpr bool OK = KT % 2 == 0 && NT % NWN == 0 && LDS <= kLdsBytes && P * E >= 32 &&
                               N * E >= 32 && WP <= THREADS && (Q * XPIECES) % 64 == 0 &&
                               (Q * BPIECES) % 64 == 0;
};

// The output tiles of chunk_state's wave w: n tiles [nt0, nt0 + NTW), p tiles [pt0, pt0 + PTW).
struct StateTiles {
    int nt0, pt0;
};
__host__ __device__ constexpr StateTiles state_wave_tiles(int w, int NWN, int NTW, int PTW, int PS) {
    return PS == 1 ? StateTiles{w * NTW, 0} : StateTiles{(w % NWN) * NTW, (w / NWN) * PTW};
}

// Every (Q, P, N) compiled for chunk_state (X(T, Q, P, N)).
#define SSD_STATE_SHAPES(X, T)                                                             \
    X(T, 32, 32, 64) X(T, 32, 64, 64) X(T, 32, 64, 128)                                    \
    X(T, 64, 16, 16) X(T, 64, 16, 32) X(T, 64, 16, 64) X(T, 64, 16, 128)                   \
    X(T, 64, 32, 32) X(T, 64, 32, 64) X(T, 64, 32, 128) X(T, 64, 64, 64) X(T, 64, 64, 128) \
    X(T, 128, 32, 64) X(T, 128, 64, 64) X(T, 128, 64, 128)                                 \
    X(T, 256, 16, 32) X(T, 256, 32, 64) X(T, 256, 64, 64) X(T, 256, 64, 128)               \
    X(T, 256, 128, 128) X(T, 256, 64, 256)

// ---------------------------------------------------------------------------------
// state_pass: element e (a multiple of 4) of a P x N state in tile order ->
// (p, first n of the 4 consecutive n held there).  Tile order: 16x16 tiles indexed
// [n / 16][p / 16], 64 lanes x 4 values each; lane l, value r holds p = 16 pt + l % 16,
// n = 16 nt + 4 (l / 16) + r.
// ---------------------------------------------------------------------------------
struct StateIdx {
    int p, n0;
};
__host__ __device__ constexpr StateIdx tile_elem(int e, int P) {
    const int tile = e >> 8, l = (e >> 2) & 63;
    const int PT = P >> 4;
    return StateIdx{(tile % PT) * 16 + (l & 15), (tile / PT) * 16 + 4 * (l >> 4)};
}

}  // namespace ssd

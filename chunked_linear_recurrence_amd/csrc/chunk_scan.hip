// chunk_scan: every chunk's output, [分块推理 §2.1-§2.2] of the page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理":
//
//   by_intra_i = sum_{j <= i} (C_i . B_j) 2^(cum_i - cum_j) x_j      (zero-state intra part)
//   by_inter_i = 2^(cum_i) (b(c-1) C_i)                                (diag(L) C(c) b(c-1))
//   y_i        = by_intra_i + by_inter_i + D x_i  (+ x_i with SSD_FLAG_RESIDUAL)
//
// rounded once to the activation dtype.  cum is the chunk's dA_cum row, the base-2 prefix
// sums of dt A (so 2^(cum_i - cum_j) is the decay from token j to token i), and b(c-1) is
// b_in[c] from state_pass.
//
// One workgroup per (batch, chunk, group of heads that read the same B and C).  A chunk
// is cut into Q/16 row blocks of 16 tokens and the workgroup has Q/32 waves; wave w owns
// row blocks I0 = w and I1 = Q/16-1-w, so every wave has the same number (Q/16 + 1) of
// causal 16x16 tiles (J <= I).  The wave's tile list ("slots") is: slot s <= w is
// (I0, J = s), slot w + 1 is a zero pad, slot s >= w + 2 is (I1, J = s - w - 2); the pad
// keeps pairs of slots inside one row block.  The wave index is read as a scalar, so
// every choice that depends on it is a uniform branch.
//
// Once per workgroup, each wave computes its causal tiles of S^T = B_c C_c^T on the
// matrix cores (B fragments from the chunk's B tile, staged in LDS by DMA where it fits,
// else from L2; C fragments kept in registers), zero above the diagonal, and keeps them in
// fp32 registers for every head of the group: C.B^T is formed once per chunk and group,
// never per head.
//
// Per head, x is brought into LDS by buffer DMA (tokens x channels, read back as
// transposed fragments), b_in likewise, and the chunk's prefix sums cum and block decays
// dblk.  A head whose inputs do not fit in LDS twice (P = 128; fp32 at Q = 256) is taken as
// two units of P/2 channels, each a head of its own for the copies, products and stores
// (ScanCfg::PS), so those shapes are double-buffered too.  The products are computed transposed (y^T[p][i]) so that a lane's 4 accumulator
// values are 4 consecutive channels of one token:
//     Z^T = b(c-1) C^T, column i scaled by G_i = 2^(cum_i);
//     y^T += x^T (S^T . decay), the decay of tile entry (j, i) being 2^(cum_i - cum_j)
//       (cum holds base-2 sums of dt A).  Below the diagonal (token j in an earlier 16-token
//       block J than i) it is factored through the end e_J of j's block:
//         2^(cum_i - cum_j) = 2^(cum_i - cum_{e_J}) * dblk_j,   dblk_j = 2^(cum_{e_J} - cum_j),
//       both factors <= 1 (cum is non-increasing), dblk precomputed per token by
//       chunk_cumsum: one 2^x per tile and lane instead of one per entry.  On diagonal
//       tiles it is 2^(min(cum_i - cum_j, 0)) per entry (the zeroed upper triangle of S^T
//       does the masking).  A lane's 4 S^T values are 4 consecutive k values of the B
//       operand (and share one column i), so no data moves between lanes;
//     y^T += x^T diag(D + residual) on the matrix cores (D split in a high and a low bf16
//       part so the skip term keeps fp32 accuracy; K = 16 products).
// Tiles are paired into 16x16x32 bf16 products (16x16x4 f32 for the fp32 dtype).
#include "ssd_tile.h"

namespace ssd {

// Slot s of wave w: row block, column block, pad flag (all uniform).
struct Slot {
    int I, J;
    bool pad, first;
};
__device__ __forceinline__ Slot slot_of(int s, int w, int NRB) {
    Slot r;
    r.pad = s == w + 1;
    r.first = s <= w;
    r.I = r.first ? w : NRB - 1 - w;
    r.J = r.pad ? 0 : (r.first ? s : s - w - 2);
    return r;
}

// ---------------------------------------------------------------------------------
// chunk_scan: one (batch, chunk, group of heads)
// ---------------------------------------------------------------------------------
// x^T fragment for (16-token block J, 16-channel tile pt): lane (col, g) gets
// x[16J + 4g + e][16pt + col], e = 0..3 (tile_frag of the row-major x tile).
template <typename T, int P>
__device__ __forceinline__ typename TF<T>::type x_frag(const unsigned char *xs, int J, int pt, int lane) {
    return tile_frag<T, P>(xs, J, pt, lane);
}

// Per-head products of wave W (all slot choices and offsets are compile-time):
// Z^T scaled by G, the decayed S^T tiles times x^T, and (D + res) x.  hook(k, nbuf, ys)
// is called at 1 + PT + NPAIR fixed points of the body (k known at compile time once
// unrolled); the caller uses it to spread its memory traffic through the matrix-core
// work.  buf (this head's inputs), nbuf (the next head's, being filled by DMA) and ys
// (staged outputs) are disjoint LDS regions; saying so (restrict) lets the compiler
// keep this head's LDS reads from waiting on the next head's DMA.
template <typename T, int Q, int P, int N, int W, typename Hook>
__device__ __forceinline__ void scan_head(const unsigned char *__restrict__ buf, unsigned char *__restrict__ nbuf,
                                      unsigned char *__restrict__ ys,
                                      const f32x4 (&sT)[ScanCfg<T, Q, P, N>::NSLOT],
                                      const typename TF<T>::type (&cf)[2][ScanCfg<T, Q, P, N>::NT],
                                      float dres, int lane, f32x4 (&acc)[2][ScanCfg<T, Q, P, N>::PT],
                                      Hook &&hook) {
    using Cfg = ScanCfg<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int NRB = Cfg::NRB, PT = Cfg::PT, NT = Cfg::NT;
    constexpr int NSTEP = sizeof(T) == 2 ? 2 : 1;
    constexpr int w = W, I0 = W, I1 = NRB - 1 - W;
    const int col = lane & 15, g4 = 4 * (lane >> 4);
    const unsigned char *xs = buf;
    const T *stb = reinterpret_cast<const T *>(buf + Cfg::O_ST);
    const S *cm = reinterpret_cast<const S *>(buf + Cfg::O_CM);
    const float *dlk = reinterpret_cast<const float *>(buf + Cfg::O_DL);

    // Output tiles are transposed: acc[ri][pt] lane (col, g), value r holds
    // y^T[p = pt*16 + 4g + r][i = I*16 + col].
    // Z^T = b(c-1) C^T, then column i scaled by G_i = 2^(cum_i)
#pragma unroll
    for (int ri = 0; ri < 2; ++ri)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[ri][pt] = zero_frag<f32x4>();
    hook(0, nbuf, ys);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
        for (int nt = 0; nt < NT; nt += NSTEP) {
            const F s0 = *reinterpret_cast<const F *>(stb + ((nt * PT + pt) * 64 + lane) * 4);
            if constexpr (sizeof(T) == 2) {
                const F s1 = *reinterpret_cast<const F *>(stb + (((nt + 1) * PT + pt) * 64 + lane) * 4);
#pragma unroll
                for (int ri = 0; ri < 2; ++ri)
                    acc[ri][pt] = mma_pair(s0, cf[ri][nt], s1, cf[ri][nt + 1], acc[ri][pt]);
            } else {
#pragma unroll
                for (int ri = 0; ri < 2; ++ri) acc[ri][pt] = mma_one(s0, cf[ri][nt], acc[ri][pt]);
            }
        }
        hook(1 + pt, nbuf, ys);
    }
    const S ci0 = cm[I0 * 16 + col], ci1 = cm[I1 * 16 + col];
    {
        const float gi0 = exp2_fast((float)ci0), gi1 = exp2_fast((float)ci1);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[0][pt][r] *= gi0;
                acc[1][pt][r] *= gi1;
            }
    }

    // by_intra: pairs of slots, each pair feeding one of the two row blocks
#pragma unroll
    for (int q = 0; q < Cfg::NPAIR; ++q) {
        F a[2];
        int Jx[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int s = 2 * q + u;
            const Slot sl = slot_of(s, w, NRB);
            const S ci = sl.first ? ci0 : ci1;
            Jx[u] = sl.J;
            f32x4 m;
            if (sl.pad) {                                   // uniform: the zero pad slot
                m = zero_frag<f32x4>();
            } else if (sl.J < sl.I) {                       // uniform: off-diagonal tile
                // 2^(cum_i - cum_{e_J}) times dblk_j; cum is non-increasing (dt A <= 0), so
                // both factors are <= 1
                const float f = exp2_fast((float)(ci - cm[sl.J * 16 + 15]));
                const f32x4 dl = *reinterpret_cast<const f32x4 *>(dlk + sl.J * 16 + g4);
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] = sT[s][r] * (f * dl[r]);
            } else {                                        // diagonal (masked in S^T)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    m[r] = sT[s][r] * exp2_fast(fminf((float)(ci - cm[sl.J * 16 + g4 + r]), 0.f));
            }
            a[u] = frag_from_f32<T>(m);
        }
        const bool owner1 = (2 * q) >= (w + 1);             // uniform
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const F x0 = x_frag<T, Cfg::PV>(xs, Jx[0], pt, lane);
            const F x1 = x_frag<T, Cfg::PV>(xs, Jx[1], pt, lane);
            if (owner1) acc[1][pt] = mma_pair(x0, a[0], x1, a[1], acc[1][pt]);
            else acc[0][pt] = mma_pair(x0, a[0], x1, a[1], acc[0][pt]);
        }
        hook(1 + PT + q, nbuf, ys);
    }

    // + (D + residual) x on the matrix cores: B operand diag(D + res) split into a high
    // and a low part in the operand dtype, A operand the x fragments of the diagonal block.
    {
        F dhi, dlo;
        const float hi = to_f32(from_f32<T>(dres)), lo = dres - hi;   // uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dhi[e] = from_f32<T>((g4 + e == col) ? hi : 0.f);
            dlo[e] = from_f32<T>((g4 + e == col) ? lo : 0.f);
        }
#pragma unroll
        for (int ri = 0; ri < 2; ++ri) {
            const int I = ri ? I1 : I0;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                // K = 16 products: x's fragment is the A operand as it is (a K = 32 product
                // would need it twice in consecutive registers)
                const F xv = x_frag<T, Cfg::PV>(xs, I, pt, lane);
                acc[ri][pt] = mma_one(xv, dhi, acc[ri][pt]);
                if constexpr (sizeof(T) == 2) acc[ri][pt] = mma_one(xv, dlo, acc[ri][pt]);
            }
        }
    }
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((ScanCfg<T, Q, P, N>::THREADS)) void chunk_scan_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.y);
    using Cfg = ScanCfg<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int NW = Cfg::NW;
    constexpr int NRB = Cfg::NRB, NSLOT = Cfg::NSLOT, PT = Cfg::PT, NT = Cfg::NT;
    constexpr int XPIECES = Cfg::XPIECES, YPIECES = Cfg::YPIECES;
    constexpr int PS = Cfg::PS, PV = Cfg::PV;    // units per head, channels per unit
    // memory work per head and wave, in single-instruction items (Cfg): XK x pieces, SK
    // b_in pieces, one cum row, one dblk row, then NSTQ staged-output stores
    constexpr int XK = Cfg::XK, SK = Cfg::SK, NDMA = Cfg::NDMA, NSTQ = Cfg::NSTQ;
    constexpr int NHOOK = 1 + PT + Cfg::NPAIR;
    constexpr int NITEM = NDMA + (Cfg::STAGED ? NSTQ : 0);
    static_assert(NSTQ * 64 == 32 * YPIECES, "output rows must fill whole store instructions");
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int col = lane & 15, g4 = 4 * (lane >> 4);
    const int hpg = p.H / p.G;
    const int hg_per_group = (hpg + p.heads_per_wg_scan - 1) / p.heads_per_wg_scan;
    const int nhg = p.G * hg_per_group;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int hgi = logical % nhg;
    const int bc = logical / nhg;
    const int c = bc % p0.nc, b = bc / p0.nc;     // grid layout: chunks of the longest step
    if (c >= p.nc) return;                        // past a short last segment (uniform)
    const int grp = hgi / hg_per_group;
    const int h0 = grp * hpg + (hgi % hg_per_group) * p.heads_per_wg_scan;
    const int h1 = min(h0 + p.heads_per_wg_scan, (grp + 1) * hpg);
    const int t0 = c * Q;
    const int Qc = min(Q, p.L - t0);
    const int HP = p.H * P;
    const int64_t PN = (int64_t)P * N;
    const int64_t bcp = (int64_t)p.G * N;
    const int I0 = w, I1 = NRB - 1 - w;

    const unsigned char *xchunk = reinterpret_cast<const unsigned char *>(p.x) +
                                  ((int64_t)b * p.x_bs + (int64_t)t0 * HP) * (int64_t)sizeof(T);
    // Per-lane byte offsets of this lane's x pieces inside one unit's slice of the chunk
    // (the same for every unit: the unit only moves the uniform base), kept in 32 bits
    // (the host bounds a chunk's span of x, Q * H * P * sizeof(T), below 2^31).
    const uint32_t xrow = (uint32_t)(HP * (int)sizeof(T)), xunit = (uint32_t)(PV * (int)sizeof(T));
    const uint32_t xhead = (uint32_t)(P * (int)sizeof(T));
    uint32_t xoff[XK];
#pragma unroll
    for (int k = 0; k < XK; ++k) {
        const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, XPIECES, sizeof(T) == 2);
        const int rr = min(d.row, Qc - 1);                      // rows past a short chunk repeat the last
        xoff[k] = (uint32_t)rr * xrow + (uint32_t)(d.piece * 16);
    }
    // DMA item k of unit (h, half) into buffer buf (indices from ssd_index.h): x pieces,
    // then b_in pieces, then the cum row (waves from 0 up) and the dblk row (waves from
    // NW - 1 down).  Each source is one buffer covering exactly this (head, chunk)'s data
    // (x: the unit's channels).
    auto dma_item = [&](int k, int h, int half, unsigned char *buf) {
        if (k < XK) {
            const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, XPIECES, sizeof(T) == 2);
            if (d.on)                                           // uniform (whole waves of pieces)
                dma16_buf(make_rsrc(xchunk + (int64_t)h * xhead + half * xunit, (uint32_t)(Qc - 1) * xrow + xunit),
                          xoff[k], buf + d.lds - lane * 16);
        } else if (k < XK + SK) {
            const DmaPiece d = scan_flat_piece(k - XK, w, lane, NW, Cfg::SP);
            if (d.on) {
                const unsigned char *sv = reinterpret_cast<const unsigned char *>(p.b_in) +
                                          (((int64_t)b * p.nc + c) * p.H + h) * PN * (int64_t)sizeof(T);
                const int src = PS == 1 ? d.piece : scan_state_src_piece(d.piece, half, PT, Cfg::PTH, Cfg::TP);
                dma16_buf(make_rsrc(sv, Cfg::STH), (uint32_t)(src * 16), buf + Cfg::O_ST + d.lds - lane * 16);
            }
        } else {
            const int64_t tok = (((int64_t)b * p.H + h) * p.nc + c) * Q;
            if (k == XK + SK) {                                 // cum row
                const DmaPiece d = scan_row_piece(w, lane, Cfg::CP);
                if (d.on)
                    dma16_buf(make_rsrc(reinterpret_cast<const S *>(p.dA_cum) + tok, Cfg::CM),
                              (uint32_t)(d.piece * 16), buf + Cfg::O_CM + d.lds - lane * 16);
            } else {                                            // dblk row
                const DmaPiece d = scan_row_piece(NW - 1 - w, lane, Cfg::DP);
                if (d.on)
                    dma16_buf(make_rsrc(p.dblk + tok, Cfg::DL), (uint32_t)(d.piece * 16),
                              buf + Cfg::O_DL + d.lds - lane * 16);
            }
        }
    };
    // the x, state and B pieces always fill whole waves, so their guards are uniform
    static_assert((Q * XPIECES) % 64 == 0 && Cfg::SP % 64 == 0 && (Q * Cfg::BPIECES) % 64 == 0,
                  "x, state and B tiles are whole waves of 16-byte pieces");

    T *ychunk = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_bs + (int64_t)t0 * HP;
    unsigned char *ys = smem + (Cfg::DB ? 2 : 1) * Cfg::HEAD_BYTES + (Cfg::YS ? w * Cfg::YW : 0);
    // Store item k of head hs: 64 pieces of this wave's staged rows, 16 bytes per lane,
    // whole output rows per group of YPIECES lanes; per-lane byte offsets inside one head's
    // slice of the chunk (32 bits, as for x).
    uint32_t yoff[NSTQ];
#pragma unroll
    for (int k = 0; k < NSTQ; ++k) {
        const DmaPiece d = scan_y_piece(k, lane, YPIECES, Cfg::IP, w, NW);
        const int i = (d.row < 16 ? I0 : I1) * 16 + (d.row & 15);
        yoff[k] = (uint32_t)i * (uint32_t)(HP * (int)sizeof(T)) + (uint32_t)(d.piece * 16);
    }
    auto store_item = [&](int k, int hs, int half, const unsigned char *ys) {
        const DmaPiece d = scan_y_piece(k, lane, YPIECES, Cfg::IP, w, NW);
        const int i = (d.row < 16 ? I0 : I1) * 16 + (d.row & 15);
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ys + d.lds);
        // y is written once and not read again in this step: non-temporal.  Only the last
        // chunk can be short, so full chunks skip the per-lane row check.
        const rsrc_t r = make_rsrc(ychunk + (int64_t)hs * P + half * PV, (uint32_t)(Qc - 1) * xrow + xunit);
        if (Qc == Q || i < Qc) __builtin_amdgcn_raw_buffer_store_b128(v, r, yoff[k], 0, kCachePolicyNT);
    };

#pragma unroll
    for (int k = 0; k < NDMA; ++k) dma_item(k, h0, 0, smem);

    // ---- per workgroup: this wave's C fragments, then its causal S^T = B C^T tiles
    constexpr int NSTEP = sizeof(T) == 2 ? 2 : 1;
    F cf[2][NT];
    {
        const T *Cb = reinterpret_cast<const T *>(p.C) + (int64_t)b * p.bc_bs + (int64_t)t0 * bcp + grp * N;
#pragma unroll
        for (int ri = 0; ri < 2; ++ri) {
            const int i = (ri ? I1 : I0) * 16 + col;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                cf[ri][nt] = (i < Qc) ? *reinterpret_cast<const F *>(Cb + (int64_t)i * bcp + nt * 16 + g4)
                                      : zero_frag<F>();
        }
    }
    // Tile (I, J): rows j of block J (A operand: B[j][n], lane (col, g) holding 4
    // consecutive n), columns i of block I (B operand: the C fragments above); output
    // lane (col, g) value r holds S^T[16J + 4g + r][16I + col].  Rows past a short chunk
    // are zero.
    f32x4 sT[NSLOT];
    {
        const T *Bb = reinterpret_cast<const T *>(p.B) + (int64_t)b * p.bc_bs + (int64_t)t0 * bcp + grp * N;
        // B fragment of row j, columns n0..n0+3: from the staged tile (piece q of row j at
        // position q ^ bsw(j), so the 16 rows read by one load hit different banks) or
        // from L2.
        constexpr int BMASK = b_mask(Cfg::BPIECES);
        const unsigned char *bst = smem + Cfg::HEAD_BYTES;
        auto bfrag = [&](int j, int n0) -> F {
            if (j >= Qc) return zero_frag<F>();
            if constexpr (Cfg::BL) {
                const int byte = n0 * (int)sizeof(T);
                const int pos = (byte >> 4) ^ (j & BMASK);
                return *reinterpret_cast<const F *>(bst + (j * Cfg::BPIECES + pos) * 16 + (byte & 15));
            } else {
                return *reinterpret_cast<const F *>(Bb + (int64_t)j * bcp + n0);
            }
        };
        if constexpr (Cfg::BL) {
            // DMA the tile (rows past a short chunk repeat the last row; bfrag zeroes them)
            const unsigned char *bsrc = reinterpret_cast<const unsigned char *>(Bb);
#pragma unroll
            for (int k = 0; k < Cfg::BK; ++k) {
                const DmaPiece d = scan_b_piece(k, w, lane, NW, Q, Cfg::BPIECES);
                if (d.on)                                       // uniform
                    dma16(bsrc + (int64_t)min(d.row, Qc - 1) * bcp * (int64_t)sizeof(T) + d.piece * 16,
                          smem + Cfg::HEAD_BYTES + d.lds - lane * 16);
            }
            __builtin_amdgcn_s_waitcnt(0);    // the tile (and the first head's inputs) landed
            __builtin_amdgcn_s_barrier();
        }
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
            const Slot sl = slot_of(s, w, NRB);
            f32x4 t = zero_frag<f32x4>();
            if (!sl.pad) {                                       // uniform
                const int j = sl.J * 16 + col;
                const int ri = sl.first ? 0 : 1;
#pragma unroll
                for (int nt = 0; nt < NT; nt += NSTEP) {
                    const F a0 = bfrag(j, nt * 16 + g4);
                    if constexpr (sizeof(T) == 2) {
                        const F a1 = bfrag(j, (nt + 1) * 16 + g4);
                        t = ri ? mma_pair(a0, cf[1][nt], a1, cf[1][nt + 1], t)
                               : mma_pair(a0, cf[0][nt], a1, cf[0][nt + 1], t);
                    } else {
                        t = ri ? mma_one(a0, cf[1][nt], t) : mma_one(a0, cf[0][nt], t);
                    }
                }
                if (sl.J == sl.I) {                              // uniform: diagonal tile
#pragma unroll
                    for (int r = 0; r < 4; ++r) t[r] = (g4 + r <= col) ? t[r] : 0.f;
                }
            }
            sT[s] = t;
        }
        // The staged tile sits in the second head buffer and the staging rows; the barrier
        // at the top of the head loop orders these reads before the first DMA into them.
    }

    const float res = (p.flags & 1u) ? 1.f : 0.f;
    // In-place staging (Cfg::IP): a unit's rounded outputs wait in registers until the top
    // of the next unit, when every wave is past the finished buffer; each wave then writes
    // them into its own x slots there, stores them, and only then copies the unit after
    // next into that buffer (after its own reads of the staged rows: lgkmcnt(0)).
    F yres[2][PT];
    auto stage = [&](unsigned char *area) {
#pragma unroll
        for (int ri = 0; ri < 2; ++ri)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int row = ri * 16 + col;
                const int byte = (pt * 16 + g4) * (int)sizeof(T);
                *reinterpret_cast<F *>(area + scan_y_stage(row, byte, YPIECES, true, w, NW)) = yres[ri][pt];
            }
    };
    constexpr int kWaitLds = 0xC07F;          // s_waitcnt lgkmcnt(0) alone (vmcnt 63, expcnt 7)
    // units (h, half): head h, channels [half PV, (half + 1) PV)
    for (int h = h0, half = 0, it = 0; h < h1; ++it) {
        const int hn = half + 1 < PS ? h : h + 1, halfn = half + 1 < PS ? half + 1 : 0;   // next unit
        const int hp = half > 0 ? h : h - 1, halfp = half > 0 ? half - 1 : PS - 1;       // previous unit
        unsigned char *buf = smem + (Cfg::DB ? (it & 1) * Cfg::HEAD_BYTES : 0);
        unsigned char *nbuf = smem + (Cfg::DB ? ((it + 1) & 1) * Cfg::HEAD_BYTES : 0);
        __builtin_amdgcn_s_waitcnt(0);        // this unit's DMA (and older stores) complete
        __builtin_amdgcn_s_barrier();         // ... for every wave; the other buffer is free
        const bool more = hn < h1;
        if constexpr (Cfg::IP) {
            if (it > 0) stage(nbuf);          // the previous unit's outputs, into its own buffer
        }
        // Item k: the next unit's DMA (double buffer), then the previous unit's staged stores;
        // staged in place, the stores come first.
        auto hook = [&](int k, unsigned char *nb, const unsigned char *yst) {
            if constexpr (Cfg::IP) {
                if (k < NSTQ) {
                    if (it > 0) store_item(k, hp, halfp, nb);
                } else if (k < NITEM) {
                    if (more) {
                        if (k == NSTQ && it > 0) __builtin_amdgcn_s_waitcnt(kWaitLds);
                        dma_item(k - NSTQ, hn, halfn, nb);
                    }
                }
            } else {
                if (k < NDMA) {
                    if (Cfg::DB && more) dma_item(k, hn, halfn, nb);
                } else if (k < NITEM) {
                    if (Cfg::YS && it > 0) store_item(k - NDMA, hp, halfp, yst);
                }
            }
        };
        const float dres = (p.D ? p.D[h] : 0.f) + res;
        f32x4 acc[2][PT];
        switch (w) {   // uniform: every wave runs the body specialised for its own index
#define SSD_W(WW) case WW: if constexpr (WW < NW) scan_head<T, Q, P, N, WW>(buf, nbuf, ys, sT, cf, dres, lane, acc, hook); break;
            SSD_W(0) SSD_W(1) SSD_W(2) SSD_W(3) SSD_W(4) SSD_W(5) SSD_W(6) SSD_W(7)
#undef SSD_W
            default: break;
        }
#pragma unroll
        for (int k = NHOOK; k < NITEM; ++k) hook(k, nbuf, ys);   // items the body had no room for

        if constexpr (Cfg::YS) {
            // rounded outputs into this wave's staging rows; stored during the next unit
#pragma unroll
            for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int row = ri * 16 + col;
                    const int byte = (pt * 16 + g4) * (int)sizeof(T);
                    *reinterpret_cast<F *>(ys + scan_y_stage(row, byte, YPIECES)) = frag_from_f32<T>(acc[ri][pt]);
                }
        } else if constexpr (Cfg::IP) {
#pragma unroll
            for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) yres[ri][pt] = frag_from_f32<T>(acc[ri][pt]);
        } else {
            T *yh = ychunk + h * P + half * PV;
#pragma unroll
            for (int ri = 0; ri < 2; ++ri) {
                const int i = (ri ? I1 : I0) * 16 + col;
                if (i < Qc) {
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        *reinterpret_cast<F *>(yh + (int64_t)i * HP + pt * 16 + g4) = frag_from_f32<T>(acc[ri][pt]);
                }
            }
        }
        if (!Cfg::DB && more) {               // single buffer: refill after every wave is done
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int k = 0; k < NDMA; ++k) dma_item(k, hn, halfn, smem);
        }
        h = hn;
        half = halfn;
    }
    if constexpr (Cfg::YS) {                  // last unit's staged outputs (own rows: no barrier)
#pragma unroll
        for (int k = 0; k < NSTQ; ++k) store_item(k, h1 - 1, PS - 1, ys);
    }
    if constexpr (Cfg::IP) {                  // last unit: staged once every wave is past its x
        unsigned char *last = smem + (((h1 - h0) * PS - 1) & 1) * Cfg::HEAD_BYTES;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        stage(last);
#pragma unroll
        for (int k = 0; k < NSTQ; ++k) store_item(k, h1 - 1, PS - 1, last);
    }
}

template <typename T, int Q, int P, int N>
static hipError_t launch_scan_t(const Problem &p, hipStream_t s) {
    using Cfg = ScanCfg<T, Q, P, N>;
    if constexpr (!Cfg::OK) {
        return hipErrorInvalidValue;
    } else {
        if (const hipError_t attr = allow_lds<chunk_scan_kernel<T, Q, P, N>>(Cfg::LDS); attr != hipSuccess)
            return attr;
        const int hpg = p.H / p.G;
        const int nhg = p.G * ((hpg + p.heads_per_wg_scan - 1) / p.heads_per_wg_scan);
        const int64_t nblk = (int64_t)p.batch * p.nc * nhg;
        if (nblk <= 0 || nblk > 0x7fffffff) return hipErrorInvalidValue;
        chunk_scan_kernel<T, Q, P, N><<<dim3((unsigned)nblk, step_count(p)), Cfg::THREADS, Cfg::LDS, s>>>(p);
        return hipGetLastError();
    }
}

#define SSD_SCAN_CASE(T, q, pp, nn) \
    if (p.Q == q && p.P == pp && p.N == nn) return launch_scan_t<T, q, pp, nn>(p, s);
#define SSD_SCAN_OK(T, q, pp, nn) \
    if (Q == q && P == pp && N == nn) return ScanCfg<T, q, pp, nn>::OK;

hipError_t launch_chunk_scan(const Problem &p, hipStream_t s) {
    if (p.dtype == 1) { SSD_SCAN_SHAPES(SSD_SCAN_CASE, bf16) }
    else { SSD_SCAN_SHAPES(SSD_SCAN_CASE, float) }
    return hipErrorInvalidValue;
}

bool chunk_scan_supported(int dtype, int Q, int P, int N) {
    if (dtype == 1) {
        if (N % 32 != 0) return false;
        SSD_SCAN_SHAPES(SSD_SCAN_OK, bf16)
    } else {
        SSD_SCAN_SHAPES(SSD_SCAN_OK, float)
    }
    return false;
}

}  // namespace ssd

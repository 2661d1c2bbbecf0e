// chunk_scan: every chunk's output, [分块推理 §2.1-§2.2] of the page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理":
//
//   by_intra_i = sum_{j <= i} (C_i . B_j) exp(cum_i - cum_j) x_j      (zero-state intra part)
//   by_inter_i = exp(cum_i) (b(c-1) C_i)                               (diag(L) C(c) b(c-1))
//   y_i        = by_intra_i + by_inter_i + D x_i  (+ x_i with SSD_FLAG_RESIDUAL)
//
// rounded once to the activation dtype.  cum is the chunk's dA_cum row and b(c-1) is
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
// Per head, x is brought into LDS by DMA (tokens x channels, read back as transposed
// fragments), b_in likewise, and the chunk's log-decay prefix sums cum.  The products are
// computed transposed (y^T[p][i]) so that a lane's 4 accumulator values are 4 consecutive
// channels of one token:
//     Z^T = b(c-1) C^T, column i scaled by G_i = exp(cum_i);
//     y^T += x^T (S^T . decay), the decay of tile entry (j, i) being exp(cum_i - cum_j):
//       <= 1 below the diagonal (cum is non-increasing), and exp(min(cum_i - cum_j, 0)) on
//       diagonal tiles (the zeroed upper triangle of S^T does the masking); a lane's 4 S^T
//       values are 4 consecutive k values of the B operand, so no data moves between
//       lanes;
//     y^T += x^T diag(D + residual) on the matrix cores (D split in a high and a low bf16
//       part so the skip term keeps fp32 accuracy; K = 16 products).
// Tiles are paired into 16x16x32 bf16 products (16x16x4 f32 for the fp32 dtype).
#include "ssd_common.h"

namespace ssd {

template <typename T, int Q, int P, int N>
struct ScanCfg {
    static constexpr int NRB = Q / 16, NW = NRB / 2, THREADS = NW * 64;
    static constexpr int NSLOT = NRB + 2, NPAIR = NSLOT / 2;
    static constexpr int NTRI = NRB * (NRB + 1) / 2;            // causal tiles per chunk
    static constexpr int PT = P / 16, NT = N / 16;
    // one head's inputs in LDS: x tile, b(c-1) tile, cum row (the layout of HeadBuf)
    static constexpr int HEAD_BYTES = Q * P * (int)sizeof(T) + P * N * (int)sizeof(T) +
                                      Q * (int)sizeof(typename CumT<T>::type);
    static constexpr bool DB = 2 * HEAD_BYTES <= kLdsBytes;     // double-buffered head data
    static constexpr int YPIECES = P * (int)sizeof(T) / 16;      // 16-byte pieces per output row
    static constexpr int YW = 32 * P * (int)sizeof(T);           // one wave's staged outputs
    static constexpr bool YS = DB && 2 * HEAD_BYTES + NW * YW <= kLdsBytes;
    static constexpr int LDS = (DB ? 2 * HEAD_BYTES : HEAD_BYTES) + (YS ? NW * YW : 0);
    // The chunk's B tile (Q x N) is staged in LDS for the S^T products when it fits beside
    // the first head's buffer; otherwise the B fragments are loaded from L2.
    static constexpr int BPIECES = N * (int)sizeof(T) / 16;      // 16-byte pieces per B row
    static constexpr bool BL = DB && Q * N * (int)sizeof(T) <= LDS - HEAD_BYTES;
    static constexpr bool OK = LDS <= kLdsBytes &&
                               (sizeof(T) == 4 || NT % 2 == 0) && (Q == 32 || Q == 64 || Q == 128 || Q == 256) &&
                               P * (int)sizeof(T) >= 32;
};

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
// Raw LDS pointers for the gfx950 LDS-DMA and transpose-read builtins.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// 16-byte global -> LDS copy: lane l of the wave writes lds_base + 16 * l.  The copies
// carry the non-temporal cache policy: every stream this kernel reads is used once per
// step (measured: the whole step is ~4% faster with the streams marked so).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 16, 0, kCachePolicyNT);
}

// x tile in LDS: row-major [Q][P] in 16-byte pieces; piece q of row r is stored at
// position q ^ swz(r) of that row, which spreads the 4 rows read by one transpose load
// over different banks.
template <int PIECES>
__device__ __forceinline__ int x_swz(int r) { return (((r >> 1) & 3) << 1) & (PIECES - 1); }

// A operand fragment of x^T for (16-token block J, 16-channel tile pt): lane (col, g) gets
// x[16J + 4g + e][16pt + col], e = 0..3.
template <typename T, int P>
__device__ __forceinline__ typename TF<T>::type x_frag(const unsigned char *xs, int J, int pt, int lane);

template <>
__device__ __forceinline__ bf16x4 x_frag<bf16, 16>(const unsigned char *xs, int J, int pt, int lane) {
    constexpr int P = 16, PIECES = P * 2 / 16;
    const int s = lane & 15, g = lane >> 4;
    const int r = J * 16 + 4 * g + (s >> 2);
    const int c = pt * 16 + 4 * (s & 3);
    const int q = (c >> 3) ^ x_swz<PIECES>(r);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(xs + r * (P * 2) + q * 16 + (c & 7) * 2));
}
#define SSD_XFRAG_BF16(PP)                                                                           \
    template <>                                                                                      \
    __device__ __forceinline__ bf16x4 x_frag<bf16, PP>(const unsigned char *xs, int J, int pt, int lane) { \
        constexpr int PIECES = PP * 2 / 16;                                                          \
        const int s = lane & 15, g = lane >> 4;                                                      \
        const int r = J * 16 + 4 * g + (s >> 2);                                                     \
        const int c = pt * 16 + 4 * (s & 3);                                                         \
        const int q = (c >> 3) ^ x_swz<PIECES>(r);                                                   \
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(xs + r * (PP * 2) + q * 16 + (c & 7) * 2)); \
    }
SSD_XFRAG_BF16(32)
SSD_XFRAG_BF16(64)
SSD_XFRAG_BF16(128)
#undef SSD_XFRAG_BF16

// fp32: no transpose load for 32-bit data; four scalar reads (no swizzle for fp32 tiles).
#define SSD_XFRAG_F32(PP)                                                                            \
    template <>                                                                                      \
    __device__ __forceinline__ f32x4 x_frag<float, PP>(const unsigned char *xs, int J, int pt, int lane) { \
        const int col = lane & 15, g = lane >> 4;                                                    \
        const float *base = reinterpret_cast<const float *>(xs) + (J * 16 + 4 * g) * PP + pt * 16 + col; \
        f32x4 v;                                                                                     \
        v[0] = base[0]; v[1] = base[PP]; v[2] = base[2 * PP]; v[3] = base[3 * PP];                   \
        return v;                                                                                    \
    }
SSD_XFRAG_F32(16)
SSD_XFRAG_F32(32)
SSD_XFRAG_F32(64)
SSD_XFRAG_F32(128)
#undef SSD_XFRAG_F32

template <typename T, int Q, int P, int N>
struct HeadBuf {
    typedef typename CumT<T>::type S;
    static constexpr int X = Q * P * (int)sizeof(T);
    static constexpr int ST = P * N * (int)sizeof(T);
    static constexpr int CM = Q * (int)sizeof(S);
    static constexpr int O_ST = X, O_CM = X + ST;
    static constexpr int BYTES = O_CM + CM;
};

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
    using Buf = HeadBuf<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int NRB = Cfg::NRB, PT = Cfg::PT, NT = Cfg::NT;
    constexpr int NSTEP = sizeof(T) == 2 ? 2 : 1;
    constexpr int w = W, I0 = W, I1 = NRB - 1 - W;
    const int col = lane & 15, g4 = 4 * (lane >> 4);
    const unsigned char *xs = buf;
    const T *stb = reinterpret_cast<const T *>(buf + Buf::O_ST);
    const S *cm = reinterpret_cast<const S *>(buf + Buf::O_CM);

    // Output tiles are transposed: acc[ri][pt] lane (col, g), value r holds
    // y^T[p = pt*16 + 4g + r][i = I*16 + col].
    // Z^T = b(c-1) C^T, then column i scaled by G_i = exp(cum_i)
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
        const float gi0 = __expf((float)ci0), gi1 = __expf((float)ci1);
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
            if (sl.J < sl.I) {                              // uniform: off-diagonal tile or pad
                // cum is non-increasing (dt A <= 0), so ci - cum_j <= 0 here
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] = sT[s][r] * __expf((float)(ci - cm[sl.J * 16 + g4 + r]));
            } else {                                        // diagonal (masked in S^T)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    m[r] = sT[s][r] * __expf(fminf((float)(ci - cm[sl.J * 16 + g4 + r]), 0.f));
            }
            a[u] = frag_from_f32<T>(m);
        }
        const bool owner1 = (2 * q) >= (w + 1);             // uniform
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const F x0 = x_frag<T, P>(xs, Jx[0], pt, lane);
            const F x1 = x_frag<T, P>(xs, Jx[1], pt, lane);
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
                const F xv = x_frag<T, P>(xs, I, pt, lane);
                acc[ri][pt] = mma_one(xv, dhi, acc[ri][pt]);
                if constexpr (sizeof(T) == 2) acc[ri][pt] = mma_one(xv, dlo, acc[ri][pt]);
            }
        }
    }
}

// Staged outputs of one wave: 32 rows (its two row blocks) of YPIECES 16-byte pieces;
// piece q of row r sits at position q ^ ysw(r), so the fragment writes and the row reads
// both spread over all banks.
template <int YPIECES>
__device__ __forceinline__ int ysw(int r) { return r & ((YPIECES < 8 ? YPIECES : 8) - 1); }

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((ScanCfg<T, Q, P, N>::THREADS)) void chunk_scan_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.y);
    using Cfg = ScanCfg<T, Q, P, N>;
    using Buf = HeadBuf<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int THREADS = Cfg::THREADS, NW = Cfg::NW;
    constexpr int NRB = Cfg::NRB, NSLOT = Cfg::NSLOT, PT = Cfg::PT, NT = Cfg::NT;
    constexpr int XPIECES = P * (int)sizeof(T) / 16;          // 16-byte pieces per x row
    constexpr int YPIECES = Cfg::YPIECES;
    // memory work per head and wave, in single-instruction items:
    constexpr int XK = (Q * XPIECES + THREADS - 1) / THREADS;           // x tile
    constexpr int SP = Buf::ST / 16, SK = (SP + THREADS - 1) / THREADS;  // b_in state
    constexpr int CP = Buf::CM / 16;                                     // cum
    constexpr int NDMA = XK + SK + 1;
    constexpr int NSTQ = 32 * YPIECES / 64;                               // staged-output stores
    constexpr int NHOOK = 1 + PT + Cfg::NPAIR;
    constexpr int NITEM = NDMA + (Cfg::YS ? NSTQ : 0);
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
    // DMA item k of head h into buffer buf: x pieces, then b_in pieces, then cum/F/G.
    // Lane l of the wave fills LDS bytes [16 l, 16 l + 16) of the item's 1 KB block.
    auto dma_item = [&](int k, int h, unsigned char *buf) {
        if (k < XK) {
            const int piece = (k * NW + w) * 64 + lane;
            if ((k * NW + w) * 64 < Q * XPIECES) {              // uniform (Q * XPIECES % 64 == 0)
                const int r = piece / XPIECES, qp = piece % XPIECES;
                const int q = qp ^ (sizeof(T) == 2 ? x_swz<XPIECES>(r) : 0);
                const int rr = min(r, Qc - 1);                  // rows past a short chunk repeat the last
                dma16(xchunk + ((int64_t)rr * HP + (int64_t)h * P) * (int64_t)sizeof(T) + q * 16,
                      buf + (k * NW + w) * 1024);
            }
        } else if (k < XK + SK) {
            const int kk = k - XK;
            if ((kk * NW + w) * 64 < SP) {
                const unsigned char *sv = reinterpret_cast<const unsigned char *>(p.b_in) +
                                          (((int64_t)b * p.nc + c) * p.H + h) * PN * (int64_t)sizeof(T);
                dma16(sv + ((kk * NW + w) * 64 + lane) * 16, buf + Buf::O_ST + (kk * NW + w) * 1024);
            }
        } else {
            // cum of one (head, chunk) is CP 16-byte pieces, which need not fill whole
            // waves (Q < 256 for bf16): the guard is per lane, so no lane reads past the row
            // or writes past its LDS region
            const int64_t tok = (((int64_t)b * p.H + h) * p.nc + c) * Q;
            const int pc = w * 64 + lane;
            // a per-wave test where the pieces fill whole waves (no exec-mask branch)
            if ((CP % 64 == 0) ? (w * 64 < CP) : (pc < CP))
                dma16(reinterpret_cast<const unsigned char *>(reinterpret_cast<const S *>(p.dA_cum) + tok) + pc * 16,
                      buf + Buf::O_CM + w * 1024);
        }
    };
    static_assert(CP <= THREADS, "cum fits one DMA item");
    static_assert(Buf::BYTES == Cfg::HEAD_BYTES, "head buffer layout and LDS sizing agree");
    // the x, state and B pieces always fill whole waves, so their guards are uniform
    static_assert((Q * XPIECES) % 64 == 0 && SP % 64 == 0 && (Q * Cfg::BPIECES) % 64 == 0,
                  "x, state and B tiles are whole waves of 16-byte pieces");

    T *ychunk = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_bs + (int64_t)t0 * HP;
    unsigned char *ys = smem + (Cfg::DB ? 2 : 1) * Buf::BYTES + (Cfg::YS ? w * Cfg::YW : 0);
    // Store item k of head hs: 64 pieces of this wave's staged rows, 16 bytes per lane,
    // whole output rows per group of YPIECES lanes.
    auto store_item = [&](int k, int hs, const unsigned char *ys) {
        const int pc = k * 64 + lane;
        const int row = pc / YPIECES, q = pc % YPIECES;
        const int i = (row < 16 ? I0 : I1) * 16 + (row & 15);
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = *reinterpret_cast<const u32x4 *>(ys + (row * YPIECES + (q ^ ysw<YPIECES>(row))) * 16);
        // y is written once and not read again in this step: non-temporal.  Only the last
        // chunk can be short, so full chunks skip the per-lane row check.
        u32x4 *dst = reinterpret_cast<u32x4 *>(ychunk + (int64_t)i * HP + (int64_t)hs * P + q * (16 / (int)sizeof(T)));
        if (Qc == Q) __builtin_nontemporal_store(v, dst);
        else if (i < Qc) __builtin_nontemporal_store(v, dst);
    };

#pragma unroll
    for (int k = 0; k < NDMA; ++k) dma_item(k, h0, smem);

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
        constexpr int BMASK = (Cfg::BPIECES < 16 ? Cfg::BPIECES : 16) - 1;
        const unsigned char *bst = smem + Buf::BYTES;
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
            constexpr int BK = (Q * Cfg::BPIECES + THREADS - 1) / THREADS;
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                if ((k * NW + w) * 64 < Q * Cfg::BPIECES) {     // uniform
                    const int slot = (k * NW + w) * 64 + lane;
                    const int j = slot / Cfg::BPIECES, q = (slot % Cfg::BPIECES) ^ (j & BMASK);
                    dma16(bsrc + (int64_t)min(j, Qc - 1) * bcp * (int64_t)sizeof(T) + q * 16,
                          smem + Buf::BYTES + (k * NW + w) * 1024);
                }
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
    for (int h = h0, it = 0; h < h1; ++h, ++it) {
        unsigned char *buf = smem + (Cfg::DB ? (it & 1) * Buf::BYTES : 0);
        unsigned char *nbuf = smem + (Cfg::DB ? ((it + 1) & 1) * Buf::BYTES : 0);
        __builtin_amdgcn_s_waitcnt(0);        // this head's DMA (and older stores) complete
        __builtin_amdgcn_s_barrier();         // ... for every wave; the other buffer is free
        const bool more = h + 1 < h1;
        // Item k: the next head's DMA (double buffer), then the previous head's staged stores.
        auto hook = [&](int k, unsigned char *nb, const unsigned char *yst) {
            if (k < NDMA) {
                if (Cfg::DB && more) dma_item(k, h + 1, nb);
            } else if (k < NITEM) {
                if (Cfg::YS && h > h0) store_item(k - NDMA, h - 1, yst);
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
            // rounded outputs into this wave's staging rows; stored during the next head
#pragma unroll
            for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int row = ri * 16 + col;
                    const int byte = (pt * 16 + g4) * (int)sizeof(T);
                    const int q = (byte >> 4) ^ ysw<YPIECES>(row);
                    *reinterpret_cast<F *>(ys + (row * YPIECES + q) * 16 + (byte & 15)) =
                        frag_from_f32<T>(acc[ri][pt]);
                }
        } else {
            T *yh = ychunk + h * P;
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
            for (int k = 0; k < NDMA; ++k) dma_item(k, h + 1, smem);
        }
    }
    if constexpr (Cfg::YS) {                  // last head's staged outputs (own rows: no barrier)
#pragma unroll
        for (int k = 0; k < NSTQ; ++k) store_item(k, h1 - 1, ys);
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

#define SSD_SCAN_SHAPES(X, T)                                                              \
    X(T, 32, 32, 64) X(T, 32, 64, 64) X(T, 32, 64, 128)                                    \
    X(T, 64, 16, 16) X(T, 64, 16, 32) X(T, 64, 16, 64) X(T, 64, 16, 128)                   \
    X(T, 64, 32, 32) X(T, 64, 32, 64) X(T, 64, 32, 128) X(T, 64, 64, 64) X(T, 64, 64, 128) \
    X(T, 128, 32, 64) X(T, 128, 64, 64) X(T, 128, 64, 128)                                 \
    X(T, 256, 16, 32) X(T, 256, 32, 64) X(T, 256, 64, 64) X(T, 256, 64, 128)               \
    X(T, 256, 128, 128) X(T, 256, 64, 256)

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

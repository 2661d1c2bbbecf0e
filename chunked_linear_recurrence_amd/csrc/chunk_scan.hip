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
// Work: one workgroup of Q/32 waves per (batch, chunk, group of heads that read the same
// B/C).  The chunk is cut into Q/16 row blocks of 16 tokens; wave w owns row blocks
// w and Q/16-1-w, so every wave has the same number (Q/16 + 1) of causal 16x16 tiles.
//  1. Once per workgroup: S^T = B_c C_c^T restricted to the causal tiles, on the matrix
//     cores, kept in registers.  It is shared by every head of the group (the decay mask
//     is applied per head afterwards), so C.B^T is computed once per group, not per head.
//     C fragments for the wave's rows also stay in registers.
//  2. Per head: x is transposed into LDS (tokens contiguous per channel), b_in (tile
//     order, read linearly) and the cum row are copied to LDS; double-buffered, with the
//     next head's loads in flight during the current head's products.
//     Z = C b(c-1)^T on the matrix cores, scaled by exp(cum_i) per row, then
//     acc += (S^T . decay)^T x, where each S^T tile is multiplied by exp(cum_i - cum_j)
//     (masked to j <= i) in fp32, rounded to the operand dtype and used directly as the
//     A operand (a lane's 4 consecutive output rows are 4 consecutive k values).
//  3. Epilogue adds D x (and x), rounds, stores y.
// Tiles are paired into 16x16x32 bf16 products (16x16x4 f32 for the fp32 dtype); the
// slot list of a wave is padded with one zero tile so pairs never straddle its two row
// blocks.
#include "ssd_common.h"

namespace ssd {

template <typename T, int Q, int P, int N>
struct ScanCfg {
    static constexpr int NRB = Q / 16, NW = NRB / 2, THREADS = NW * 64;
    static constexpr int NSLOT = NRB + 2, NPAIR = NSLOT / 2;
    static constexpr int PT = P / 16, NT = N / 16;
    static constexpr int RS = Q + 4;
    static constexpr int RJ = 16 / (int)sizeof(T);
    static constexpr int XB = (Q / RJ) * (P / 4);
    static constexpr int XBT = (XB + THREADS - 1) / THREADS;
    static constexpr int SV = P * N * (int)sizeof(T) / 16;       // 16-byte vectors of b_in
    static constexpr int SVT = (SV + THREADS - 1) / THREADS;
    static constexpr int CT = (Q + THREADS - 1) / THREADS;
    static constexpr int XT_BYTES = P * RS * (int)sizeof(T);
    static constexpr int ST_BYTES = P * N * (int)sizeof(T);
    static constexpr int BUF_BYTES = XT_BYTES + ST_BYTES + Q * (int)sizeof(typename CumT<T>::type);
    static constexpr bool DB = 2 * BUF_BYTES <= kLdsBytes;
    static constexpr int LDS = DB ? 2 * BUF_BYTES : BUF_BYTES;
    static constexpr bool OK = BUF_BYTES <= kLdsBytes && (sizeof(T) == 4 || NT % 2 == 0) &&
                               (Q == 64 || Q == 128 || Q == 256);
};

template <typename T, int RJ>
__device__ __forceinline__ void scan_load_block(const T *base, int64_t pitch, int j0, int c0, int rows,
                                                typename TF<T>::type (&r)[RJ]) {
#pragma unroll
    for (int i = 0; i < RJ; ++i) {
        if (j0 + i < rows) r[i] = *reinterpret_cast<const typename TF<T>::type *>(base + (int64_t)(j0 + i) * pitch + c0);
        else r[i] = zero_frag<typename TF<T>::type>();
    }
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((ScanCfg<T, Q, P, N>::THREADS)) void chunk_scan_kernel(Problem p) {
    using Cfg = ScanCfg<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int RJ = Cfg::RJ, RS = Cfg::RS, THREADS = Cfg::THREADS;
    constexpr int NRB = Cfg::NRB, NSLOT = Cfg::NSLOT, PT = Cfg::PT, NT = Cfg::NT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, g4 = 4 * (lane >> 4);
    const int hpg = p.H / p.G;
    const int hg_per_group = (hpg + p.heads_per_wg_scan - 1) / p.heads_per_wg_scan;
    const int nhg = p.G * hg_per_group;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int hgi = logical % nhg;
    const int bc = logical / nhg;
    const int c = bc % p.nc, b = bc / p.nc;
    const int grp = hgi / hg_per_group;
    const int h0 = grp * hpg + (hgi % hg_per_group) * p.heads_per_wg_scan;
    const int h1 = min(h0 + p.heads_per_wg_scan, (grp + 1) * hpg);
    const int t0 = c * Q;
    const int Qc = min(Q, p.L - t0);
    const int HP = p.H * P;
    const int64_t PN = (int64_t)P * N;
    const int64_t bcp = (int64_t)p.G * N;                    // B/C row pitch
    const T *Cb = reinterpret_cast<const T *>(p.C) + (int64_t)b * p.bc_bs + (int64_t)t0 * bcp + grp * N;
    const T *Bb = reinterpret_cast<const T *>(p.B) + (int64_t)b * p.bc_bs + (int64_t)t0 * bcp + grp * N;
    const int I0 = w, I1 = NRB - 1 - w;

    // ---- C fragments of the wave's two row blocks (A operand of Z, B operand of S^T)
    F cf[2][NT];
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
        const int i = (ri ? I1 : I0) * 16 + col;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            cf[ri][nt] = (i < Qc) ? *reinterpret_cast<const F *>(Cb + (int64_t)i * bcp + nt * 16 + g4)
                                  : zero_frag<F>();
    }

    // ---- prefetch of one head's x rows, b_in vectors and cum row
    F xr[Cfg::XBT][RJ];
    uint4 sr[Cfg::SVT];
    S cr[Cfg::CT];
    const T *xbase = reinterpret_cast<const T *>(p.x) + (int64_t)b * p.x_bs + (int64_t)t0 * HP;
    auto prefetch = [&](int h) {
        const T *xh = xbase + h * P;
#pragma unroll
        for (int k = 0; k < Cfg::XBT; ++k) {
            const int blk = tid + k * THREADS;
            if (blk < Cfg::XB) {
                const int jb = blk / (P / 4), pb = blk % (P / 4);
                scan_load_block<T, RJ>(xh, HP, jb * RJ, pb * 4, Qc, xr[k]);
            }
        }
        const uint4 *sv = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const T *>(p.b_in) + (((int64_t)b * p.nc + c) * p.H + h) * PN);
#pragma unroll
        for (int k = 0; k < Cfg::SVT; ++k) {
            const int v = tid + k * THREADS;
            if (v < Cfg::SV) sr[k] = sv[v];
        }
        const S *cu = reinterpret_cast<const S *>(p.dA_cum) + (((int64_t)b * p.H + h) * p.nc + c) * Q;
#pragma unroll
        for (int k = 0; k < Cfg::CT; ++k) {
            const int v = tid + k * THREADS;
            if (v < Q) cr[k] = cu[v];
        }
    };
    auto stage = [&](unsigned char *buf) {
        T *xt = reinterpret_cast<T *>(buf);
        uint4 *st = reinterpret_cast<uint4 *>(buf + Cfg::XT_BYTES);
        S *cm = reinterpret_cast<S *>(buf + Cfg::XT_BYTES + Cfg::ST_BYTES);
#pragma unroll
        for (int k = 0; k < Cfg::XBT; ++k) {
            const int blk = tid + k * THREADS;
            if (blk < Cfg::XB) {
                const int jb = blk / (P / 4), pb = blk % (P / 4);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    F colv[RJ / 4];
#pragma unroll
                    for (int i = 0; i < RJ; ++i) colv[i / 4][i % 4] = xr[k][i][cc];
#pragma unroll
                    for (int q = 0; q < RJ / 4; ++q)
                        *reinterpret_cast<F *>(xt + (pb * 4 + cc) * RS + jb * RJ + 4 * q) = colv[q];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < Cfg::SVT; ++k) {
            const int v = tid + k * THREADS;
            if (v < Cfg::SV) st[v] = sr[k];
        }
#pragma unroll
        for (int k = 0; k < Cfg::CT; ++k) {
            const int v = tid + k * THREADS;
            if (v < Q) cm[v] = cr[k];
        }
    };
    prefetch(h0);

    // ---- S^T tiles of the wave's causal slots: slot s <= w is (I0, J = s); slot w + 1 is
    // a zero pad; slot s >= w + 2 is (I1, J = s - w - 2).
    f32x4 sT[NSLOT];
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
        sT[s] = zero_frag<f32x4>();
        if (s == w + 1) continue;
        const bool first = s <= w;
        const int I = first ? I0 : I1;
        const int J = first ? s : s - w - 2;
        const int j = J * 16 + col;
        const T *brow = Bb + (int64_t)j * bcp + g4;
        const bool jv = j < Qc;
#pragma unroll
        for (int nt = 0; nt < NT; nt += (sizeof(T) == 2 ? 2 : 1)) {
            if constexpr (sizeof(T) == 2) {
                const F b0 = jv ? *reinterpret_cast<const F *>(brow + nt * 16) : zero_frag<F>();
                const F b1 = jv ? *reinterpret_cast<const F *>(brow + (nt + 1) * 16) : zero_frag<F>();
                const F c0 = first ? cf[0][nt] : cf[1][nt];
                const F c1 = first ? cf[0][nt + 1] : cf[1][nt + 1];
                sT[s] = mma_pair(b0, c0, b1, c1, sT[s]);
            } else {
                const F b0 = jv ? *reinterpret_cast<const F *>(brow + nt * 16) : zero_frag<F>();
                const F c0 = first ? cf[0][nt] : cf[1][nt];
                sT[s] = mma_one(b0, c0, sT[s]);
            }
        }
        if (J == I) {   // causal mask on the diagonal tile: keep j <= i
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (g4 + r > col) sT[s][r] = 0.f;
        }
    }

    const bool residual = (p.flags & 1u) != 0;
    T *ybase = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_bs + (int64_t)t0 * HP;

    for (int h = h0, it = 0; h < h1; ++h, ++it) {
        unsigned char *buf = smem + ((Cfg::DB && (it & 1)) ? Cfg::BUF_BYTES : 0);
        if (!Cfg::DB && it > 0) __syncthreads();   // previous head's readers are done
        stage(buf);
        if (h + 1 < h1) prefetch(h + 1);
        __syncthreads();

        const T *xt = reinterpret_cast<const T *>(buf);
        const T *stb = reinterpret_cast<const T *>(buf + Cfg::XT_BYTES);
        const S *cm = reinterpret_cast<const S *>(buf + Cfg::XT_BYTES + Cfg::ST_BYTES);
        const float Dh = p.D ? p.D[h] : 0.f;

        // Z = C b(c-1)^T, then scale row i by exp(cum_i)
        f32x4 acc[2][PT];
#pragma unroll
        for (int ri = 0; ri < 2; ++ri)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[ri][pt] = zero_frag<f32x4>();
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
            for (int nt = 0; nt < NT; nt += (sizeof(T) == 2 ? 2 : 1)) {
                const F s0 = *reinterpret_cast<const F *>(stb + ((nt * PT + pt) * 64 + lane) * 4);
                if constexpr (sizeof(T) == 2) {
                    const F s1 = *reinterpret_cast<const F *>(stb + (((nt + 1) * PT + pt) * 64 + lane) * 4);
#pragma unroll
                    for (int ri = 0; ri < 2; ++ri)
                        acc[ri][pt] = mma_pair(cf[ri][nt], s0, cf[ri][nt + 1], s1, acc[ri][pt]);
                } else {
#pragma unroll
                    for (int ri = 0; ri < 2; ++ri) acc[ri][pt] = mma_one(cf[ri][nt], s0, acc[ri][pt]);
                }
            }
        }
#pragma unroll
        for (int ri = 0; ri < 2; ++ri) {
            const int ib = (ri ? I1 : I0) * 16 + g4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __expf((float)cm[ib + r]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[ri][pt][r] *= e;
            }
        }

        // by_intra: pairs of slots, each pair feeding one of the two row blocks
        const S ci0 = cm[I0 * 16 + col], ci1 = cm[I1 * 16 + col];
#pragma unroll
        for (int q = 0; q < Cfg::NPAIR; ++q) {
            F a[2];
            int Jx[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int s = 2 * q + u;
                if (s == w + 1) {
                    a[u] = zero_frag<F>();
                    Jx[u] = 0;
                    continue;
                }
                const bool first = s <= w;
                const int I = first ? I0 : I1;
                const int J = first ? s : s - w - 2;
                const S ci = first ? ci0 : ci1;
                Jx[u] = J;
                f32x4 m;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = (J < I) || (g4 + r <= col);
                    m[r] = valid ? sT[s][r] * __expf((float)(ci - cm[J * 16 + g4 + r])) : 0.f;
                }
                a[u] = frag_from_f32<T>(m);
            }
            const bool owner1 = (2 * q) >= (w + 1);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const T *xrow = xt + (pt * 16 + col) * RS + g4;
                const F x0 = *reinterpret_cast<const F *>(xrow + Jx[0] * 16);
                const F x1 = *reinterpret_cast<const F *>(xrow + Jx[1] * 16);
                if (owner1) acc[1][pt] = mma_pair(a[0], x0, a[1], x1, acc[1][pt]);
                else acc[0][pt] = mma_pair(a[0], x0, a[1], x1, acc[0][pt]);
            }
        }

        // epilogue: + D x (+ x), round, store
        T *yh = ybase + h * P;
#pragma unroll
        for (int ri = 0; ri < 2; ++ri) {
            const int I = ri ? I1 : I0;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const F xv = *reinterpret_cast<const F *>(xt + (pt * 16 + col) * RS + I * 16 + g4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = I * 16 + g4 + r;
                    const float xf = to_f32(xv[r]);
                    float v = acc[ri][pt][r] + Dh * xf;
                    if (residual) v += xf;
                    if (i < Qc) yh[(int64_t)i * HP + pt * 16 + col] = from_f32<T>(v);
                }
            }
        }
        // (double buffering: the next head stages into the other buffer; its barrier
        //  orders this head's reads before that buffer is written again)
    }
}

template <typename T, int Q, int P, int N>
static hipError_t launch_scan_t(const Problem &p, hipStream_t s) {
    using Cfg = ScanCfg<T, Q, P, N>;
    if constexpr (!Cfg::OK) {
        return hipErrorInvalidValue;
    } else {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void *)chunk_scan_kernel<T, Q, P, N>, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
        if (attr != hipSuccess) return attr;
        const int hpg = p.H / p.G;
        const int nhg = p.G * ((hpg + p.heads_per_wg_scan - 1) / p.heads_per_wg_scan);
        const int64_t nblk = (int64_t)p.batch * p.nc * nhg;
        if (nblk <= 0 || nblk > 0x7fffffff) return hipErrorInvalidValue;
        chunk_scan_kernel<T, Q, P, N><<<(unsigned)nblk, Cfg::THREADS, Cfg::LDS, s>>>(p);
        return hipGetLastError();
    }
}

#define SSD_SCAN_SHAPES(X, T)                                                              \
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

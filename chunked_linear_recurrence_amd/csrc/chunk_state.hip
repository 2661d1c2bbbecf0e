// chunk_state: every chunk's local end state from a zero initial state, b_intra(c) of
// [分块推理 §2.1] (page "分块推理：解锁循环模型并行计算，实现长序列高效处理"):
//
//     b_intra(c)[p][n] = sum_j  2^(cum[last] - cum[j]) * x[j][p] * B[j][n]
//
// over the chunk's tokens j, where cum is the chunk's dA_cum row (base-2 sums of dt A).  Written as a matrix
// product it is  b_intra^T = B_c^T (N x Q) * (w . x_c) (Q x P)  with w_j the decay from
// token j to the chunk end, a K = Q contraction on the matrix cores (bf16 in, fp32
// accumulate; fp32 in for the fp32 dtype).
//
// Work: one workgroup per (batch, chunk, group of heads that read the same B).  The B
// chunk is transposed once into LDS (tokens contiguous per state index n) and every wave
// keeps its A-operand fragments (its share of the n rows, all Q tokens) in registers for
// all heads of the group.  Per head, x is scaled by w in fp32, rounded to the activation
// dtype, transposed into LDS (double-buffered), and read as B-operand fragments; the
// result tiles are rounded once to the activation dtype and stored in tile order, 4
// values per lane (coalesced 512 B or 1 KiB per wave).
// The next head's x rows and decays are loaded into registers as soon as the current
// head's x is in LDS, so their HBM latency overlaps the current head's products.
#include "ssd_common.h"

namespace ssd {

template <typename T, int Q, int P, int N>
struct StateCfg {
    static constexpr int NT = N / 16, PT = P / 16, KT = Q / 16;
    static constexpr int NWS = N >= 32 ? N / 32 : 1;          // waves
    static constexpr int NTW = NT / NWS;                       // n tiles per wave
    static constexpr int THREADS = NWS * 64;
    static constexpr int RS = Q + 4;                           // LDS row stride (elements)
    static constexpr int RJ = 16 / (int)sizeof(T);             // rows per transpose block
    static constexpr int CW = 16 / (int)sizeof(T);             // columns per block (16-byte rows)
    static constexpr int XB = (Q / RJ) * (P / CW);             // x transpose blocks
    static constexpr int XBT = (XB + THREADS - 1) / THREADS;
    static constexpr int BB = (Q / RJ) * (N / CW);
    static constexpr int BT_BYTES = N * RS * (int)sizeof(T);
    static constexpr int XW_BYTES = P * RS * (int)sizeof(T);
    static constexpr int LDS = BT_BYTES > 2 * XW_BYTES ? BT_BYTES : 2 * XW_BYTES;
    static constexpr bool OK = (KT % 2 == 0) && LDS <= kLdsBytes && NT % NWS == 0;
};

// 16 bytes of one row: 8 bf16 or 4 float.
template <typename T> struct Row16T;
template <> struct Row16T<bf16> { typedef bf16x8 type; };
template <> struct Row16T<float> { typedef f32x4 type; };

// Loads rows [j0, j0 + RJ) x cols [c0, c0 + 16 bytes) of a token-major tile (row pitch
// `pitch` elements), zero past `rows`.  Non-temporal: x and B are streamed once here.
template <typename T, int RJ>
__device__ __forceinline__ void load_block(const T *base, int64_t pitch, int j0, int c0, int rows,
                                           typename Row16T<T>::type (&r)[RJ]) {
    typedef typename Row16T<T>::type V;
#pragma unroll
    for (int i = 0; i < RJ; ++i) {
        if (j0 + i < rows) r[i] = __builtin_nontemporal_load(reinterpret_cast<const V *>(base + (int64_t)(j0 + i) * pitch + c0));
        else r[i] = V{};
    }
}

// Writes the transpose of an RJ x CW block into LDS rows c0..c0+CW-1 at column j0,
// optionally scaling row i by w[i] (in fp32, then rounded to T).
template <typename T, int RJ, int RS, bool SCALE>
__device__ __forceinline__ void store_block_t(T *lds, int j0, int c0, const typename Row16T<T>::type (&r)[RJ],
                                              const float *w) {
    constexpr int CW = 16 / (int)sizeof(T);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
        typename TF<T>::type col[RJ / 4];
#pragma unroll
        for (int i = 0; i < RJ; ++i) {
            T v = r[i][cc];
            if (SCALE) v = from_f32<T>(to_f32(v) * w[i]);
            col[i / 4][i % 4] = v;
        }
#pragma unroll
        for (int q = 0; q < RJ / 4; ++q)
            *reinterpret_cast<typename TF<T>::type *>(lds + (c0 + cc) * RS + j0 + 4 * q) = col[q];
    }
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((StateCfg<T, Q, P, N>::THREADS)) void chunk_state_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.y);
    using Cfg = StateCfg<T, Q, P, N>;
    using F = typename TF<T>::type;
    typedef typename CumT<T>::type S;
    constexpr int RJ = Cfg::RJ, RS = Cfg::RS, THREADS = Cfg::THREADS;
    extern __shared__ __align__(16) unsigned char smem[];
    T *bt = reinterpret_cast<T *>(smem);                    // [N][RS], then reused:
    T *xw0 = reinterpret_cast<T *>(smem);                   // [P][RS] x 2 buffers
    T *xw1 = reinterpret_cast<T *>(smem + Cfg::XW_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hpg = p.H / p.G;                                // heads per B group
    const int hg_per_group = (hpg + p.heads_per_wg_state - 1) / p.heads_per_wg_state;
    const int nhg = p.G * hg_per_group;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int hgi = logical % nhg;
    const int bc = logical / nhg;
    const int c = bc % p0.nc, b = bc / p0.nc;     // grid layout: chunks of the longest step
    if (c >= p.nc) return;                        // past a short last segment (uniform)
    const int grp = hgi / hg_per_group;
    const int h0 = grp * hpg + (hgi % hg_per_group) * p.heads_per_wg_state;
    const int h1 = min(h0 + p.heads_per_wg_state, (grp + 1) * hpg);
    const int t0 = c * Q;
    const int Qc = min(Q, p.L - t0);
    const int HP = p.H * P;

    const T *xb = reinterpret_cast<const T *>(p.x) + (int64_t)b * p.x_bs + (int64_t)t0 * HP;
    const S *cumb = reinterpret_cast<const S *>(p.dA_cum) + ((int64_t)b * p.H) * p.nc * Q + (int64_t)c * Q;

    // x rows and decays of one head, loaded into registers one head ahead of their use
    typedef typename Row16T<T>::type V;
    constexpr int CW = Cfg::CW;
    V xr[Cfg::XBT][RJ];
    S cw[Cfg::XBT][RJ];
    S clast = 0;
    auto prefetch = [&](int h, V (&xv)[Cfg::XBT][RJ], S (&cv)[Cfg::XBT][RJ], S &cl) {
        const T *xh = xb + h * P;
        const S *cu = cumb + (int64_t)h * p.nc * Q;
#pragma unroll
        for (int k = 0; k < Cfg::XBT; ++k) {
            const int blk = tid + k * THREADS;
            if (blk < Cfg::XB) {
                const int jb = blk / (P / CW), pb = blk % (P / CW);
                load_block<T, RJ>(xh, HP, jb * RJ, pb * CW, Qc, xv[k]);
                // the block's RJ consecutive decay sums, as 16-byte loads
                if constexpr (sizeof(S) == 4) {
#pragma unroll
                    for (int q = 0; q < RJ / 4; ++q) {
                        const float4 u = reinterpret_cast<const float4 *>(cu + jb * RJ)[q];
                        cv[k][4 * q + 0] = u.x;
                        cv[k][4 * q + 1] = u.y;
                        cv[k][4 * q + 2] = u.z;
                        cv[k][4 * q + 3] = u.w;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < RJ / 2; ++q) {
                        const double2 u = reinterpret_cast<const double2 *>(cu + jb * RJ)[q];
                        cv[k][2 * q + 0] = u.x;
                        cv[k][2 * q + 1] = u.y;
                    }
                }
            }
        }
        cl = cu[Q - 1];
    };
    prefetch(h0, xr, cw, clast);

    // B chunk -> LDS, transposed: bt[n][j]
    {
        const T *Bb = reinterpret_cast<const T *>(p.B) + (int64_t)b * p.bc_bs + (int64_t)t0 * p.G * N + grp * N;
        for (int blk = tid; blk < Cfg::BB; blk += THREADS) {
            const int jb = blk / (N / CW), nb = blk % (N / CW);
            V r[RJ];
            load_block<T, RJ>(Bb, (int64_t)p.G * N, jb * RJ, nb * CW, Qc, r);
            store_block_t<T, RJ, RS, false>(bt, jb * RJ, nb * CW, r, nullptr);
        }
    }
    __syncthreads();
    F af[Cfg::NTW][Cfg::KT];
#pragma unroll
    for (int i = 0; i < Cfg::NTW; ++i) {
        const int n = (wave * Cfg::NTW + i) * 16 + (lane & 15);
#pragma unroll
        for (int kt = 0; kt < Cfg::KT; ++kt)
            af[i][kt] = *reinterpret_cast<const F *>(bt + n * RS + kt * 16 + 4 * (lane >> 4));
    }
    __syncthreads();   // bt is overwritten by the x buffers below

    const int64_t PN = (int64_t)P * N;
    for (int h = h0, it = 0; h < h1; ++h, ++it) {
        T *xw = (it & 1) ? xw1 : xw0;
        // scale by the decay to the chunk end, transpose into LDS
#pragma unroll
        for (int k = 0; k < Cfg::XBT; ++k) {
            const int blk = tid + k * THREADS;
            if (blk < Cfg::XB) {
                const int jb = blk / (P / CW), pb = blk % (P / CW);
                float w[RJ];
#pragma unroll
                for (int i = 0; i < RJ; ++i) w[i] = exp2_fast((float)(clast - cw[k][i]));
                store_block_t<T, RJ, RS, true>(xw, jb * RJ, pb * CW, xr[k], w);
            }
        }
        if (h + 1 < h1) prefetch(h + 1, xr, cw, clast);   // overlaps this head's products
        __syncthreads();

        f32x4 acc[Cfg::NTW][Cfg::PT];
#pragma unroll
        for (int i = 0; i < Cfg::NTW; ++i)
#pragma unroll
            for (int pt = 0; pt < Cfg::PT; ++pt) acc[i][pt] = zero_frag<f32x4>();
#pragma unroll
        for (int kt = 0; kt < Cfg::KT; kt += 2) {
#pragma unroll
            for (int pt = 0; pt < Cfg::PT; ++pt) {
                const T *row = xw + (pt * 16 + (lane & 15)) * RS + 4 * (lane >> 4);
                const F x0 = *reinterpret_cast<const F *>(row + kt * 16);
                const F x1 = *reinterpret_cast<const F *>(row + (kt + 1) * 16);
#pragma unroll
                for (int i = 0; i < Cfg::NTW; ++i)
                    acc[i][pt] = mma_pair(af[i][kt], x0, af[i][kt + 1], x1, acc[i][pt]);
            }
        }
        T *out = reinterpret_cast<T *>(p.b_intra) + (((int64_t)b * p.nc + c) * p.H + h) * PN;
#pragma unroll
        for (int i = 0; i < Cfg::NTW; ++i) {
            const int nt = wave * Cfg::NTW + i;
#pragma unroll
            for (int pt = 0; pt < Cfg::PT; ++pt)
                __builtin_nontemporal_store(frag_from_f32<T>(acc[i][pt]),   // written once, read by state_pass
                                            reinterpret_cast<F *>(out + ((nt * Cfg::PT + pt) * 64 + lane) * 4));
        }
    }
}

template <typename T, int Q, int P, int N>
static hipError_t launch_state_t(const Problem &p, hipStream_t s) {
    using Cfg = StateCfg<T, Q, P, N>;
    if constexpr (!Cfg::OK) {
        return hipErrorInvalidValue;
    } else {
        const int hpg = p.H / p.G;
        const int nhg = p.G * ((hpg + p.heads_per_wg_state - 1) / p.heads_per_wg_state);
        const int64_t nblk = (int64_t)p.batch * p.nc * nhg;
        if (nblk <= 0 || nblk > 0x7fffffff) return hipErrorInvalidValue;
        if (const hipError_t attr = allow_lds<chunk_state_kernel<T, Q, P, N>>(Cfg::LDS); attr != hipSuccess)
            return attr;
        chunk_state_kernel<T, Q, P, N><<<dim3((unsigned)nblk, step_count(p)), Cfg::THREADS, Cfg::LDS, s>>>(p);
        return hipGetLastError();
    }
}

#define SSD_STATE_SHAPES(X, T)                                                             \
    X(T, 32, 32, 64) X(T, 32, 64, 64) X(T, 32, 64, 128)                                    \
    X(T, 64, 16, 16) X(T, 64, 16, 32) X(T, 64, 16, 64) X(T, 64, 16, 128)                   \
    X(T, 64, 32, 32) X(T, 64, 32, 64) X(T, 64, 32, 128) X(T, 64, 64, 64) X(T, 64, 64, 128) \
    X(T, 128, 32, 64) X(T, 128, 64, 64) X(T, 128, 64, 128)                                 \
    X(T, 256, 16, 32) X(T, 256, 32, 64) X(T, 256, 64, 64) X(T, 256, 64, 128)               \
    X(T, 256, 128, 128) X(T, 256, 64, 256)

#define SSD_STATE_CASE(T, q, pp, nn) \
    if (p.Q == q && p.P == pp && p.N == nn) return launch_state_t<T, q, pp, nn>(p, s);
#define SSD_STATE_OK(T, q, pp, nn) \
    if (Q == q && P == pp && N == nn) return StateCfg<T, q, pp, nn>::OK;

hipError_t launch_chunk_state(const Problem &p, hipStream_t s) {
    if (p.dtype == 1) { SSD_STATE_SHAPES(SSD_STATE_CASE, bf16) }
    else { SSD_STATE_SHAPES(SSD_STATE_CASE, float) }
    return hipErrorInvalidValue;
}

bool chunk_state_supported(int dtype, int Q, int P, int N) {
    if (dtype == 1) {
        if (N < 32) return false;
        SSD_STATE_SHAPES(SSD_STATE_OK, bf16)
    } else {
        SSD_STATE_SHAPES(SSD_STATE_OK, float)
    }
    return false;
}

}  // namespace ssd

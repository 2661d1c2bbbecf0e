// chunk_scan_assoc: the chunk outputs of [分块推理 §2.1-§2.2] (page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理") computed in the scan form the page
// describes for the intra-chunk part: within a chunk the recurrence h_t = a_t h_{t-1} +
// x_t (outer) B_t is a prefix computation over the associative pairs (a_t, x_t B_t), with
// (a1, v1) then (a2, v2) combining to (a1 a2, a2 v1 + v2), so it can be evaluated as a
// log-depth tree.  This kernel is the alternative to chunk_scan's matrix-core form (same
// inputs, same outputs); it exists to measure that choice.
//
// One workgroup per (batch, chunk, head), one wave per window of 64 tokens, lane = token.
// For each state element (p, n):
//   - every lane forms v_t = x_t[p] B_t[n] and the wave runs an inclusive tree scan over
//     its 64 tokens in log2(64) = 6 cross-lane steps: spans 1, 2, 4, 8 inside each
//     16-lane row (DPP row shifts), then the end of row r joined to row r + 1 and lane 31
//     to rows 2-3 (DPP row broadcasts); every step multiplies the incoming partial value
//     by the decay across the span it skips, 2^(cum_t - cum_s) (per lane, computed once
//     from the chunk's dA_cum row);
//   - lane 63 leaves its window's end value in LDS; the state entering window w is then
//     2^(cum_{64w-1}) b_in + sum_{w' < w} 2^(cum_{64w-1} - cum_{64w'+63}) end_{w'}
//     (the top levels of the tree, across the chunk's Q/64 windows), and reaches token t
//     with the factor 2^(cum_t - cum_{64w-1}) (cum: base-2 sums of dt A);
//   - y_t[p] accumulates C_t[n] h_t[n] over n in a register.
// y_t = sum_n C_t[n] h_t[n] + (D + residual) x_t, rounded once to the activation dtype.
// B and C of the chunk are staged once in LDS with one padding word per row, so the 64
// lanes (64 different rows) read different banks; b(c-1) is staged row-major.
#include "ssd_common.h"

namespace ssd {

template <typename T, int Q, int P, int N>
struct AssocCfg {
    static constexpr int NWIN = Q >= 64 ? Q / 64 : 1;           // waves (64-token windows)
    static constexpr int THREADS = NWIN * 64;
    static constexpr int EPW = 4 / (int)sizeof(T);             // elements per 4-byte word
    static constexpr int WPR = N / EPW;                         // words per row
    static constexpr int RSW = WPR + 1;                         // LDS row stride in words
    static constexpr int TILE_BYTES = Q * RSW * 4;              // one of B, C
    static constexpr int END_BYTES = 2 * NWIN * N * 4;          // window end values, double-buffered
    static constexpr int BIN_BYTES = P * N * (int)sizeof(T);    // b(c-1), row-major
    static constexpr int LDS = 2 * TILE_BYTES + END_BYTES + BIN_BYTES;
    static constexpr bool OK = LDS <= kLdsBytes;
};

// One step of the in-wave tree: the value of the lane selected by the DPP control (0
// where there is none), times this lane's decay across the skipped span, added.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float tree_step(float v, float m) {
    const int u = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xf, true);
    return fmaf(m, __builtin_bit_cast(float, u), v);
}

// Element e (0 .. EPW-1) of an LDS word.
template <typename T>
__device__ __forceinline__ float word_elem(uint32_t wd, int e);
template <>
__device__ __forceinline__ float word_elem<float>(uint32_t wd, int) { return __uint_as_float(wd); }
template <>
__device__ __forceinline__ float word_elem<bf16>(uint32_t wd, int e) {
    return __uint_as_float(e ? (wd & 0xffff0000u) : (wd << 16));
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((AssocCfg<T, Q, P, N>::THREADS)) void chunk_scan_assoc_kernel(Problem p0) {
    using Cfg = AssocCfg<T, Q, P, N>;
    typedef typename CumT<T>::type S;
    constexpr int NWIN = Cfg::NWIN, EPW = Cfg::EPW, WPR = Cfg::WPR, RSW = Cfg::RSW;
    constexpr int PT = P / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *Bs = reinterpret_cast<uint32_t *>(smem);
    uint32_t *Cs = Bs + Q * RSW;
    float *endv = reinterpret_cast<float *>(Cs + Q * RSW);    // [2][NWIN][N]
    uint32_t *bins = reinterpret_cast<uint32_t *>(endv + 2 * NWIN * N);   // b(c-1) [P][N] as words

    const Problem p = step_problem(p0, blockIdx.y);
    const int logical = blockIdx.x;                            // (b, c, h)
    const int h = logical % p0.H;
    const int bc = logical / p0.H;
    const int c = bc % p0.nc, b = bc / p0.nc;
    if (c >= p.nc) return;                                     // past a short last segment (uniform)
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);    // window of this wave
    const int t = w * 64 + lane;                               // token within the chunk
    const int t0 = c * Q;
    const int Qc = min(Q, p.L - t0);
    const bool act = t < Qc;
    const int g = h / (p.H / p.G);
    const int64_t HP = (int64_t)p.H * P;

    // B and C rows of the chunk -> LDS (zero past the chunk's last token)
    {
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(p.B) +
                                  (((int64_t)b * p.bc_bs + (int64_t)t0 * p.G * N + (int64_t)g * N) * sizeof(T));
        const unsigned char *Cb = reinterpret_cast<const unsigned char *>(p.C) +
                                  (((int64_t)b * p.bc_bs + (int64_t)t0 * p.G * N + (int64_t)g * N) * sizeof(T));
        const int64_t rowb = (int64_t)p.G * N * sizeof(T);
        for (int idx = tid; idx < Q * WPR; idx += Cfg::THREADS) {
            const int j = idx / WPR, k = idx % WPR;
            uint32_t bw = 0, cw = 0;
            if (j < Qc) {
                bw = *reinterpret_cast<const uint32_t *>(Bb + j * rowb + k * 4);
                cw = *reinterpret_cast<const uint32_t *>(Cb + j * rowb + k * 4);
            }
            Bs[j * RSW + k] = bw;
            Cs[j * RSW + k] = cw;
        }
    }

    // per-lane decay factors from the chunk's log-decay prefix sums
    const S *cum = reinterpret_cast<const S *>(p.dA_cum) + (((int64_t)b * p.H + h) * p.nc + c) * Q;
    const int tc = t < Q ? t : Q - 1;
    const S ct = cum[tc];
    const S cws = w > 0 ? cum[w * 64 - 1] : (S)0;             // sum before this window
    const float Pw = exp2_fast((float)(ct - cws));                // window start .. t
    // decays of the six tree steps: row shifts by d = 1, 2, 4, 8 (from lane t - d of the
    // same 16-lane row), then row ends (rows 1 and 3 take the end of the row before) and
    // lane 31 (rows 2 and 3); zero where the step adds nothing or the lane is past Q
    const int lr = lane & 15, row = lane >> 4, w0 = w * 64;
    float M[6];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int d = 1 << s;
        M[s] = (lr >= d && t < Q) ? exp2_fast((float)(ct - cum[t - d >= 0 ? t - d : 0])) : 0.f;
    }
    M[4] = ((row & 1) && t < Q) ? exp2_fast((float)(ct - cum[min(w0 + 16 * row - 1, Q - 1)])) : 0.f;
    M[5] = (row >= 2 && t < Q) ? exp2_fast((float)(ct - cum[w0 + 31])) : 0.f;
    const float Dwin = exp2_fast((float)cws);                     // chunk start .. window start
    float Dww[NWIN];                                           // end of window w' .. window start
#pragma unroll
    for (int v = 0; v < NWIN; ++v) Dww[v] = v < w ? exp2_fast((float)(cws - cum[min(v * 64 + 63, Q - 1)])) : 0.f;
    const float dres = (p.D ? p.D[h] : 0.f) + ((p.flags & 1u) ? 1.f : 0.f);
    const T *xr = reinterpret_cast<const T *>(p.x) + (int64_t)b * p.x_bs + (int64_t)(t0 + (act ? t : 0)) * HP + h * P;
    T *yr = reinterpret_cast<T *>(p.y) + (int64_t)b * p.y_bs + (int64_t)(t0 + (act ? t : 0)) * HP + h * P;
    // b(c-1) (tile order in the workspace) -> LDS, row-major [P][N]: 4 consecutive n per piece
    {
        const T *bin = reinterpret_cast<const T *>(p.b_in) + (((int64_t)b * p.nc + c) * p.H + h) * (int64_t)P * N;
        T *bl = reinterpret_cast<T *>(bins);
        for (int e4 = tid; e4 < P * N / 4; e4 += Cfg::THREADS) {
            const int e = e4 * 4, tile = e >> 8, l = (e >> 2) & 63;
            const int pr = (tile % PT) * 16 + (l & 15), n0 = (tile / PT) * 16 + 4 * (l >> 4);
            typedef typename TF<T>::type F;
            *reinterpret_cast<F *>(bl + pr * N + n0) = *reinterpret_cast<const F *>(bin + e);
        }
    }
    __syncthreads();

    for (int pp = 0, par = 0; pp < P; ++pp, par ^= 1) {
        const float xv = act ? to_f32(xr[pp]) : 0.f;
        float yl = 0.f;
        float *ev = endv + (par * NWIN + w) * N;
        // elements in groups of 64: lane 63's end value of element n is selected into lane
        // n % 64 of endacc (no per-element branch), then one LDS write per group
        constexpr int NH = (N + 63) / 64, WPH = 64 / EPW;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            int endacc = 0;
            // several words per iteration: their scans are independent chains, which hides
            // the latency of the cross-lane steps (one wave per SIMD at this LDS size)
#pragma unroll 8
            for (int k = hh * WPH; k < (WPR < (hh + 1) * WPH ? WPR : (hh + 1) * WPH); ++k) {
                const uint32_t bw = Bs[t < Q ? t * RSW + k : k];
                const uint32_t cw = Cs[t < Q ? t * RSW + k : k];
#pragma unroll
                for (int e = 0; e < EPW; ++e) {
                    float v = t < Q ? xv * word_elem<T>(bw, e) : 0.f;
                    // inclusive tree scan over the window (DPP: row_shr 1, 2, 4, 8; row_bcast
                    // 15 into rows 1 and 3; row_bcast 31 into rows 2 and 3)
                    v = tree_step<0x111, 0xf>(v, M[0]);
                    v = tree_step<0x112, 0xf>(v, M[1]);
                    v = tree_step<0x114, 0xf>(v, M[2]);
                    v = tree_step<0x118, 0xf>(v, M[3]);
                    v = tree_step<0x142, 0xa>(v, M[4]);
                    v = tree_step<0x143, 0xc>(v, M[5]);
                    yl = fmaf(word_elem<T>(cw, e), v, yl);
                    const int last = __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63);
                    endacc = lane == k * EPW + e - hh * 64 ? last : endacc;
                }
            }
            if (hh * 64 + lane < N) ev[hh * 64 + lane] = __builtin_bit_cast(float, endacc);
        }
        __syncthreads();                                        // every window's end values
        // state entering this window, contracted with C_t
        float yc = 0.f;
        const float *e0 = endv + par * NWIN * N;
#pragma unroll 8
        for (int k = 0; k < WPR; ++k) {
            const uint32_t bw = bins[pp * WPR + k];            // same word for every lane
            const uint32_t cw = Cs[(t < Q ? t : 0) * RSW + k];
#pragma unroll
            for (int e = 0; e < EPW; ++e) {
                const int n = k * EPW + e;
                float K = Dwin * word_elem<T>(bw, e);
#pragma unroll
                for (int v = 0; v < NWIN; ++v)
                    if (v < w) K = fmaf(Dww[v], e0[v * N + n], K);
                yc = fmaf(word_elem<T>(cw, e), K, yc);
            }
        }
        if (act) yr[pp] = from_f32<T>(fmaf(Pw, yc, yl) + dres * xv);
    }
}

template <typename T, int Q, int P, int N>
static hipError_t launch_assoc_t(const Problem &p, hipStream_t s) {
    using Cfg = AssocCfg<T, Q, P, N>;
    if constexpr (!Cfg::OK) {
        return hipErrorInvalidValue;
    } else {
        if (const hipError_t attr = allow_lds<chunk_scan_assoc_kernel<T, Q, P, N>>(Cfg::LDS); attr != hipSuccess)
            return attr;
        const int64_t nblk = (int64_t)p.batch * p.nc * p.H;
        if (nblk <= 0 || nblk > 0x7fffffff) return hipErrorInvalidValue;
        chunk_scan_assoc_kernel<T, Q, P, N><<<dim3((unsigned)nblk, step_count(p)), Cfg::THREADS, Cfg::LDS, s>>>(p);
        return hipGetLastError();
    }
}

#define SSD_ASSOC_SHAPES(X, T) \
    X(T, 32, 64, 64) X(T, 64, 32, 64) X(T, 64, 64, 64) X(T, 64, 64, 128) X(T, 128, 64, 128) X(T, 256, 64, 128)
#define SSD_ASSOC_CASE(T, q, pp, nn) \
    if (p.Q == q && p.P == pp && p.N == nn) return launch_assoc_t<T, q, pp, nn>(p, s);
#define SSD_ASSOC_OK(T, q, pp, nn) \
    if (Q == q && P == pp && N == nn) return AssocCfg<T, q, pp, nn>::OK;

hipError_t launch_chunk_scan_assoc(const Problem &p, hipStream_t s) {
    if (p.dtype == 1) { SSD_ASSOC_SHAPES(SSD_ASSOC_CASE, bf16) }
    else { SSD_ASSOC_SHAPES(SSD_ASSOC_CASE, float) }
    return hipErrorInvalidValue;
}

bool chunk_scan_assoc_supported(int dtype, int Q, int P, int N) {
    if (dtype == 1) { SSD_ASSOC_SHAPES(SSD_ASSOC_OK, bf16) }
    else { SSD_ASSOC_SHAPES(SSD_ASSOC_OK, float) }
    return false;
}

}  // namespace ssd

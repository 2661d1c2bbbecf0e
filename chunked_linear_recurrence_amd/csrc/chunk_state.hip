// chunk_state: every chunk's local end state from a zero initial state, b_intra(c) of
// [分块推理 §2.1] (page "分块推理：解锁循环模型并行计算，实现长序列高效处理"):
//
//     b_intra(c)[p][n] = sum_j  w_j * x[j][p] * B[j][n],   w_j = 2^(cum[last] - cum[j])
//
// over the chunk's tokens j, where cum is the chunk's dA_cum row (base-2 sums of dt A) and
// w_j, the decay from token j to the chunk's end, comes precomputed from chunk_cumsum
// (wend, 0 past a short chunk).  As a matrix product it is
//     b_intra^T = (B_c . w)^T (N x Q) * x_c (Q x P),
// a K = Q contraction on the matrix cores (bf16 in, fp32 accumulate; fp32 in for the fp32
// dtype).
//
// Work: one workgroup per (batch, chunk, group of heads that read the same B), N/32 waves,
// each owning NTW n tiles and all P/16 p tiles of the output; shapes whose LDS allows only
// one workgroup per CU take twice the waves, each with half of the p tiles (StateCfg).
//   - Once per workgroup the chunk's B tile arrives in LDS by DMA (row-major, swizzled
//     16-byte pieces), and each wave reads its B^T fragments (k = token) with the gfx950
//     transpose read and keeps them in registers for every head of the group.
//   - Per head, the x tile and the wend row arrive in LDS by DMA, double-buffered: the
//     next head's copies are issued at the start of the current head's products.  x fragments
//     (k = token) come straight from the transpose read; the weights are applied to the
//     wave's B^T fragments in fp32 and rounded once to the operand dtype, so no tile is
//     rewritten in LDS.
//   - The result tiles are rounded once to the activation dtype and stored in tile order,
//     4 values per lane (coalesced 512 B or 1 KiB per wave), during the next head.
#include "ssd_tile.h"

namespace ssd {

template <typename T>
__device__ __forceinline__ typename TF<T>::type scale_frag(const typename TF<T>::type &a, const f32x4 &w) {
    typename TF<T>::type r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = from_f32<T>(to_f32(a[e]) * w[e]);
    return r;
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__((StateCfg<T, Q, P, N>::THREADS), (StateCfg<T, Q, P, N>::MINB)) void chunk_state_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.y);
    using Cfg = StateCfg<T, Q, P, N>;
    using F = typename TF<T>::type;
    constexpr int NW = Cfg::NWS, NTW = Cfg::NTW, PT = Cfg::PT, PTW = Cfg::PTW, KT = Cfg::KT;
    constexpr int XK = Cfg::XK, NDMA = Cfg::NDMA, XPIECES = Cfg::XPIECES;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const StateTiles tiles = state_wave_tiles(w, Cfg::NWN, NTW, PTW, Cfg::PS);
    const int g4 = 4 * (lane >> 4);
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

    // Per-lane byte offsets of this lane's x pieces inside one head's slice of the chunk
    // (the same for every head), 32 bits (the host bounds a chunk's span of x below 2^31).
    const unsigned char *xchunk = reinterpret_cast<const unsigned char *>(p.x) +
                                  ((int64_t)b * p.x_bs + (int64_t)t0 * HP) * (int64_t)sizeof(T);
    const uint32_t xrow = (uint32_t)(HP * (int)sizeof(T)), xhead = (uint32_t)(P * (int)sizeof(T));
    uint32_t xoff[XK];
#pragma unroll
    for (int k = 0; k < XK; ++k) {
        const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, XPIECES, sizeof(T) == 2);
        const int rr = min(d.row, Qc - 1);                      // rows past a short chunk repeat the last
        xoff[k] = (uint32_t)rr * xrow + (uint32_t)(d.piece * 16);
    }
    // DMA item k of head h into buffer buf: x pieces, then the wend row (waves from NW - 1
    // down).  Each source is one buffer covering exactly this (head, chunk)'s data.
    auto dma_item = [&](int k, int h, unsigned char *buf) {
        if (k < XK) {
            const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, XPIECES, sizeof(T) == 2);
            if (d.on)                                           // uniform (whole waves of pieces)
                dma16_buf(make_rsrc(xchunk + (int64_t)h * xhead, (uint32_t)(Qc - 1) * xrow + xhead), xoff[k],
                          buf + d.lds - lane * 16);
        } else {
            const DmaPiece d = scan_row_piece(NW - 1 - w, lane, Cfg::WP);
            if (d.on) {
                const int64_t tok = (((int64_t)b * p.H + h) * p.nc + c) * Q;
                dma16_buf(make_rsrc(p.wend + tok, Cfg::WB), (uint32_t)(d.piece * 16),
                          buf + Cfg::O_W + d.lds - lane * 16);
            }
        }
    };

    // ---- per workgroup: the chunk's B tile into LDS, this wave's B^T fragments into
    // registers.  Rows past a short chunk repeat the last row; their weights are 0.
    F af[NTW][KT];
    {
        const int64_t bcp = (int64_t)p.G * N;
        const unsigned char *Bb = reinterpret_cast<const unsigned char *>(p.B) +
                                  ((int64_t)b * p.bc_bs + (int64_t)t0 * bcp + grp * N) * (int64_t)sizeof(T);
#pragma unroll
        for (int k = 0; k < Cfg::BK; ++k) {
            const DmaPiece d = scan_x_piece(k, w, lane, NW, Q, Cfg::BPIECES, sizeof(T) == 2);
            if (d.on)                                           // uniform
                dma16(Bb + (int64_t)min(d.row, Qc - 1) * bcp * (int64_t)sizeof(T) + d.piece * 16,
                      smem + d.lds - lane * 16);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) af[i][kt] = tile_frag<T, N>(smem, kt, tiles.nt0 + i, lane);
        // every wave's fragment reads have completed before the head buffers are refilled
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    }
#pragma unroll
    for (int k = 0; k < NDMA; ++k) dma_item(k, h0, smem);

    // The result tiles of head h are stored in the middle of head h + 1's products, so the
    // wait at the top of each head (for its copies) never waits on stores just issued.
    const int64_t PN = (int64_t)P * N;
    F res[NTW][PTW];
    auto store_results = [&](int hs) {
        T *out = reinterpret_cast<T *>(p.b_intra) + (((int64_t)b * p.nc + c) * p.H + hs) * PN;
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int nt = tiles.nt0 + i;
#pragma unroll
            for (int pt = 0; pt < PTW; ++pt)    // written once, read by state_pass
                __builtin_nontemporal_store(res[i][pt],
                                            reinterpret_cast<F *>(out + ((nt * PT + tiles.pt0 + pt) * 64 + lane) * 4));
        }
    };
    for (int h = h0, it = 0; h < h1; ++h, ++it) {
        const unsigned char *buf = smem + (it & 1) * Cfg::HEAD_BYTES;
        unsigned char *nbuf = smem + ((it + 1) & 1) * Cfg::HEAD_BYTES;
        __builtin_amdgcn_s_waitcnt(0);        // this head's copies (and older stores) complete
        __builtin_amdgcn_s_barrier();         // ... for every wave; the other buffer is free
        const bool more = h + 1 < h1;
        const float *wl = reinterpret_cast<const float *>(buf + Cfg::O_W);

        // the next head's copies go out first, so their latency overlaps all of this head's
        // products (spreading them through the products left the last ones exposed)
        if (more) {
#pragma unroll
            for (int k = 0; k < NDMA; ++k) dma_item(k, h + 1, nbuf);
        }
        f32x4 acc[NTW][PTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int pt = 0; pt < PTW; ++pt) acc[i][pt] = zero_frag<f32x4>();
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp) {
            if (kp == KT / 4 && h > h0) store_results(h - 1);   // the previous head's results
            const int kt0 = 2 * kp, kt1 = 2 * kp + 1;
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(wl + 16 * kt0 + g4);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(wl + 16 * kt1 + g4);
            F a0[NTW], a1[NTW];
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                a0[i] = scale_frag<T>(af[i][kt0], w0);
                a1[i] = scale_frag<T>(af[i][kt1], w1);
            }
#pragma unroll
            for (int pt = 0; pt < PTW; ++pt) {
                const F x0 = tile_frag<T, P>(buf, kt0, tiles.pt0 + pt, lane);
                const F x1 = tile_frag<T, P>(buf, kt1, tiles.pt0 + pt, lane);
#pragma unroll
                for (int i = 0; i < NTW; ++i) acc[i][pt] = mma_pair(a0[i], x0, a1[i], x1, acc[i][pt]);
            }
        }

#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int pt = 0; pt < PTW; ++pt) res[i][pt] = frag_from_f32<T>(acc[i][pt]);
    }
    store_results(h1 - 1);
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

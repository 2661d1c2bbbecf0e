// chunk_cumsum: per chunk and head, the inclusive prefix sum of dt * A over the chunk's
// tokens.  exp of entry i is the decay weight L_i of diag(L) in [分块推理 §2.2] (page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理"), exp of the last entry is the chunk's
// total decay (the product of A_t over the chunk), and exp of differences gives every
// intra-chunk decay.
//
// Layout: dA_cum[b, h, c, i], i < Q.  Positions past a short last chunk hold the chunk
// total, so later kernels can read any index without special cases.  The totals are also
// written contiguously, ctot[b, h, c], for the state pass.
// Sums are float64 for float32 activations (dt * A is then exact) and float32 for
// bfloat16 activations.
//
// Work: one workgroup per (batch, chunk, block of kCumHeads heads), one wave per head.  The
// Q x kCumHeads tile of dt * A is staged in LDS with coalesced loads; each wave then scans
// its head: every lane sums Q/64 consecutive values, and a 6-step wave shuffle scan
// combines the lane totals.  HBM-bound (reads dt once, writes 4 bytes per token-head).
#include "ssd_common.h"

namespace ssd {

// Heads per workgroup (the Q x heads tile of dt * A staged in LDS) and threads: one wave
// per head, so each wave runs a single scan (measured fastest: 8 heads x 8 waves, against 16
// heads x 4 waves with four scans per wave, or whole 64-head token rows).
constexpr int kCumHeads = 8, kCumThreads = kCumHeads * 64;

// A lane's E consecutive values as one vector store (E * sizeof(V) bytes).
template <typename V, int E>
__device__ __forceinline__ void store_run(V *dst, const V (&v)[E]) {
    if constexpr (E * sizeof(V) % 16 == 0) {
#pragma unroll
        for (int k = 0; k < E * (int)sizeof(V) / 16; ++k) {
            uint4 u;
            __builtin_memcpy(&u, reinterpret_cast<const unsigned char *>(v) + 16 * k, 16);
            reinterpret_cast<uint4 *>(dst)[k] = u;
        }
    } else if constexpr (E * sizeof(V) == 8) {
        uint2 u;
        __builtin_memcpy(&u, v, 8);
        *reinterpret_cast<uint2 *>(dst) = u;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) dst[e] = v[e];
    }
}

template <typename T, int Q>
__global__ __launch_bounds__(kCumThreads) void chunk_cumsum_kernel(Problem p0) {
    typedef typename CumT<T>::type S;
    constexpr int E = Q >= 64 ? Q / 64 : 1;      // values per lane
    constexpr int NA = Q / E;                    // lanes holding tokens (64, or Q when Q < 64)
    static_assert(16 % E == 0 && NA <= 64, "a lane's tokens lie in one 16-token block");
    __shared__ S tile[kCumHeads][Q + 1];
    const int c = blockIdx.x, hb = blockIdx.y * kCumHeads, b = blockIdx.z % p0.batch;
    const Problem p = step_problem(p0, blockIdx.z / p0.batch);
    if (c >= p.nc) return;                       // past a short last segment (uniform)
    const int t0 = c * Q;
    const int Qc = min(Q, p.L - t0);
    const T *dt = reinterpret_cast<const T *>(p.dt) + (int64_t)b * p.dt_bs;
    const int nh = min(kCumHeads, p.H - hb);

    for (int idx = threadIdx.x; idx < Q * kCumHeads; idx += kCumThreads) {
        const int j = idx / kCumHeads, hh = idx % kCumHeads;
        S v = 0;
        if (hh < nh && j < Qc) v = (S)to_f32(dt[(int64_t)(t0 + j) * p.H + hb + hh]) * (S)p.A[hb + hh];
        tile[hh][j] = v;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool active = lane < NA;
    for (int hh = wave; hh < nh; hh += kCumThreads / 64) {
        S v[E];
        S run = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (active) run += tile[hh][lane * E + e];
            v[e] = run;
        }
        // inclusive scan of the lane totals across the wave
        S incl = run;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const S up = __shfl_up(incl, d, 64);
            if (lane >= d) incl += up;
        }
        // exclusive prefix taken from the neighbour's inclusive value (not incl - run), so
        // a run of zero inputs past a short chunk repeats the chunk total exactly
        S excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0;
        S *out = reinterpret_cast<S *>(p.dA_cum) + (((int64_t)b * p.H + hb + hh) * p.nc + c) * Q + lane * E;
        // value at the chunk's last token, broadcast to the padded positions
        const int last = Qc - 1;
        S lastv = excl + v[0];
#pragma unroll
        for (int e = 1; e < E; ++e)
            if (e == last % E) lastv = excl + v[e];
        lastv = __shfl(lastv, last / E, 64);
        S cv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) cv[e] = (lane * E + e <= last) ? excl + v[e] : lastv;
        if (active) store_run<S, E>(out, cv);
        if (lane == 0)                               // the chunk's total, for the state pass
            reinterpret_cast<S *>(p.ctot)[((int64_t)b * p.H + hb + hh) * p.nc + c] = lastv;
    }
}

hipError_t launch_chunk_cumsum(const Problem &p, hipStream_t s) {
    dim3 grid(p.nc, (p.H + kCumHeads - 1) / kCumHeads, p.batch * step_count(p));
    if (p.dtype == 1) {
        if (p.Q == 32) chunk_cumsum_kernel<bf16, 32><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 64) chunk_cumsum_kernel<bf16, 64><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 128) chunk_cumsum_kernel<bf16, 128><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 256) chunk_cumsum_kernel<bf16, 256><<<grid, kCumThreads, 0, s>>>(p);
        else return hipErrorInvalidValue;
    } else {
        if (p.Q == 32) chunk_cumsum_kernel<float, 32><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 64) chunk_cumsum_kernel<float, 64><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 128) chunk_cumsum_kernel<float, 128><<<grid, kCumThreads, 0, s>>>(p);
        else if (p.Q == 256) chunk_cumsum_kernel<float, 256><<<grid, kCumThreads, 0, s>>>(p);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd

// state_pass: the sequential pass of global states across chunks, [分块推理 §2.2] of the
// page "分块推理：解锁循环模型并行计算，实现长序列高效处理":
//
//     b(-1) = init_state (or 0),   b(c) = b_intra(c) + 2^(chunk c's total of dA_cum) * b(c-1)
//
// It writes b_in[c] = b(c-1), the state entering chunk c, and final_state = b(nc-1) in
// float32.  b_intra and b_in are stored in the activation dtype (what chunk_scan's matrix
// cores consume); the carried state b stays in float32 registers for the whole pass, so
// only the per-chunk terms are rounded, never the running sum.
//
// The recurrence is elementwise over the P x N state, so the state of one (batch, head)
// is split across workgroups of one wave, each owning 256 elements (4 per lane), giving
// batch * H * P * N / 256 independent waves.  The loads of b_intra do not depend on the
// carried state, so they run two groups of K chunks ahead of the dependent multiply-adds
// (K loads of the next group are in flight while the current group is consumed); the pass
// is a pure HBM stream (read and write act bytes per state element per chunk); b_intra is
// read with the non-temporal policy (used once), b_in is stored normally (chunk_scan reads
// it next, and keeping its stores cacheable measured faster than streaming them).  Short
// chains (at most 16 chunks: a segment of the layer stack, a 4K-token sequence) are loaded
// whole at once by a second kernel whose waves own 2 or 4 element groups each, so every
// wave has enough loads in flight to cover its own start-up.
//
// b_intra and b_in use the tile order of the other kernels (see libssdscan.h); only
// init_state / final_state use the row-major [P][N] order, so the thread owning tile
// element (tile, lane l, r = 0..3) maps to p = 16 * pt + l % 16, n = 16 * nt + 4 (l / 16) + r.
#include "ssd_index.h"

namespace ssd {

template <typename T>
__device__ __forceinline__ void store_state(T *dst, const float4 &v);
template <>
__device__ __forceinline__ void store_state<float>(float *dst, const float4 &v) {
    *reinterpret_cast<float4 *>(dst) = v;
}
template <>
__device__ __forceinline__ void store_state<bf16>(bf16 *dst, const float4 &v) {
    bf16x4 o;
    o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
    *reinterpret_cast<bf16x4 *>(dst) = o;
}

__device__ __forceinline__ float4 as_float4(const f32x4 &v) { return make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ float4 as_float4(const bf16x4 &v) {
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

__device__ __forceinline__ float4 fma4(float a, const float4 &s, const float4 &b) {
    return make_float4(fmaf(a, s.x, b.x), fmaf(a, s.y, b.y), fmaf(a, s.z, b.z), fmaf(a, s.w, b.w));
}

// One wave per 256-element group of a (batch, head) state; loads run two groups of K
// chunks ahead of the dependent multiply-adds.
template <typename T, int K>
__global__ __launch_bounds__(64) void state_pass_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.z / p0.batch);
    typedef typename TF<T>::type V;
    typedef typename CumT<T>::type S;
    const int PN = p.P * p.N;
    const int e4 = blockIdx.x * 64 + threadIdx.x;        // 4-element group within one state
    const int h = blockIdx.y, b = blockIdx.z % p0.batch;
    if (e4 * 4 >= PN) return;
    const int e = e4 * 4;
    const StateIdx pn = tile_elem(e, p.P);                     // (p, n0) of tile-order element e
    const int64_t std_off = (((int64_t)b * p.H + h) * p.P + pn.p) * p.N + pn.n0;

    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.init) s = *reinterpret_cast<const float4 *>(p.init + std_off);

    const int64_t cstride = (int64_t)p.H * PN;            // between chunks
    const T *bi = reinterpret_cast<const T *>(p.b_intra) + ((int64_t)b * p.nc * p.H + h) * PN + e;
    T *bo = reinterpret_cast<T *>(p.b_in) + ((int64_t)b * p.nc * p.H + h) * PN + e;
    const S *tot = reinterpret_cast<const S *>(p.ctot) + ((int64_t)b * p.H + h) * p.nc;   // chunk totals
    const int nc = p.nc;

    V va[K], vb[K];
    S da[K], db[K];
    auto load = [&](int c0, V (&v)[K], S (&d)[K]) {
#pragma unroll
        for (int u = 0; u < K; ++u)
            if (c0 + u < nc) {                               // uniform
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const V *>(bi + (int64_t)(c0 + u) * cstride));
                d[u] = tot[c0 + u];
            }
    };
    auto consume = [&](int c0, const V (&v)[K], const S (&d)[K]) {
#pragma unroll
        for (int u = 0; u < K; ++u)
            if (c0 + u < nc) {
                store_state<T>(bo + (int64_t)(c0 + u) * cstride, s);
                s = fma4(exp2_fast((float)d[u]), s, as_float4(v[u]));
            }
    };
    load(0, va, da);
    for (int c = 0; c < nc; c += 2 * K) {
        load(c + K, vb, db);
        consume(c, va, da);
        load(c + 2 * K, va, da);
        consume(c + K, vb, db);
    }
    if (p.final_state) *reinterpret_cast<float4 *>(p.final_state + std_off) = s;
}

// Short chains (at most KS chunks, the whole chain in one load phase): EPT groups of 256
// elements per wave, so that a wave has enough loads in flight to cover its own start-up.
// Each chunk's state is a uniform base plus a 32-bit per-lane offset.
template <typename T, int KS, int EPT>
__global__ __launch_bounds__(64) void state_pass_short_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.z / p0.batch);
    typedef typename TF<T>::type V;
    typedef typename CumT<T>::type S;
    const int PN = p.P * p.N;
    const int h = blockIdx.y, b = blockIdx.z % p0.batch;
    const int nc = p.nc;
    const int64_t cbytes = (int64_t)p.H * PN * (int64_t)sizeof(T);    // between chunks
    const int64_t hbase = (((int64_t)b * p.nc * p.H + h) * PN) * (int64_t)sizeof(T);
    const unsigned char *bi = reinterpret_cast<const unsigned char *>(p.b_intra) + hbase;
    unsigned char *bo = reinterpret_cast<unsigned char *>(p.b_in) + hbase;
    const S *tot = reinterpret_cast<const S *>(p.ctot) + ((int64_t)b * p.H + h) * p.nc;

    uint32_t voff[EPT];
    bool on[EPT];
    float4 s[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = ((blockIdx.x * EPT + j) * 64 + threadIdx.x) * 4;
        on[j] = e < PN;                                      // uniform: PN is a multiple of 256
        voff[j] = (uint32_t)(on[j] ? e : 0) * (uint32_t)sizeof(T);
        s[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    V v[KS][EPT];
#pragma unroll
    for (int u = 0; u < KS; ++u)
        if (u < nc) {                                        // uniform
            const unsigned char *src = bi + u * cbytes;
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (on[j]) v[u][j] = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + voff[j]));
        }
    if (p.init) {
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (on[j]) {
                const StateIdx pn = tile_elem((int)(voff[j] / sizeof(T)), p.P);
                s[j] = *reinterpret_cast<const float4 *>(p.init + (((int64_t)b * p.H + h) * p.P + pn.p) * p.N + pn.n0);
            }
    }
#pragma unroll
    for (int u = 0; u < KS; ++u)
        if (u < nc) {
            const float a = exp2_fast((float)tot[u]);
            unsigned char *dst = bo + u * cbytes;
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (on[j]) {
                    store_state<T>(reinterpret_cast<T *>(dst + voff[j]), s[j]);
                    s[j] = fma4(a, s[j], as_float4(v[u][j]));
                }
        }
    if (p.final_state) {
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (on[j]) {
                const StateIdx pn = tile_elem((int)(voff[j] / sizeof(T)), p.P);
                *reinterpret_cast<float4 *>(p.final_state + (((int64_t)b * p.H + h) * p.P + pn.p) * p.N + pn.n0) = s[j];
            }
    }
}

template <typename T, int KS, int EPT>
static void launch_short(const Problem &p, hipStream_t s) {
    const int PN = p.P * p.N;
    dim3 grid((PN / 4 + 64 * EPT - 1) / (64 * EPT), p.H, p.batch * step_count(p));
    state_pass_short_kernel<T, KS, EPT><<<grid, 64, 0, s>>>(p);
}

hipError_t launch_state_pass(const Problem &p, hipStream_t s) {
    const int PN = p.P * p.N;
    const int z = p.batch * step_count(p);
    // chains of at most 8 chunks: 4 element groups per wave; at most 16: 2
    if (p.nc <= 8) {
        if (p.dtype == 1) launch_short<bf16, 8, 4>(p, s);
        else launch_short<float, 8, 4>(p, s);
    } else if (p.nc <= 16) {
        if (p.dtype == 1) launch_short<bf16, 16, 2>(p, s);
        else launch_short<float, 16, 2>(p, s);
    } else {
        dim3 grid((PN / 4 + 63) / 64, p.H, z);
        if (p.dtype == 1) state_pass_kernel<bf16, 16><<<grid, 64, 0, s>>>(p);
        else state_pass_kernel<float, 8><<<grid, 64, 0, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace ssd

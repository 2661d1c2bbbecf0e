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
// it next, and keeping its stores cacheable measured faster than streaming them).
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

template <typename T>
__global__ __launch_bounds__(64) void state_pass_kernel(Problem p0) {
    const Problem p = step_problem(p0, blockIdx.z / p0.batch);
    typedef typename TF<T>::type V;
    typedef typename CumT<T>::type S;
    constexpr int K = sizeof(T) == 2 ? 16 : 8;         // chunks per load group
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

hipError_t launch_state_pass(const Problem &p, hipStream_t s) {
    const int PN = p.P * p.N;
    dim3 grid((PN / 4 + 63) / 64, p.H, p.batch * step_count(p));
    if (p.dtype == 1) state_pass_kernel<bf16><<<grid, 64, 0, s>>>(p);
    else state_pass_kernel<float><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace ssd

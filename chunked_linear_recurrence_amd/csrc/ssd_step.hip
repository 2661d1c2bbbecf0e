// ssd_step: one token of the recurrence of [分块推理 §2] of the page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理", continuing from a carried state
// (the per-layer fixed-size state that the page's §2.3 keeps in memory, here used to
// generate one token at a time after a chunked prefill):
//
//     a = exp(dt[b,h] * A[h]);   S = a S + x (outer) B;   y[b,h,p] = sum_n C[n] S[p,n] + D[h] x[p]
//
// State S is float32 [batch, H, P, N], updated in place; y is rounded once to the
// activation dtype.  The step is a pure HBM stream over the state (read and write 4 bytes
// per element), so each thread owns 4 consecutive n of one state row (one float4 load and
// store), and the N/4 threads of a row reduce their partial C.S sums with wave shuffles.
#include "ssd_common.h"

namespace ssd {

template <typename T>
__device__ __forceinline__ float4 load4(const T *p);
template <>
__device__ __forceinline__ float4 load4<float>(const float *p) { return *reinterpret_cast<const float4 *>(p); }
template <>
__device__ __forceinline__ float4 load4<bf16>(const bf16 *p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// Threads of one row: LPR = N / 4 (a power of two dividing 64); rows per workgroup of 256.
template <typename T, int N>
__global__ __launch_bounds__(256) void ssd_step_kernel(StepArgs a) {
    constexpr int LPR = N / 4;
    constexpr int RPW = 256 / LPR;
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "a state row must fit in one wave");
    const int h = blockIdx.y, b = blockIdx.z;
    const int r = blockIdx.x * RPW + threadIdx.x / LPR;     // state row p of this thread
    const int q = threadIdx.x % LPR;                         // its 4 columns: n = 4q .. 4q+3
    if (r >= a.P) return;                                    // whole rows leave together
    const int g = h / (a.H / a.G);
    const T *x = reinterpret_cast<const T *>(a.x) + ((int64_t)b * a.H + h) * a.P;
    const T *dt = reinterpret_cast<const T *>(a.dt) + (int64_t)b * a.H + h;
    const T *Bv = reinterpret_cast<const T *>(a.B) + ((int64_t)b * a.G + g) * N + 4 * q;
    const T *Cv = reinterpret_cast<const T *>(a.C) + ((int64_t)b * a.G + g) * N + 4 * q;
    float *S = a.state + (((int64_t)b * a.H + h) * a.P + r) * N + 4 * q;

    const float decay = expf(to_f32(*dt) * a.A[h]);
    const float xr = to_f32(x[r]);
    const float4 bb = load4<T>(Bv), cc = load4<T>(Cv);
    float4 s = *reinterpret_cast<const float4 *>(S);
    s.x = fmaf(decay, s.x, xr * bb.x);
    s.y = fmaf(decay, s.y, xr * bb.y);
    s.z = fmaf(decay, s.z, xr * bb.z);
    s.w = fmaf(decay, s.w, xr * bb.w);
    *reinterpret_cast<float4 *>(S) = s;
    float part = cc.x * s.x + cc.y * s.y + cc.z * s.z + cc.w * s.w;
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (q == 0) {
        const float dres = (a.D ? a.D[h] : 0.f) + ((a.flags & 1u) ? 1.f : 0.f);
        T *y = reinterpret_cast<T *>(a.y) + ((int64_t)b * a.H + h) * a.P;
        y[r] = from_f32<T>(part + dres * xr);
    }
}

template <typename T, int N>
static hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
    constexpr int RPW = 256 / (N / 4);
    dim3 grid((a.P + RPW - 1) / RPW, a.H, a.batch);
    ssd_step_kernel<T, N><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

bool step_supported(int dstate) {
    return dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128 || dstate == 256;
}

hipError_t launch_ssd_step(const StepArgs &a, hipStream_t s) {
#define SSD_STEP_N(T)                                          \
    switch (a.N) {                                             \
        case 16: return launch_step_t<T, 16>(a, s);            \
        case 32: return launch_step_t<T, 32>(a, s);            \
        case 64: return launch_step_t<T, 64>(a, s);            \
        case 128: return launch_step_t<T, 128>(a, s);          \
        case 256: return launch_step_t<T, 256>(a, s);          \
        default: return hipErrorInvalidValue;                  \
    }
    if (a.dtype == 1) { SSD_STEP_N(bf16) }
    else { SSD_STEP_N(float) }
#undef SSD_STEP_N
}

}  // namespace ssd

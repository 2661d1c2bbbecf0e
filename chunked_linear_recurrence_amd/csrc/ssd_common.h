// Shared definitions of the libssdscan kernels (gfx950 only).
//
// Method: the chunked decomposition of the page
// "分块推理：解锁循环模型并行计算，实现长序列高效处理", §2-§2.2, cited [分块推理 §n].
//
// Matrix-core conventions used by every kernel.  All products are built from 16x16
// output tiles.  For such a tile a lane l (0..63) with row group g = l / 16 holds:
//   output / accumulator  D[4g + r][l % 16]          r = 0..3   (f32x4)
//   A operand             A[l % 16][k]  for 4 values of k
//   B operand             B[k][l % 16]  for the same 4 values of k
// and one "tile fragment" (TF) is those 4 operand values: for a K-slice of 16 the lane
// holds k = 4g + e, e = 0..3.  The contraction only needs A and B to agree on which k
// each (lane group, element) carries, so any consistent assignment is valid; the kernels
// use k = 4g + e everywhere.  This lets the 4 consecutive output rows a lane holds be fed
// back as an A operand without moving data between lanes.
//   bf16: two K=16 slices are fused into one v_mfma_f32_16x16x32_bf16 (8 values/lane).
//   fp32: one K=16 slice is four v_mfma_f32_16x16x4f32 (value e feeds the e-th one).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace ssd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

typedef __bf16 bf16;

constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

// A batch of steps (segment s, layer l) of the vertical stack that run in one launch:
// step k of the batch is segment s = s_first + k of layer l = d - s (all steps of one
// anti-diagonal d = s + l are independent).  Every step is one layer call over one
// segment; its pointers follow from the stack's buffers (see step_problem below).
struct Steps {
    int count;                 // steps in this launch; 0: not a stack launch
    int d, s_first, n_layers, depth;
    int64_t V, Ltotal;         // segment length, tokens of the whole sequence
    const void *x0;            // stack input [batch, Ltotal, H, P]
    void *y_out;               // stack output, same layout
    unsigned char *act;        // [2][depth] segment activation buffers of act_each bytes
    size_t act_each;
    unsigned char *lws;        // [depth] layer workspaces of lws_each bytes
    size_t lws_each;
    size_t o_dA, o_bintra, o_bin, o_ctot, o_dblk, o_wend;   // offsets inside one layer workspace
    const void *dt0, *B0, *C0; // full-sequence dt, B, C
    const float *A0, *D0;      // [n_layers, H]; D0 may be null
    float *states;             // [n_layers, batch, H, P, N]
};

// One layer's arguments, as the kernels see them.  Token t of batch row b of x/y is at
// x + b * x_bs + t * H * P; dt at dt + b * dt_bs + t * H; B/C at B + b * bc_bs + t * G * N.
// For a stack launch (st.count > 0) the fields describe the longest step of the batch
// (L = V, nc = chunks of V): they size the grid, and each block takes its own step's
// fields from step_problem().
struct Problem {
    int batch, L, H, P, N, G, Q, nc;
    int dtype;                 // 0 = f32, 1 = bf16
    const void *x;  int64_t x_bs;
    void *y;        int64_t y_bs;
    const void *dt; int64_t dt_bs;
    const void *B;  const void *C; int64_t bc_bs;
    const float *A; const float *D;          // [H]; D may be null
    const float *init;                       // [batch, H, P, N] or null
    float *final_state;                      // [batch, H, P, N] or null
    uint32_t flags;
    void *dA_cum;      // [batch, H, nc, Q] of CumT<act>: log2-domain prefix sums of dt * A
    void *ctot;        // [batch, H, nc] of CumT<act>: each chunk's total (its last dA_cum)
    float *dblk;       // [batch, H, nc, Q]: decay from each token to the end of its 16-token block
    float *wend;       // [batch, H, nc, Q]: decay from each token to the chunk's end (0 past it)
    void *b_intra;     // [batch, nc, H, P*N] act dtype, tile order
    void *b_in;        // [batch, nc, H, P*N] tile order, act dtype
    int heads_per_wg_state;   // head group of chunk_state
    int heads_per_wg_scan;    // head group of chunk_scan
    Steps st;
};

// Steps in one launch (1 for a plain layer call).
__host__ __device__ inline int step_count(const Problem &p) { return p.st.count > 0 ? p.st.count : 1; }

// The arguments of step k of a stack launch (p itself for a plain layer call).  Segment s
// covers tokens [s V, s V + len); layer 0 reads the stack input, the last layer writes the
// stack output, and layer l in between reads the buffer layer l-1 wrote for the same
// segment: act[(l-1) & 1][s % depth] (the steps of one diagonal have distinct s % depth,
// and a buffer is rewritten only after its reader, one diagonal later, has run).  Layer
// l's state (init and final) is states[l]; the step's intermediates use workspace slot
// s % depth.
__device__ __forceinline__ Problem step_problem(const Problem &p, int k) {
    if (p.st.count == 0) return p;
    const Steps &st = p.st;
    Problem q = p;
    const int s = st.s_first + k, l = st.d - s;
    const int64_t s0 = (int64_t)s * st.V;
    const int64_t len = min(st.V, st.Ltotal - s0);
    q.L = (int)len;
    q.nc = (int)((len + p.Q - 1) / p.Q);
    const int64_t e = p.dtype == 1 ? 2 : 4;
    const int64_t HP = (int64_t)p.H * p.P, GN = (int64_t)p.G * p.N;
    const int slot = s % st.depth;
    if (l == 0) {
        q.x = static_cast<const unsigned char *>(st.x0) + s0 * HP * e;
        q.x_bs = st.Ltotal * HP;
    } else {
        q.x = st.act + (size_t)(((l - 1) & 1) * st.depth + slot) * st.act_each;
        q.x_bs = st.V * HP;
    }
    if (l == st.n_layers - 1) {
        q.y = static_cast<unsigned char *>(st.y_out) + s0 * HP * e;
        q.y_bs = st.Ltotal * HP;
    } else {
        q.y = st.act + (size_t)((l & 1) * st.depth + slot) * st.act_each;
        q.y_bs = st.V * HP;
    }
    q.dt = static_cast<const unsigned char *>(st.dt0) + s0 * p.H * e;
    q.dt_bs = st.Ltotal * p.H;
    q.B = static_cast<const unsigned char *>(st.B0) + s0 * GN * e;
    q.C = static_cast<const unsigned char *>(st.C0) + s0 * GN * e;
    q.bc_bs = st.Ltotal * GN;
    q.A = st.A0 + (size_t)l * p.H;
    q.D = st.D0 ? st.D0 + (size_t)l * p.H : nullptr;
    float *ls = st.states + (size_t)l * p.batch * HP * p.N;
    q.init = ls;
    q.final_state = ls;
    unsigned char *w = st.lws + (size_t)slot * st.lws_each;
    q.dA_cum = w + st.o_dA;
    q.ctot = w + st.o_ctot;
    q.dblk = reinterpret_cast<float *>(w + st.o_dblk);
    q.wend = reinterpret_cast<float *>(w + st.o_wend);
    q.b_intra = w + st.o_bintra;
    q.b_in = w + st.o_bin;
    return q;
}

// One decode step (ssd_step): one token per (batch, head), state updated in place.
struct StepArgs {
    int batch, H, P, N, G, dtype;
    const void *x;       // [batch, H, P] act
    const void *dt;      // [batch, H] act
    const void *B;       // [batch, G, N] act
    const void *C;       // [batch, G, N] act
    const float *A;      // [H]
    const float *D;      // [H] or null
    float *state;        // [batch, H, P, N]
    void *y;             // [batch, H, P] act
    uint32_t flags;
};

hipError_t launch_ssd_step(const StepArgs &a, hipStream_t s);

// Lets Kernel use `bytes` of dynamic LDS (beyond the 64 KB default) on the current device.
// The attribute is per device, so it is set once per (kernel, device): a process may call
// the library on several GPUs.
template <auto Kernel>
inline hipError_t allow_lds(int bytes) {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute((const void *)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}
bool step_supported(int dstate);
hipError_t launch_chunk_cumsum(const Problem &p, hipStream_t s);
hipError_t launch_chunk_state(const Problem &p, hipStream_t s);
hipError_t launch_state_pass(const Problem &p, hipStream_t s);
hipError_t launch_chunk_scan(const Problem &p, hipStream_t s);
hipError_t launch_chunk_scan_assoc(const Problem &p, hipStream_t s);
bool chunk_scan_assoc_supported(int dtype, int Q, int P, int N);
bool chunk_state_supported(int dtype, int Q, int P, int N);
bool chunk_scan_supported(int dtype, int Q, int P, int N);

// ---------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------
// Type of the log-decay prefix sums: float64 for float32 activations (the differences
// cum_i - cum_j then keep full fp32 accuracy however large |cum| grows within a chunk),
// float32 for bfloat16 activations.  The sums are kept in base 2 (dt * A / ln 2), so every
// decay exp(sum of dt A) is one hardware 2^x (exp2_fast) with no scaling.
template <typename T> struct CumT { typedef float type; };
template <> struct CumT<float> { typedef double type; };

// 1 / ln 2: converts natural-log decay rates dt * A to base 2.
constexpr double kLog2e = 1.4426950408889634074;

// 2^x with the hardware's transcendental unit (v_exp_f32, ~1 ulp; 0 for x below the
// smallest representable result).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct TF;
template <> struct TF<float> { typedef f32x4 type; };
template <> struct TF<bf16> { typedef bf16x4 type; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// acc += A0 * B0 (+ A1 * B1): one or two K=16 slices.
__device__ __forceinline__ f32x4 mma_one(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                       __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_pair(bf16x4 a0, bf16x4 b0, bf16x4 a1, bf16x4 b1, f32x4 c) {
    bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_one(f32x4 a, f32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mma_pair(f32x4 a0, f32x4 b0, f32x4 a1, f32x4 b1, f32x4 c) {
    return mma_one(a1, b1, mma_one(a0, b0, c));
}

template <typename V> __device__ __forceinline__ V zero_frag() { V v; for (int i = 0; i < 4; ++i) v[i] = 0; return v; }

template <typename T>
__device__ __forceinline__ typename TF<T>::type frag_from_f32(f32x4 v) {
    typename TF<T>::type r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = from_f32<T>(v[i]);
    return r;
}

// Consecutive workgroups go round-robin to the 8 XCDs (each with its own L2).  Remap so
// that logically adjacent workgroups (which share B/C data) land on the same XCD.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    if ((n & 7) != 0) return bid;
    const int per = n >> 3;
    return (bid & 7) * per + (bid >> 3);
}

}  // namespace ssd

// C-ABI entry points of libssdscan: argument checks, workspace carving and the launch
// sequence chunk_cumsum -> chunk_state -> state_pass -> chunk_scan on the caller's
// stream.  Nothing here allocates device memory or waits on the device.
//
// Steps follow the page "分块推理：解锁循环模型并行计算，实现长序列高效处理":
// [分块推理 §2.1] (intra-chunk parts from a zero state), [分块推理 §2.2] (state pass and
// the by_inter correction) and, for the layer stack, [分块推理 §3.2] (vertical segments
// with a per-layer state store).
#include "libssdscan.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "ssd_common.h"

namespace {

thread_local std::string g_err;

ssd_status_t fail(ssd_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

ssd_status_t ok() {
    g_err.clear();
    return SSD_OK;
}

constexpr size_t kAlign = 256;
constexpr int kStages = 4;   // chunk_cumsum, chunk_state, state_pass, chunk_scan
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t dA, bintra, bin, ctot, dblk, wend, total;
};

int64_t act_bytes(int32_t dtype) { return dtype == SSD_BF16 ? 2 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t lim, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > lim / a) return false;
    *out = a * b;
    return true;
}

// Workspace of one layer call over `L` tokens.
bool layout_for(const ssd_dims_t &d, int64_t L, int32_t Q, Layout *lo) {
    const int64_t lim = INT64_C(1) << 60;
    const int64_t nc = (L + Q - 1) / Q;
    int64_t bhn, states, t;
    if (!mul_ok(d.batch, d.nheads, lim, &bhn) || !mul_ok(bhn, nc, lim, &bhn)) return false;
    if (!mul_ok(d.headdim, d.dstate, lim, &states) || !mul_ok(states, bhn, lim, &states)) return false;
    if (!mul_ok(bhn, Q, lim, &t)) return false;
    size_t off = 0;
    lo->dA = off;
    off += align_up((size_t)t * (d.dtype == SSD_F32 ? 8 : 4));
    lo->bintra = off;
    off += align_up((size_t)states * act_bytes(d.dtype));
    lo->bin = off;
    off += align_up((size_t)states * act_bytes(d.dtype));
    // each chunk's total log-decay, contiguous per (batch, head) for the state pass
    lo->ctot = off;
    off += align_up((size_t)bhn * (d.dtype == SSD_F32 ? 8 : 4));
    // per token, the decay to the end of its 16-token block (float32), for chunk_scan
    lo->dblk = off;
    off += align_up((size_t)t * 4);
    // per token, the decay to the end of its chunk (float32, 0 past a short chunk), for
    // chunk_state
    lo->wend = off;
    off += align_up((size_t)t * 4);
    lo->total = off;
    return true;
}

ssd_status_t check_dims(const ssd_dims_t *d, int32_t Q) {
    if (!d) return fail(SSD_ERR_NULL_ARG, "dims is NULL");
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16)
        return fail(SSD_ERR_BAD_DTYPE, "dtype %d is not SSD_F32 (0) or SSD_BF16 (1)", d->dtype);
    if (d->reserved != 0) return fail(SSD_ERR_BAD_SHAPE, "dims.reserved must be 0");
    if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 ||
        d->ngroups <= 0)
        return fail(SSD_ERR_BAD_SHAPE, "every dimension must be >= 1 (batch %lld seqlen %lld nheads %lld "
                    "headdim %lld dstate %lld ngroups %lld)", (long long)d->batch, (long long)d->seqlen,
                    (long long)d->nheads, (long long)d->headdim, (long long)d->dstate, (long long)d->ngroups);
    if (d->nheads % d->ngroups != 0)
        return fail(SSD_ERR_BAD_SHAPE, "nheads %lld is not a multiple of ngroups %lld",
                    (long long)d->nheads, (long long)d->ngroups);
    if (Q <= 0) return fail(SSD_ERR_BAD_SHAPE, "chunk_Q must be >= 1 (got %d)", Q);
    if (d->seqlen > INT32_MAX || d->nheads > 65536 || d->batch > 65536 ||
        d->nheads * d->headdim > INT32_MAX / 16)
        return fail(SSD_ERR_UNSUPPORTED, "dimensions exceed the 32-bit index range of the kernels");
    // the kernels address one chunk of x, y, B or C with 32-bit byte offsets
    const int64_t e = act_bytes(d->dtype);
    if ((int64_t)Q * d->nheads * d->headdim * e > INT32_MAX || (int64_t)Q * d->ngroups * d->dstate * e > INT32_MAX ||
        d->headdim * d->dstate * e > INT32_MAX)
        return fail(SSD_ERR_UNSUPPORTED, "one chunk of x or B, or one state, spans more than 2^31 bytes");
    if (!ssd_shape_supported(d->dtype, Q, d->headdim, d->dstate))
        return fail(SSD_ERR_UNSUPPORTED, "no compiled kernel for dtype %d chunk_Q %d headdim %lld dstate %lld",
                    d->dtype, Q, (long long)d->headdim, (long long)d->dstate);
    const int64_t nc = (d->seqlen + Q - 1) / Q;
    if (d->batch * nc * d->nheads > INT32_MAX)
        return fail(SSD_ERR_UNSUPPORTED, "batch * chunks * heads exceeds the grid range");
    return SSD_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Tensors read or written with 16-byte vector accesses must be 16-byte aligned; A and D
// (scalar float loads) need 4 bytes, dt its element size.
ssd_status_t check_alignment(const void *x, const void *dt, const void *A, const void *B, const void *C,
                             const void *D, const void *init, const void *y, const void *fin,
                             const void *ws, int32_t dtype) {
    const void *vec[] = {x, B, C, init, y, fin, ws};
    for (const void *q : vec)
        if (q && !aligned16(q)) return fail(SSD_ERR_MISALIGNED, "pointer %p is not 16-byte aligned", q);
    const uintptr_t dtal = dtype == SSD_BF16 ? 2 : 4;
    if (((uintptr_t)dt & (dtal - 1)) || ((uintptr_t)A & 3u) || (D && ((uintptr_t)D & 3u)))
        return fail(SSD_ERR_MISALIGNED, "dt, A or D is not aligned to its element size");
    return SSD_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Work partition: heads per workgroup so that there are at least `target` workgroups
// (when the problem has that many heads to spread).  Only the split changes, never the
// arithmetic of any output element.
int env_heads(const char *env, int64_t hpg) {
    if (const char *s = getenv(env)) {
        const int v = atoi(s);
        if (v >= 1) return (int)(v < hpg ? v : hpg);
    }
    return 0;
}

constexpr int64_t kCUs = 256;     // compute units of one MI355X

// chunk_scan takes most of a CU's LDS, so one workgroup runs per CU: the smallest equal
// split of the group's heads that fits the grid in one round of workgroups (all heads of
// the group when even that is more than one round).  Fewer heads per workgroup leave the
// C.B^T tiles amortised over fewer heads; a second round leaves a tail.  Measured: 48 heads
// per workgroup at the 128K-token layer (443 us, against 460-496 with 24, 16 or 12), 16 at
// batch 8 x 4K tokens (80 us, against 93 with 8 and 126 with 32), 2 at the Mamba-2-130M
// layer (batch 2 x 2K tokens: 25 us, against 38 with 1 and 31 with 4).
int heads_per_wg_scan(int64_t units, int64_t hpg) {
    if (const int v = env_heads("SSD_HEADS_PER_WG_SCAN", hpg)) return v;
    for (int d = 1; d < hpg; ++d)
        if (hpg % d == 0 && units * (hpg / d) <= kCUs) return d;
    return (int)hpg;
}

// chunk_state: the largest divisor of the group's heads, at most 16, that still leaves a
// full round of resident workgroups (two per CU on 256 CUs).  Equal groups: a ragged last
// group measured 5-10% slower; 16 heads measured best at the 128K-token layer (238 us
// against 252 with 24 or 12) and 8 at batch 8 x 4K tokens (50 us against 51.5 with 4).
int heads_per_wg_state(int64_t units, int64_t hpg) {
    if (const int v = env_heads("SSD_HEADS_PER_WG_STATE", hpg)) return v;
    int best = 1;
    for (int d = 1; d <= 16 && d <= hpg; ++d)
        if (hpg % d == 0 && units * (hpg / d) >= 2 * kCUs) best = d;
    return best;
}

ssd::Problem make_problem(const ssd_dims_t &d, int64_t L, int32_t Q, int steps = 1) {
    ssd::Problem p;
    memset(&p, 0, sizeof(p));
    p.batch = (int)d.batch;
    p.L = (int)L;
    p.H = (int)d.nheads;
    p.P = (int)d.headdim;
    p.N = (int)d.dstate;
    p.G = (int)d.ngroups;
    p.Q = Q;
    p.nc = (int)((L + Q - 1) / Q);
    p.dtype = d.dtype;
    const int64_t units = d.batch * p.nc * d.ngroups * steps;
    const int64_t hpg = d.nheads / d.ngroups;
    p.heads_per_wg_state = heads_per_wg_state(units, hpg);
    p.heads_per_wg_scan = heads_per_wg_scan(units, hpg);
    return p;
}

ssd_status_t run_layer(const ssd::Problem &p, hipStream_t s, int first_stage, int last_stage) {
    hipError_t e = hipSuccess;
    auto in = [&](int k) { return first_stage <= k && k <= last_stage; };
    if (in(1) && (e = ssd::launch_chunk_cumsum(p, s)) != hipSuccess)
        return fail(SSD_ERR_HIP, "chunk_cumsum launch failed: %s", hipGetErrorString(e));
    if (in(2) && (e = ssd::launch_chunk_state(p, s)) != hipSuccess)
        return fail(SSD_ERR_HIP, "chunk_state launch failed: %s", hipGetErrorString(e));
    if (in(3) && (e = ssd::launch_state_pass(p, s)) != hipSuccess)
        return fail(SSD_ERR_HIP, "state_pass launch failed: %s", hipGetErrorString(e));
    if (in(4) && (e = (p.flags & SSD_FLAG_SCAN_FORM) ? ssd::launch_chunk_scan_assoc(p, s)
                                                      : ssd::launch_chunk_scan(p, s)) != hipSuccess)
        return fail(SSD_ERR_HIP, "chunk_scan launch failed: %s", hipGetErrorString(e));
    return SSD_OK;
}

ssd_status_t fwd_impl(const ssd_dims_t *dims, const void *x, const void *dt, const float *A,
                      const void *B, const void *C, const float *D, const float *init_state,
                      int32_t chunk_Q, void *y, float *final_state, uint32_t flags, void *workspace,
                      size_t workspace_bytes, void *stream, int first_stage, int last_stage) {
    ssd_status_t st = check_dims(dims, chunk_Q);
    if (st != SSD_OK) return st;
    const ssd_dims_t &d = *dims;
    if (!x || !dt || !A || !B || !C || !y)
        return fail(SSD_ERR_NULL_ARG, "x, dt, A, B, C and y must be non-NULL");
    if (flags & ~(SSD_FLAG_RESIDUAL | SSD_FLAG_SCAN_FORM)) return fail(SSD_ERR_BAD_SHAPE, "unknown flag bits 0x%x", flags);
    if ((flags & SSD_FLAG_SCAN_FORM) && !ssd::chunk_scan_assoc_supported(d.dtype, chunk_Q, (int)d.headdim, (int)d.dstate))
        return fail(SSD_ERR_UNSUPPORTED, "no scan-form kernel for dtype %d chunk_Q %d headdim %lld dstate %lld",
                    d.dtype, chunk_Q, (long long)d.headdim, (long long)d.dstate);
    if (st = check_alignment(x, dt, A, B, C, D, init_state, y, final_state, workspace, d.dtype); st != SSD_OK)
        return st;
    Layout lo;
    if (!layout_for(d, d.seqlen, chunk_Q, &lo)) return fail(SSD_ERR_BAD_SHAPE, "sizes overflow");
    if (!workspace || workspace_bytes < lo.total)
        return fail(SSD_ERR_WORKSPACE, "workspace %p of %zu bytes; %zu bytes are needed", workspace,
                    workspace_bytes, lo.total);
    const size_t e = (size_t)act_bytes(d.dtype);
    const size_t nx = (size_t)(d.batch * d.seqlen * d.nheads * d.headdim) * e;
    const size_t ns = (size_t)(d.batch * d.nheads * d.headdim * d.dstate) * 4;
    if (overlap(y, nx, x, nx)) return fail(SSD_ERR_ALIAS, "y overlaps x");
    if (final_state && init_state && final_state != init_state && overlap(final_state, ns, init_state, ns))
        return fail(SSD_ERR_ALIAS, "final_state partially overlaps init_state");
    if (overlap(workspace, lo.total, x, nx) || overlap(workspace, lo.total, y, nx))
        return fail(SSD_ERR_ALIAS, "workspace overlaps x or y");
    if (final_state && overlap(final_state, ns, y, nx)) return fail(SSD_ERR_ALIAS, "final_state overlaps y");

    ssd::Problem p = make_problem(d, d.seqlen, chunk_Q);
    p.x = x;
    p.x_bs = d.seqlen * d.nheads * d.headdim;
    p.y = y;
    p.y_bs = p.x_bs;
    p.dt = dt;
    p.dt_bs = d.seqlen * d.nheads;
    p.B = B;
    p.C = C;
    p.bc_bs = d.seqlen * d.ngroups * d.dstate;
    p.A = A;
    p.D = D;
    p.init = init_state;
    p.final_state = final_state;
    p.flags = flags;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.dA_cum = ws + lo.dA;
    p.ctot = ws + lo.ctot;
    p.dblk = reinterpret_cast<float *>(ws + lo.dblk);
    p.wend = reinterpret_cast<float *>(ws + lo.wend);
    p.b_intra = ws + lo.bintra;
    p.b_in = ws + lo.bin;
    st = run_layer(p, static_cast<hipStream_t>(stream), first_stage, last_stage);
    return st == SSD_OK ? ok() : st;
}

// Scratch of ssd_chunk_scan_fwd_noalloc: the layer workspace lives in this file-scope
// device array instead of caller memory.  Each GPU the library runs on holds its own copy
// (SSD_NOALLOC_SCRATCH_BYTES) from module load until the process ends.  In host code the
// array's name is only a stand-in: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device (scratch_on_current_device) and used for
// every kernel argument.  Nothing in the workspace needs to start at zero (every stage
// writes what the next one reads), so nothing is cleared between calls.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The address of this GPU's scratch array (the device current on the calling thread).
ssd_status_t scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SSD_ERR_UNSUPPORTED, "device index %d is beyond the %d devices the scratch table covers",
                    dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

}  // namespace

extern "C" {

int32_t ssd_scan_form_supported(int32_t dtype, int32_t chunk_Q, int64_t headdim, int64_t dstate) {
    if (dtype != SSD_F32 && dtype != SSD_BF16) return 0;
    if (headdim > 1024 || dstate > 1024 || !ssd_shape_supported(dtype, chunk_Q, headdim, dstate)) return 0;
    return ssd::chunk_scan_assoc_supported(dtype, chunk_Q, (int)headdim, (int)dstate);
}

int32_t ssd_shape_supported(int32_t dtype, int32_t chunk_Q, int64_t headdim, int64_t dstate) {
    if (dtype != SSD_F32 && dtype != SSD_BF16) return 0;
    if (headdim > 1024 || dstate > 1024) return 0;
    const int P = (int)headdim, N = (int)dstate;
    return ssd::chunk_state_supported(dtype, chunk_Q, P, N) && ssd::chunk_scan_supported(dtype, chunk_Q, P, N);
}

size_t ssd_chunk_scan_workspace_bytes(const ssd_dims_t *dims, int32_t chunk_Q) {
    if (check_dims(dims, chunk_Q) != SSD_OK) return 0;
    Layout lo;
    if (!layout_for(*dims, dims->seqlen, chunk_Q, &lo)) return 0;
    return lo.total;
}

ssd_status_t ssd_chunk_scan_fwd(const ssd_dims_t *dims, const void *x, const void *dt, const float *A,
                                const void *B, const void *C, const float *D, const float *init_state,
                                int32_t chunk_Q, void *y, float *final_state, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_impl(dims, x, dt, A, B, C, D, init_state, chunk_Q, y, final_state, flags, workspace,
                    workspace_bytes, stream, 1, kStages);
}

ssd_status_t ssd_chunk_scan_fwd_noalloc(const ssd_dims_t *dims, const void *x, const void *dt, const float *A,
                                        const void *B, const void *C, const float *D, const float *init_state,
                                        int32_t chunk_Q, void *y, float *final_state, uint32_t flags,
                                        void *stream) {
    // The size check runs before anything touches the device.
    ssd_status_t st = check_dims(dims, chunk_Q);
    if (st != SSD_OK) return st;
    Layout lo;
    if (!layout_for(*dims, dims->seqlen, chunk_Q, &lo)) return fail(SSD_ERR_BAD_SHAPE, "sizes overflow");
    if (lo.total > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
        return fail(SSD_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the no-allocation entry "
                    "point has %zu (use ssd_chunk_scan_fwd with a caller workspace)", lo.total,
                    (size_t)SSD_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != SSD_OK) return st;
    return fwd_impl(dims, x, dt, A, B, C, D, init_state, chunk_Q, y, final_state, flags, ws,
                    (size_t)SSD_NOALLOC_SCRATCH_BYTES, stream, 1, kStages);
}

ssd_status_t ssd_chunk_scan_stages(const ssd_dims_t *dims, const void *x, const void *dt, const float *A,
                                   const void *B, const void *C, const float *D, const float *init_state,
                                   int32_t chunk_Q, void *y, float *final_state, uint32_t flags,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   int32_t first_stage, int32_t last_stage) {
    if (first_stage < 1 || last_stage > kStages || first_stage > last_stage)
        return fail(SSD_ERR_BAD_SHAPE, "stages must satisfy 1 <= first_stage <= last_stage <= %d", kStages);
    return fwd_impl(dims, x, dt, A, B, C, D, init_state, chunk_Q, y, final_state, flags, workspace,
                    workspace_bytes, stream, first_stage, last_stage);
}

ssd_status_t ssd_workspace_layout(const ssd_dims_t *dims, int32_t chunk_Q, size_t offsets[4]) {
    ssd_status_t st = check_dims(dims, chunk_Q);
    if (st != SSD_OK) return st;
    if (!offsets) return fail(SSD_ERR_NULL_ARG, "offsets is NULL");
    Layout lo;
    if (!layout_for(*dims, dims->seqlen, chunk_Q, &lo)) return fail(SSD_ERR_BAD_SHAPE, "sizes overflow");
    offsets[0] = lo.dA;
    offsets[1] = lo.bintra;
    offsets[2] = lo.bin;
    offsets[3] = lo.total;
    return ok();
}

// Segmented (vertical) stack: workspace = 2 * depth segment activation buffers + depth
// layer workspaces over one segment (depth 1 without SSD_FLAG_WAVEFRONT).
struct SegLayout {
    int64_t Vs;          // tokens of the longest segment
    int nseg, depth;
    size_t act_each, lws_each, act_off, lws_off, total;
    Layout lo;           // one layer workspace over Vs tokens
};

static bool seg_layout(const ssd_dims_t &d, int32_t Q, int64_t V, int32_t n_layers, uint32_t flags,
                       SegLayout *sl) {
    if (V < 1 || n_layers < 1) return false;
    sl->Vs = V < d.seqlen ? V : d.seqlen;
    const int64_t nseg = (d.seqlen + V - 1) / V;
    if (nseg > INT32_MAX) return false;
    sl->nseg = (int)nseg;
    sl->depth = (flags & SSD_FLAG_WAVEFRONT) ? (int)(nseg < n_layers ? nseg : n_layers) : 1;
    if (!layout_for(d, sl->Vs, Q, &sl->lo)) return false;
    int64_t act;
    if (!mul_ok(d.batch * sl->Vs, d.nheads * d.headdim, INT64_C(1) << 60, &act)) return false;
    sl->act_each = align_up((size_t)act * (size_t)act_bytes(d.dtype));
    sl->lws_each = sl->lo.total;
    sl->act_off = 0;
    sl->lws_off = 2 * (size_t)sl->depth * sl->act_each;
    sl->total = sl->lws_off + (size_t)sl->depth * sl->lws_each;
    return true;
}

size_t ssd_segmented_workspace_bytes(const ssd_dims_t *dims, int32_t chunk_Q, int64_t V, int32_t n_layers,
                                     uint32_t flags) {
    if (check_dims(dims, chunk_Q) != SSD_OK || (flags & ~(SSD_FLAG_RESIDUAL | SSD_FLAG_WAVEFRONT))) return 0;
    SegLayout sl;
    if (!seg_layout(*dims, chunk_Q, V, n_layers, flags, &sl)) return 0;
    return sl.total;
}

ssd_status_t ssd_chunk_scan_segmented(const ssd_dims_t *dims, int32_t n_layers, int64_t V, const void *x0,
                                      const void *dt, const float *A, const void *B, const void *C,
                                      const float *D, float *layer_states, int32_t chunk_Q, uint32_t flags,
                                      void *y, void *workspace, size_t workspace_bytes, void *stream) {
    ssd_status_t st = check_dims(dims, chunk_Q);
    if (st != SSD_OK) return st;
    const ssd_dims_t &d = *dims;
    if (n_layers < 1) return fail(SSD_ERR_BAD_SHAPE, "n_layers must be >= 1 (got %d)", n_layers);
    if (V < 1) return fail(SSD_ERR_BAD_SHAPE, "V must be >= 1 (got %lld)", (long long)V);
    if (!x0 || !dt || !A || !B || !C || !layer_states || !y)
        return fail(SSD_ERR_NULL_ARG, "x0, dt, A, B, C, layer_states and y must be non-NULL");
    if (flags & ~(SSD_FLAG_RESIDUAL | SSD_FLAG_WAVEFRONT))
        return fail(SSD_ERR_BAD_SHAPE, "unknown flag bits 0x%x", flags);
    if (st = check_alignment(x0, dt, A, B, C, D, layer_states, y, layer_states, workspace, d.dtype); st != SSD_OK)
        return st;
    SegLayout sl;
    if (!seg_layout(d, chunk_Q, V, n_layers, flags, &sl)) return fail(SSD_ERR_BAD_SHAPE, "sizes overflow");
    if (!workspace || workspace_bytes < sl.total)
        return fail(SSD_ERR_WORKSPACE, "workspace %p of %zu bytes; %zu bytes are needed", workspace,
                    workspace_bytes, sl.total);
    const size_t e = (size_t)act_bytes(d.dtype);
    const size_t nx = (size_t)(d.batch * d.seqlen * d.nheads * d.headdim) * e;
    const size_t ns = (size_t)n_layers * (size_t)(d.batch * d.nheads * d.headdim * d.dstate) * 4;
    if (overlap(y, nx, x0, nx)) return fail(SSD_ERR_ALIAS, "y overlaps x0");
    if (overlap(workspace, sl.total, x0, nx) || overlap(workspace, sl.total, y, nx) ||
        overlap(workspace, sl.total, layer_states, ns) || overlap(layer_states, ns, y, nx))
        return fail(SSD_ERR_ALIAS, "workspace, layer_states and y must not overlap each other or x0");

    unsigned char *ws = static_cast<unsigned char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Every step (segment s, layer l) is the same layer call in both schedules; only how
    // many of them share a launch differs.  The steps of anti-diagonal dg are segments
    // s_lo..s_hi with l = dg - s.
    const int S = sl.nseg;
    const int last_diag = S - 1 + n_layers - 1;
    for (int dg = 0; sl.depth > 1 && dg <= last_diag; ++dg) {
        const int s_lo = dg - (n_layers - 1) > 0 ? dg - (n_layers - 1) : 0;
        const int s_hi = dg < S - 1 ? dg : S - 1;
        ssd::Problem p = make_problem(d, sl.Vs, chunk_Q, s_hi - s_lo + 1);
        p.flags = flags & SSD_FLAG_RESIDUAL;
        ssd::Steps &q = p.st;
        q.count = s_hi - s_lo + 1;
        q.d = dg;
        q.s_first = s_lo;
        q.n_layers = n_layers;
        q.depth = sl.depth;
        q.V = V;
        q.Ltotal = d.seqlen;
        q.x0 = x0;
        q.y_out = y;
        q.act = ws + sl.act_off;
        q.act_each = sl.act_each;
        q.lws = ws + sl.lws_off;
        q.lws_each = sl.lws_each;
        q.o_dA = sl.lo.dA;
        q.o_ctot = sl.lo.ctot;
        q.o_dblk = sl.lo.dblk;
        q.o_wend = sl.lo.wend;
        q.o_bintra = sl.lo.bintra;
        q.o_bin = sl.lo.bin;
        q.dt0 = dt;
        q.B0 = B;
        q.C0 = C;
        q.A0 = A;
        q.D0 = D;
        q.states = layer_states;
        st = run_layer(p, s, 1, kStages);
        if (st != SSD_OK) return st;
    }
    if (sl.depth == 1) {
        // one step at a time, in the page's order: segment s through every layer, then
        // segment s + 1
        void *act[2] = {ws + sl.act_off, ws + sl.act_off + sl.act_each};
        unsigned char *lws = ws + sl.lws_off;
        const int64_t HP = d.nheads * d.headdim, GN = d.ngroups * d.dstate;
        const int64_t state_elems = d.batch * d.nheads * d.headdim * d.dstate;
        for (int64_t s0 = 0; s0 < d.seqlen; s0 += V) {
            const int64_t len = (d.seqlen - s0) < V ? (d.seqlen - s0) : V;
            for (int l = 0; l < n_layers; ++l) {
                ssd::Problem p = make_problem(d, len, chunk_Q);
                if (l == 0) {
                    p.x = static_cast<const unsigned char *>(x0) + (size_t)(s0 * HP) * e;
                    p.x_bs = d.seqlen * HP;
                } else {
                    p.x = act[(l - 1) & 1];
                    p.x_bs = sl.Vs * HP;
                }
                if (l == n_layers - 1) {
                    p.y = static_cast<unsigned char *>(y) + (size_t)(s0 * HP) * e;
                    p.y_bs = d.seqlen * HP;
                } else {
                    p.y = act[l & 1];
                    p.y_bs = sl.Vs * HP;
                }
                p.dt = static_cast<const unsigned char *>(dt) + (size_t)(s0 * d.nheads) * e;
                p.dt_bs = d.seqlen * d.nheads;
                p.B = static_cast<const unsigned char *>(B) + (size_t)(s0 * GN) * e;
                p.C = static_cast<const unsigned char *>(C) + (size_t)(s0 * GN) * e;
                p.bc_bs = d.seqlen * GN;
                p.A = A + (size_t)l * d.nheads;
                p.D = D ? D + (size_t)l * d.nheads : nullptr;
                p.init = layer_states + (size_t)l * state_elems;
                p.final_state = layer_states + (size_t)l * state_elems;
                p.flags = flags & SSD_FLAG_RESIDUAL;
                p.dA_cum = lws + sl.lo.dA;
                p.ctot = lws + sl.lo.ctot;
                p.dblk = reinterpret_cast<float *>(lws + sl.lo.dblk);
                p.wend = reinterpret_cast<float *>(lws + sl.lo.wend);
                p.b_intra = lws + sl.lo.bintra;
                p.b_in = lws + sl.lo.bin;
                st = run_layer(p, s, 1, kStages);
                if (st != SSD_OK) return st;
            }
        }
    }
    return ok();
}

ssd_status_t ssd_step(const ssd_dims_t *dims, const void *x, const void *dt, const float *A, const void *B,
                      const void *C, const float *D, float *state, void *y, uint32_t flags, void *stream) {
    if (!dims) return fail(SSD_ERR_NULL_ARG, "dims is NULL");
    const ssd_dims_t &d = *dims;
    if (d.dtype != SSD_F32 && d.dtype != SSD_BF16)
        return fail(SSD_ERR_BAD_DTYPE, "dtype %d is not SSD_F32 (0) or SSD_BF16 (1)", d.dtype);
    if (d.reserved != 0) return fail(SSD_ERR_BAD_SHAPE, "dims.reserved must be 0");
    if (d.seqlen != 1) return fail(SSD_ERR_BAD_SHAPE, "ssd_step takes one token: seqlen must be 1 (got %lld)",
                                   (long long)d.seqlen);
    if (d.batch <= 0 || d.nheads <= 0 || d.headdim <= 0 || d.dstate <= 0 || d.ngroups <= 0)
        return fail(SSD_ERR_BAD_SHAPE, "every dimension must be >= 1");
    if (d.nheads % d.ngroups != 0)
        return fail(SSD_ERR_BAD_SHAPE, "nheads %lld is not a multiple of ngroups %lld", (long long)d.nheads,
                    (long long)d.ngroups);
    if (!ssd::step_supported((int)d.dstate))
        return fail(SSD_ERR_UNSUPPORTED, "ssd_step supports dstate 16, 32, 64, 128 or 256 (got %lld)",
                    (long long)d.dstate);
    if (d.batch > 65535 || d.nheads > 65535 || d.headdim > (1 << 20))
        return fail(SSD_ERR_UNSUPPORTED, "dimensions exceed the grid range");
    if (!x || !dt || !A || !B || !C || !state || !y)
        return fail(SSD_ERR_NULL_ARG, "x, dt, A, B, C, state and y must be non-NULL");
    if (flags & ~SSD_FLAG_RESIDUAL) return fail(SSD_ERR_BAD_SHAPE, "unknown flag bits 0x%x", flags);
    const uintptr_t e = (uintptr_t)act_bytes(d.dtype);
    if (!aligned16(state) || !aligned16(B) || !aligned16(C))
        return fail(SSD_ERR_MISALIGNED, "state, B and C must be 16-byte aligned");
    if (((uintptr_t)x & (e - 1)) || ((uintptr_t)dt & (e - 1)) || ((uintptr_t)y & (e - 1)) ||
        ((uintptr_t)A & 3u) || (D && ((uintptr_t)D & 3u)))
        return fail(SSD_ERR_MISALIGNED, "x, dt, y, A or D is not aligned to its element size");
    const size_t nx = (size_t)(d.batch * d.nheads * d.headdim) * e;
    const size_t ns = (size_t)(d.batch * d.nheads * d.headdim * d.dstate) * 4;
    if (overlap(y, nx, x, nx) || overlap(y, nx, state, ns)) return fail(SSD_ERR_ALIAS, "y overlaps x or state");
    ssd::StepArgs a;
    a.batch = (int)d.batch;
    a.H = (int)d.nheads;
    a.P = (int)d.headdim;
    a.N = (int)d.dstate;
    a.G = (int)d.ngroups;
    a.dtype = d.dtype;
    a.x = x;
    a.dt = dt;
    a.B = B;
    a.C = C;
    a.A = A;
    a.D = D;
    a.state = state;
    a.y = y;
    a.flags = flags;
    const hipError_t err = ssd::launch_ssd_step(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(SSD_ERR_HIP, "ssd_step launch failed: %s", hipGetErrorString(err));
    return ok();
}

const char *ssd_status_string(ssd_status_t status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG";
        case SSD_ERR_BAD_SHAPE: return "SSD_ERR_BAD_SHAPE";
        case SSD_ERR_BAD_DTYPE: return "SSD_ERR_BAD_DTYPE";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
        case SSD_ERR_MISALIGNED: return "SSD_ERR_MISALIGNED";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
        case SSD_ERR_HIP: return "SSD_ERR_HIP";
        case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS";
    }
    return "SSD_ERR_UNKNOWN";
}

const char *ssd_last_error_message(void) { return g_err.c_str(); }

int32_t ssd_version(void) { return 100; }

}  // extern "C"

/*
 * libssdscan -- chunked scan of a diagonal-decay selective state-space layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the page
 *   "分块推理：解锁循环模型并行计算，实现长序列高效处理"
 * (chunked inference for recurrent models), cited below as [分块推理 §n].
 *
 * One layer computes, for every batch row b and head h, the recurrence of [分块推理 §2]
 *
 *     a_t = exp(dt[b,t,h] * A[h])                      (per-token, per-head decay)
 *     S_t = a_t * S_{t-1} + x[b,t,h,:] (outer) B[b,t,g,:]   (state S is P x N)
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * S_t[p,n] + D[h] * x[b,t,h,p]
 *
 * with S_{-1} = init_state (or 0) and g = h / (H / G).  The library reaches this result by
 * the chunked decomposition of [分块推理 §2.1-§2.2]: split the sequence into chunks of Q
 * tokens; compute every chunk's intra output and local end state from a zero state;
 * pass the global state b(c) = b_intra(c) + (prod of a_t over chunk c) * b(c-1) across
 * chunks; and correct every chunk's output by diag(L) C b(c-1), where L_i is the product
 * of a_t from the chunk start to token i inclusive.
 *
 * Conventions (readings of the page, which leaves them open):
 *   - dt enters only through a_t; the input term is x (outer) B with no dt factor.
 *   - No softplus, bias or clamp is applied to dt; it is used as given.
 *   - D (skip term) is optional; NULL means no skip term.
 *
 * ---------------------------------------------------------------------------------
 * Memory, ownership, streams
 *   Every pointer argument is device memory owned by the caller (for example a torch
 *   tensor's data pointer).  The library never allocates or frees device memory; the
 *   caller provides a workspace of at least the size the *_workspace_bytes query returns.
 *   All work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *   returns without waiting.  Argument errors are detected on the host before anything
 *   is enqueued, and then nothing is written.  A fault inside a kernel surfaces at the
 *   caller's next synchronisation.  No C++ exception crosses this interface.
 *   The library holds no global mutable state except a per-thread error message (and a
 *   once-per-device kernel attribute), so concurrent calls on different workspaces are
 *   safe.  No entry point allocates or synchronises, so calls can be captured in HIP
 *   graphs.
 *
 * Layouts (row-major, contiguous, element types in parentheses; "act" = the dims' dtype)
 *   x, y             [batch, seqlen, nheads, headdim]          (act)
 *   dt               [batch, seqlen, nheads]                   (act)
 *   A, D             [nheads]                                  (float32)
 *   B, C             [batch, seqlen, ngroups, dstate]          (act)
 *   init_state,
 *   final_state      [batch, nheads, headdim, dstate]          (float32)
 *   x, y, B, C, init_state, final_state, layer_states and the workspace must be 16-byte
 *   aligned; A and D 4-byte aligned; dt aligned to its element size.
 *
 * Supported shapes on the GPU path (others return SSD_ERR_UNSUPPORTED):
 *   chunk_Q in {32, 64, 128, 256}; headdim in {16, 32, 64, 128}; dstate in {16, 32, 64, 128,
 *   256} (bfloat16 needs dstate >= 32); the set actually compiled is reported by
 *   ssd_shape_supported().  Any batch, seqlen >= 1, nheads >= 1 with nheads % ngroups == 0.
 *   The last chunk may be shorter than Q.
 *
 * Values: every a_t must be a decay, 0 <= a_t <= 1, i.e. dt >= 0 and A <= 0, both finite
 *   (as the state transition of [分块推理 §2] is in every workload).  The kernels rely on
 *   it: the log-decay prefix sums of dt * A never increase along a chunk, so every decay
 *   they form between two tokens is exp of a non-positive number (the diagonal tiles of
 *   ssd_chunk_scan_fwd clamp that exponent at 0 to mask the tokens after i).  With a
 *   growing a_t (dt * A > 0) the results are unspecified: they are wrong, and may
 *   overflow.  The library cannot check device-resident values without synchronising, so
 *   it does not; this contract applies to ssd_chunk_scan_fwd, ssd_chunk_scan_stages,
 *   ssd_chunk_scan_segmented and ssd_step.
 *
 * Tuning (environment, read at each call; optional): SSD_HEADS_PER_WG_STATE and
 *   SSD_HEADS_PER_WG_SCAN set how many heads one workgroup of chunk_state / chunk_scan
 *   processes (by default chosen from the problem size).  They change only how the work
 *   is split, never the arithmetic: results are bit-identical for every value.
 */
#ifndef LIBSSDSCAN_H
#define LIBSSDSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
    SSD_ERR_BAD_SHAPE = 2,    /* a dimension <= 0, nheads % ngroups != 0, V < 1, ... */
    SSD_ERR_BAD_DTYPE = 3,    /* dims.dtype is not an ssd_dtype_t value               */
    SSD_ERR_UNSUPPORTED = 4,  /* a valid shape that no compiled kernel covers         */
    SSD_ERR_MISALIGNED = 5,   /* a pointer is not 16-byte aligned                     */
    SSD_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than the query's size      */
    SSD_ERR_HIP = 7,          /* a HIP launch failed (message has the HIP error)      */
    SSD_ERR_ALIAS = 8         /* an output overlaps an input it must not overlap      */
} ssd_status_t;

typedef enum ssd_dtype {
    SSD_F32 = 0,   /* activations stored and computed in float32 (fp32 matrix cores)        */
    SSD_BF16 = 1   /* activations stored in bfloat16, products on bf16 matrix cores, fp32
                      accumulation.  The state carried across chunks is summed in float32;
                      the per-chunk states stored in the workspace (b_intra, b_in) are
                      rounded to bfloat16; decays, init_state and final_state are float32 */
} ssd_dtype_t;

typedef struct ssd_dims {
    int64_t batch;     /* b                                   */
    int64_t seqlen;    /* L, tokens in this call              */
    int64_t nheads;    /* H                                   */
    int64_t headdim;   /* P, x channels per head              */
    int64_t dstate;    /* N, state size per channel           */
    int64_t ngroups;   /* G, B/C groups; head h reads group h / (H / G) */
    int32_t dtype;     /* ssd_dtype_t                         */
    int32_t reserved;  /* must be 0                           */
} ssd_dims_t;

/* flags */
#define SSD_FLAG_RESIDUAL 1u   /* y = (recurrence output + D x) + x, rounded once to act */
#define SSD_FLAG_WAVEFRONT 2u  /* segmented stack only: run independent (segment, layer)
                                  steps together (see ssd_chunk_scan_segmented) */
#define SSD_FLAG_SCAN_FORM 4u  /* ssd_chunk_scan_fwd / _stages only: compute the chunk outputs
                                  with the associative-scan form of [分块推理 §2.1] (a
                                  log-depth tree over the pairs (a_t, x_t B_t) on the vector
                                  units) instead of the matrix-core form; same results within
                                  the tolerances, for comparison.  Shapes:
                                  ssd_scan_form_supported(). */

/* Size in bytes of the workspace ssd_chunk_scan_fwd needs for these dims and chunk_Q,
 * or 0 when the arguments are invalid.  The workspace holds the per-chunk log-decay
 * prefix sums (with each chunk's total), each token's decay to the end of its 16-token
 * block (4 bytes per token and head), and two per-chunk state buffers (nheads * headdim *
 * dstate * 2 * act bytes / chunk_Q bytes per token). */
size_t ssd_chunk_scan_workspace_bytes(const ssd_dims_t *dims, int32_t chunk_Q);

/* One layer, the whole sequence [分块推理 §2-§2.2].
 *   x, dt, A, B, C     inputs (layouts above); D and init_state may be NULL.
 *   chunk_Q            chunk length Q [分块推理 §2, §4.1].
 *   y                  output [batch, seqlen, nheads, headdim] (act); must not overlap x.
 *   final_state        state after the last token, or NULL; may be the same pointer as
 *                      init_state (updated in place), no other overlap allowed.
 *   flags              0, SSD_FLAG_RESIDUAL and/or SSD_FLAG_SCAN_FORM.
 *   workspace          caller-owned device scratch; its contents on entry do not matter.
 * Returns SSD_OK once the kernels are enqueued on `stream`. */
ssd_status_t ssd_chunk_scan_fwd(const ssd_dims_t *dims, const void *x, const void *dt,
                                const float *A, const void *B, const void *C,
                                const float *D, const float *init_state, int32_t chunk_Q,
                                void *y, float *final_state, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream);

/* ssd_chunk_scan_fwd for callers that cannot allocate or pass device memory for a
 * workspace (code under HIP graph capture that must not allocate, tight serving loops,
 * harnesses that forbid allocation): the same computation, the same kernels and
 * bit-identical results, with the workspace taken from a scratch array inside the
 * library instead of a caller buffer.  Nothing is allocated or freed here.
 *   Arguments as for ssd_chunk_scan_fwd, without workspace and workspace_bytes.
 *   Limit: the workspace ssd_chunk_scan_workspace_bytes reports for these dims and chunk_Q
 *   must not exceed SSD_NOALLOC_SCRATCH_BYTES (64 MiB; for example up to ~41K tokens of
 *   batch * seqlen at nheads 24, headdim 64, dstate 128, chunk_Q 256, bf16); larger calls
 *   return SSD_ERR_WORKSPACE before anything is enqueued.
 *   Each GPU the library runs on holds one such array from the library's load until the
 *   process ends, shared by every call on that GPU: calls that overlap on one GPU (on
 *   different streams, or from several threads) race on it and must be serialised by
 *   the caller.  The first call on a device resolves the array's address there.
 * Returns SSD_OK once the kernels are enqueued on `stream`. */
#define SSD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
ssd_status_t ssd_chunk_scan_fwd_noalloc(const ssd_dims_t *dims, const void *x, const void *dt,
                                        const float *A, const void *B, const void *C,
                                        const float *D, const float *init_state, int32_t chunk_Q,
                                        void *y, float *final_state, uint32_t flags, void *stream);

/* Workspace size for ssd_chunk_scan_segmented with these n_layers and flags (0 when the
 * arguments are invalid).  Without SSD_FLAG_WAVEFRONT it is two segment buffers and one
 * layer workspace over V tokens; with it, depth = min(ceil(seqlen / V), n_layers) times
 * that.  Either way it is bounded independently of seqlen: memory stays at a fixed number
 * of segments plus the caller's per-layer states, whatever the sequence length
 * [分块推理 §3.2]. */
size_t ssd_segmented_workspace_bytes(const ssd_dims_t *dims, int32_t chunk_Q, int64_t V,
                                     int32_t n_layers, uint32_t flags);

/* A stack of n_layers layers run in the vertical order of [分块推理 §3.2]: the sequence is
 * cut into segments of V tokens (the last may be shorter); each segment goes through
 * every layer before the next segment starts, and each layer's state is carried between
 * segments in layer_states.
 *   dims               shape of one layer; dims.seqlen is the full length L.
 *   x0                 stack input [batch, L, nheads, headdim] (act).
 *   dt, B, C           shared by every layer (layouts above).
 *   A, D               per layer, [n_layers, nheads] float32 (D may be NULL).
 *   layer_states       [n_layers, batch, nheads, headdim, dstate] float32, in: each layer's
 *                      initial state, out: its state after token L-1.  This is the
 *                      per-(layer) state store of [分块推理 §3.2]; copying it out and back
 *                      between calls resumes the stack exactly.
 *   y                  stack output [batch, L, nheads, headdim] (act): the last layer's
 *                      output; must not overlap x0.
 *   flags              SSD_FLAG_RESIDUAL (applied at every layer) and/or
 *                      SSD_FLAG_WAVEFRONT.
 * Layer l maps u to (recurrence_l(u) + D_l u [+ u]) rounded to act.  When V is a multiple
 * of chunk_Q the result is bit-identical to running ssd_chunk_scan_fwd layer by layer over
 * the whole sequence (the horizontal order of [分块推理 §3.1]).
 * Schedule: step (s, l) is segment s through layer l.  It needs (s, l-1) (its input) and
 * (s-1, l) (layer l's state), nothing else.  Without SSD_FLAG_WAVEFRONT the steps run one
 * at a time, segment by segment, as the page describes.  With it, all steps of one
 * anti-diagonal s + l = const run in the same four kernel launches (up to
 * min(segments, n_layers) steps at once), which fills the GPU when a single step is
 * small; every step computes exactly what it computes alone, so the output and states
 * are bit-identical between the two schedules. */
ssd_status_t ssd_chunk_scan_segmented(const ssd_dims_t *dims, int32_t n_layers, int64_t V,
                                      const void *x0, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      float *layer_states, int32_t chunk_Q, uint32_t flags,
                                      void *y, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* One decode step: the next token of the recurrence of [分块推理 §2], continuing from
 * a carried state (for example the final_state of a chunked prefill), as the per-layer
 * fixed-size state of [分块推理 §2.3] is kept between tokens during generation:
 *     a = exp(dt[b,h] A[h]);   state = a state + x (outer) B;
 *     y[b,h,p] = sum_n C[b,g,n] state[b,h,p,n] + D[h] x[b,h,p]   (+ x with SSD_FLAG_RESIDUAL)
 *   dims        shape of one layer; dims.seqlen must be 1.
 *   x           [batch, nheads, headdim] (act), the token's input.
 *   dt          [batch, nheads] (act).
 *   A, D        [nheads] float32; D may be NULL.
 *   B, C        [batch, ngroups, dstate] (act).
 *   state       [batch, nheads, headdim, dstate] float32, read and written in place.
 *   y           [batch, nheads, headdim] (act); must not overlap x or state.
 *   flags       0 or SSD_FLAG_RESIDUAL.
 * dstate must be one of 16, 32, 64, 128, 256; any headdim >= 1.  Alignment: state, B and
 * C 16 bytes; x, dt, y their element size; A and D 4 bytes.  No workspace; nothing is
 * allocated.  Returns SSD_OK once the kernel is enqueued on `stream`. */
ssd_status_t ssd_step(const ssd_dims_t *dims, const void *x, const void *dt, const float *A,
                      const void *B, const void *C, const float *D, float *state, void *y,
                      uint32_t flags, void *stream);

/* ---- inspection (tests and tools) ------------------------------------------------ */

/* Runs steps first_stage..last_stage of ssd_chunk_scan_fwd (1 = log-decay prefix sums,
 * 2 = per-chunk local states, 3 = state pass, 4 = chunk outputs) and leaves the
 * intermediates in the workspace (see ssd_workspace_layout).  A step reads what the
 * earlier steps left in the same workspace, so running 1..k and then k+1..4 with the same
 * arguments equals one ssd_chunk_scan_fwd call; running one step at a time is how each
 * kernel is timed on its own. */
ssd_status_t ssd_chunk_scan_stages(const ssd_dims_t *dims, const void *x, const void *dt,
                                   const float *A, const void *B, const void *C,
                                   const float *D, const float *init_state, int32_t chunk_Q,
                                   void *y, float *final_state, uint32_t flags,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   int32_t first_stage, int32_t last_stage);

/* Byte offsets of the intermediates inside the workspace:
 *   offsets[0]  dA_cum   [batch, nheads, nchunks, chunk_Q], float64 for SSD_F32 and float32
 *               for SSD_BF16 activations: sum of dt*A / ln 2 (the base-2 logarithm of the
 *               decay) from the chunk start to each token, inclusive (past a short last
 *               chunk: the chunk total);
 *   offsets[1]  b_intra  act dtype, per (batch, chunk, head) a P x N state in tile order;
 *   offsets[2]  b_in     act dtype, the state entering each chunk, same tile order;
 *   offsets[3]  total workspace bytes.
 * Tile order of one P x N state: 16x16 tiles indexed [n / 16][p / 16], each tile 64 lanes
 * x 4 values, where lane l, value r holds (p = 16 * (p / 16) + l % 16,
 * n = 16 * (n / 16) + 4 * (l / 16) + r). */
ssd_status_t ssd_workspace_layout(const ssd_dims_t *dims, int32_t chunk_Q, size_t offsets[4]);

/* 1 when the SSD_FLAG_SCAN_FORM kernel is compiled for (dtype, chunk_Q, headdim, dstate). */
int32_t ssd_scan_form_supported(int32_t dtype, int32_t chunk_Q, int64_t headdim, int64_t dstate);

/* 1 when a compiled kernel set covers (dtype, chunk_Q, headdim, dstate), else 0. */
int32_t ssd_shape_supported(int32_t dtype, int32_t chunk_Q, int64_t headdim, int64_t dstate);

const char *ssd_status_string(ssd_status_t status);
/* Detail of the calling thread's last error ("" when the last call succeeded). */
const char *ssd_last_error_message(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int32_t ssd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBSSDSCAN_H */

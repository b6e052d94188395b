/*
 * ssd.h -- C ABI of libssd: the Mamba-2 chunked SSD forward pass on gfx950.
 *
 * The operation ("Accelerating Mamba-2 with High-Performance Forward Pass
 * Kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture"): for every
 * batch b and head h, with group g = h / (nheads / ngroups),
 *
 *     h_t = exp(A[h] dt_t) h_{t-1} + dt_t B_t x_t^T        (state, dstate x headdim)
 *     y_t = C_t^T h_t + D[h] x_t                          (readout after the update)
 *
 * evaluated chunk by chunk as the pages' three stages (cumulative sum of
 * a_t = A dt_t per chunk; state jump across chunks; chunk output with the
 * causal mask that keeps the diagonal).  The result equals the recurrence up to
 * floating-point rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are dense, row-major (C-contiguous) DEVICE buffers owned by the
 *   caller.  The library allocates nothing, keeps no pointer after a call
 *   returns, holds no mutable global state and is reentrant.
 * - x, dt, B and C have the element type `shape->dtype` (fp32 or bf16); y has
 *   `shape->y_dtype`, which is either fp32 or the input type.  A, D, the
 *   workspace and both state tensors are always fp32.  All arithmetic is fp32
 *   (fp64 for the running decay sum); bf16 inputs are widened exactly.
 * - Layouts (the tile layouts of the pages' kernel sections):
 *       x, y            (batch, seqlen, nheads, headdim)
 *       dt              (batch, seqlen, nheads)
 *       A, D            (nheads)
 *       B, C            (batch, seqlen, ngroups, dstate)
 *       initial_states,
 *       final_states    (batch, nheads, headdim, dstate)   -- the state h^T
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *   the call returns without synchronising.  Buffers must stay valid until the
 *   stream reaches that point.  A fault inside a kernel surfaces at the
 *   caller's next synchronisation of the stream.
 * - Preconditions not checked (checking would need a device read): A <= 0 and
 *   dt >= 0 (so every a_t <= 0, which is what keeps the chunk-output
 *   exponentials bounded), and finite inputs.  Violating them gives
 *   unspecified values, never an out-of-bounds access.
 * - All argument checks happen before the first launch; on any error nothing
 *   is enqueued and the outputs are untouched.  No exception crosses the ABI.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERROR_INVALID_VALUE = 1, /* NULL required pointer, negative size, nheads % ngroups != 0, aliasing */
    SSD_ERROR_UNSUPPORTED = 2,   /* valid problem outside the sizes the kernels are built for */
    SSD_ERROR_MISALIGNED = 3,    /* a pointer below its required alignment */
    SSD_ERROR_WORKSPACE = 4,     /* workspace NULL or smaller than ssd_chunk_scan_fwd_workspace_size */
    SSD_ERROR_LAUNCH = 5,        /* the HIP runtime refused a launch or an event record */
    SSD_ERROR_SCRATCH = 6        /* ssd_chunk_scan_fwd_noalloc: the problem needs more workspace
                                    than the library's scratch holds (SSD_NOALLOC_SCRATCH_BYTES) */
} ssd_status;

/* Keep the per-chunk input states s_c and the chunk-start states h_c in two
 * separate workspace regions (tests read both; ssd_chunk_scan_bwd_saved reads
 * h_c).  Without it the state-passing stage of fp32 problems overwrites s_c
 * with h_c in place. */
enum { SSD_FLAG_KEEP_INTERMEDIATES = 1u };

typedef struct {
    int64_t batch;    /* >= 0 (0: nothing to do) */
    int64_t seqlen;   /* >= 0 (0: final_states = initial_states or 0) */
    int64_t nheads;   /* >= 1 */
    int64_t headdim;  /* P: supported 32, 64, 128 */
    int64_t dstate;   /* N: supported multiples of 16 in [16, 256] */
    int64_t ngroups;  /* >= 1, divides nheads; heads share B/C contiguously */
    int32_t dtype;    /* ssd_dtype of x, dt, B, C */
    uint32_t flags;   /* SSD_FLAG_* */
    int32_t y_dtype;  /* ssd_dtype of y: SSD_DTYPE_F32 (0, the zero-initialised
                         default) or the input dtype.  An fp32 y keeps the full
                         fp32-accumulated result; a bf16 y adds one rounding
                         (relative error <= 2^-9 per element). */
    int32_t reserved; /* must be 0 */
} ssd_shape;

/* Byte offsets of the intermediates inside the workspace (each 256-byte
 * aligned).  Lp = nchunks * chunk_size, nchunks = ceil(seqlen / chunk_size).
 *   G2  fp32 pair (batch, nheads, Lp) at g2_hi and g2_lo: log2(e) * the
 *       per-chunk inclusive cumsum of A dt (the pages' G, kept in base-2 units
 *       so kernels use exp2), summed in fp64 and stored as hi + lo floats so
 *       that differences of nearby entries stay accurate however large the
 *       sum grows within a chunk; positions past seqlen are padded with dt = 0
 *       and so stay flat.
 *   DT  fp32 (batch, nheads, Lp): dt widened to fp32, head-major, zero padded.
 *   W   fp32 (batch, nheads, Lp): exp(G_last - G_t) dt_t, the weight with which
 *       token t enters its chunk's state (G_last: G at the chunk's last
 *       token; the exponent is formed in fp64); 0 past seqlen.
 *   S   fp32 (batch, nheads, nchunks, headdim, dstate): the per-chunk input
 *       states s_c (what a chunk alone adds to a zero state), except for fp32
 *       problems without SSD_FLAG_KEEP_INTERMEDIATES, where H shares this
 *       region and it holds h_c after the call.
 *   H   the chunk-start states h_c (the state before the chunk's first
 *       token), same byte size as S.  fp32 problems: fp32 (batch, nheads,
 *       nchunks, headdim, dstate).  bf16 problems: per (batch, head, chunk) a
 *       hi plane then a lo plane of (headdim, dstate) bf16 with hi = bf16(h_c),
 *       lo = bf16(h_c - hi); always a region of its own.
 *   CB  bf16 problems with headdim 64 and dstate 128, or dstate 256 at chunk
 *       256, only (otherwise empty: cb == total): the fp32 products
 *       S_ij = C_i . B_j of each chunk, per (batch, chunk, group) T/32 x
 *       (T/16 + 2) tiles of 64 lanes x 4 floats.
 *       Tile k of row w holds the 16 x 16 block (I, J) with I = w, J = k when
 *       k < b = (w + 2) & ~1, else I = T/16 - 1 - w, J = k - b; lane
 *       l = 16 q + m, element r holds S_ij for i = 16 I + m, j = 16 J + 4 q + r
 *       (chunk-local token indices; rows past seqlen count as zero).  Blocks
 *       with J > I are zero. */
typedef struct {
    size_t g2_hi, g2_lo, dt, w, s, h, cb, total;
    int64_t nchunks, padded_len;
} ssd_workspace_layout;

/* Workspace bytes for this problem; 0 when the shape or chunk size is invalid
 * or unsupported. */
size_t ssd_chunk_scan_fwd_workspace_size(const ssd_shape *shape, int64_t chunk_size);

/* Fill *layout for this problem (host only, no device access). */
ssd_status ssd_chunk_scan_fwd_workspace_layout(const ssd_shape *shape, int64_t chunk_size,
                                               ssd_workspace_layout *layout);

/* The forward pass.
 *   x, dt, B, C      inputs (dtype), 16-byte aligned (dt: element aligned)
 *   A                fp32 (nheads), required
 *   D                fp32 (nheads), NULL => no skip term
 *   chunk_size       T: 64, 128 or 256
 *   initial_states   fp32 or NULL => zero state; may alias final_states
 *   y                output (y_dtype), 16-byte aligned; must not overlap any input
 *   final_states     fp32 output or NULL => not written; the state after the
 *                    last token
 *   workspace        device scratch of at least
 *                    ssd_chunk_scan_fwd_workspace_size(shape, chunk_size)
 *                    bytes, 256-byte aligned; its contents on entry are
 *                    ignored and on return hold the intermediates described by
 *                    ssd_workspace_layout
 *   stream           hipStream_t or NULL
 * The four stages run in stream order: chunk cumsum, chunk state, state
 * passing, chunk output, one kernel each (ssd_chunk_scan_fwd_stage_launches
 * says which stages launch a kernel for a given problem). */
ssd_status ssd_chunk_scan_fwd(const ssd_shape *shape,
                              const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              int64_t chunk_size, const float *initial_states,
                              void *y, float *final_states,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Same as ssd_chunk_scan_fwd; in addition times every kernel: stage_events
 * holds 8 valid hipEvent_t, a (start, stop) pair per stage in stream order
 * (chunk cumsum, chunk state, state passing, chunk output).  Each pair is
 * recorded by the kernel's own dispatch (hipExtLaunchKernel), so the elapsed
 * time between them is that kernel alone.  A stage that has nothing to do
 * (no chunks) records both of its events back to back. */
ssd_status ssd_chunk_scan_fwd_profiled(const ssd_shape *shape,
                                       const void *x, const void *dt, const float *A,
                                       const void *B, const void *C, const float *D,
                                       int64_t chunk_size, const float *initial_states,
                                       void *y, float *final_states,
                                       void *workspace, size_t workspace_bytes, void *stream,
                                       void *const *stage_events);

/* Launch plan: how the stages divide their work among thread blocks.  Every
 * plan computes the same result (up to summation order); plans differ only in
 * speed.  ssd_chunk_scan_fwd uses the plan ssd_chunk_scan_fwd_default_plan
 * returns; ssd_chunk_scan_fwd_ex accepts any valid plan, for instance one
 * chosen by ssd_chunk_scan_fwd_tune.  A plan is plain data owned by the
 * caller; the library keeps none. */
typedef enum {
    SSD_STATE_SPLIT = 0, /* the chunk states s_c in one fully parallel launch, then
                            the sequential carry across chunks in a second */
    SSD_STATE_FUSED = 1  /* one launch walks the chunks of each (batch, head,
                            dstate tile) in order, forming s_c and carrying the
                            state in registers ("Kernel 2: fwd_pass_state");
                            s_c is never written to the workspace */
} ssd_state_path;

typedef struct {
    int32_t state_path;        /* ssd_state_path */
    int32_t chunk_state_heads; /* split path: heads of one group per chunk-state
                                  block, 1 .. nheads / ngroups */
    int32_t chunk_out_heads;   /* heads of one group per chunk-output block,
                                  1 .. nheads / ngroups */
    int32_t fused_cols;        /* fused path: dstate columns per block (a
                                  multiple of 32 that divides dstate, or dstate);
                                  ignored by the split path */
    int32_t reserved[4];       /* must be 0 */
} ssd_plan;

/* The plan ssd_chunk_scan_fwd uses for this problem (host only: a static
 * model of the launch, no device access). */
ssd_status ssd_chunk_scan_fwd_default_plan(const ssd_shape *shape, int64_t chunk_size,
                                           ssd_plan *plan);

/* ssd_chunk_scan_fwd with an explicit plan (NULL: the default plan) and
 * optional stage events (NULL: none; else as ssd_chunk_scan_fwd_profiled).
 * Returns SSD_ERROR_INVALID_VALUE for a plan whose fields are out of range and
 * SSD_ERROR_UNSUPPORTED for a state path this problem has no kernel for
 * (the fused path needs bf16 inputs). */
ssd_status ssd_chunk_scan_fwd_ex(const ssd_shape *shape,
                                 const void *x, const void *dt, const float *A,
                                 const void *B, const void *C, const float *D,
                                 int64_t chunk_size, const float *initial_states,
                                 void *y, float *final_states,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const ssd_plan *plan, void *const *stage_events);

/* Per-shape autotuner ("Kernel shorts: Mamba-2 in cuTile, CompileIQ + Helion,
 * Deepgram on Trainium2", TL;DR: per-shape tuning of the kernels' tile
 * configurations).  Runs the caller's problem (same arguments and rules as
 * ssd_chunk_scan_fwd; initial_states must not alias final_states here) under
 * candidate plans on `stream` -- heads per block of the chunk-output launch,
 * then the state path: split with each chunk-state heads per block, fused
 * with 32 and 64 dstate columns where supported -- each once untimed and
 * `reps` times (1..1000) with stage events, and writes the plan with the
 * smallest median time to *best (and that time in microseconds, summed over
 * the stages, to *best_us unless it is NULL).  Synchronizes `stream` after
 * each timed run.  On return y and final_states hold the forward pass's
 * result (computed under *best).  Creates and destroys its own events; the
 * plan is plain data the caller keeps and passes to ssd_chunk_scan_fwd_ex. */
ssd_status ssd_chunk_scan_fwd_tune(const ssd_shape *shape,
                                   const void *x, const void *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   int64_t chunk_size, const float *initial_states,
                                   void *y, float *final_states,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   int reps, ssd_plan *best, float *best_us);

/* Which stages launch a kernel of their own for this problem (host only):
 * bit i of *mask is set for stage i (0 chunk cumsum, 1 chunk state, 2 state
 * passing, 3 chunk output).  Stages 0, 1 and 3 are clear when there are no
 * tokens (only the state passing runs: final state = initial state), and
 * every bit is clear for an empty batch.  Under a plan with the fused state
 * path (plan NULL: the default plan) stage 1 is that fused launch and stage 2
 * launches nothing.  A stage that launches nothing records its two profiling
 * events back to back.
 * Returns SSD_ERROR_INVALID_VALUE for a NULL mask or an invalid plan, else
 * what the shape check of ssd_chunk_scan_fwd returns. */
ssd_status ssd_chunk_scan_fwd_stage_launches(const ssd_shape *shape, int64_t chunk_size,
                                             const ssd_plan *plan, uint32_t *mask);

/* One step of the recurrence for one new token per sequence, with the state
 * kept by the caller between calls ("Accelerating Mamba-2 with
 * High-Performance Forward Pass Kernels in NVIDIA CUDA Tile", section
 * "Mamba-2 architecture": the recurrent form, suited to sequential
 * inference).  For every batch b and head h, with g = h / (nheads / ngroups):
 *     state[b,h] <- exp(A[h] dt[b,h]) state[b,h] + dt[b,h] x[b,h] B[b,g]^T
 *     y[b,h]      = state[b,h] C[b,g] + D[h] x[b,h]        (readout after the update)
 * with the state in the (headdim, dstate) orientation of initial_states.
 *   shape            seqlen must be 1; flags must be 0; other fields as for
 *                    ssd_chunk_scan_fwd (headdim 32/64/128, dstate a multiple
 *                    of 16 up to 256, dtype of x/dt/B/C, y_dtype of y)
 *   x                (batch, nheads, headdim)  dtype
 *   dt               (batch, nheads)           dtype, >= 0
 *   A, D             (nheads) fp32; D NULL => no skip term
 *   B, C             (batch, ngroups, dstate)  dtype, 16-byte aligned
 *   state            (batch, nheads, headdim, dstate) fp32, 16-byte aligned,
 *                    read and updated in place
 *   y                (batch, nheads, headdim)  y_dtype, out
 *   stream           hipStream_t or NULL
 *   events           NULL, or 2 valid hipEvent_t recorded by the kernel's own
 *                    dispatch (start, stop)
 * These are the layouts of ssd_chunk_scan_fwd with seqlen 1.  y must not
 * overlap any input or the state, and the state must not overlap an input.
 * All checks happen before the launch; on error nothing is enqueued and
 * state and y are untouched. */
ssd_status ssd_decode_step(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                           const void *B, const void *C, const float *D, float *state, void *y,
                           void *stream, void *const *events);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * pass of ssd_chunk_scan_fwd (default plan) with no workspace argument.  The
 * workspace is a device array of SSD_NOALLOC_SCRATCH_BYTES inside the library
 * (each GPU the library runs on holds its own copy from the first call on it
 * until the process ends); this call allocates nothing.  The caller still
 * owns and passes every input and output, with the conventions and checks of
 * ssd_chunk_scan_fwd.  Problems whose workspace
 * (ssd_chunk_scan_fwd_workspace_size) exceeds the scratch are rejected with
 * SSD_ERROR_SCRATCH before anything is enqueued; shape->flags must be 0.
 * All calls on one GPU share its scratch, and the scratch keeps the last
 * call's contents (nothing in it needs clearing: the stages overwrite what
 * they read): calls that overlap in time on one GPU -- from two streams or
 * two threads -- race and give undefined results.  This entry point is the
 * one exception to "no mutable global state". */
#define SSD_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_shape *shape,
                                      const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      int64_t chunk_size, const float *initial_states,
                                      void *y, float *final_states, void *stream);

/* Backward pass: the gradients of a scalar loss L through ssd_chunk_scan_fwd.
 *
 * The pages name the backward pass as what training depends on
 * ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
 * CUDA Tile", section "Mamba-2 architecture": the chunked form serves
 * training and prefill) and derive none.  This computes the chain rule through
 * the recurrence of that section, h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T,
 * y_t = C_t^T h_t + D x_t, given dy = dL/dy and dL/dh_final, evaluated chunk
 * by chunk: the chunk-start states are recomputed from the inputs (nothing of
 * the forward call is kept), the gradient of the state is carried across the
 * chunks in reverse, and per chunk the gradients take the form of the forward
 * chunk output with the operands' roles exchanged (MFMA kernels).
 *
 *   shape, x, dt, A, B, C, D, chunk_size, initial_states
 *                    exactly as passed to ssd_chunk_scan_fwd (same layouts,
 *                    dtypes and supported sizes); flags must be 0, y_dtype
 *                    plays no part
 *   dy               dL/dy, (batch, seqlen, nheads, headdim) in dtype
 *   d_final_states   dL/dh_final, (batch, nheads, headdim, dstate) fp32;
 *                    NULL => 0
 * Outputs, all fp32 and written (not accumulated):
 *   dx               (batch, seqlen, nheads, headdim)
 *   ddt              (batch, seqlen, nheads)
 *   dA               (nheads)             summed over batch and tokens
 *   dB, dC           (batch, seqlen, ngroups, dstate), summed over the heads
 *                    of each group
 *   dD               (nheads) or NULL => not written (computed as if D were
 *                    given when D is NULL, i.e. the gradient at D = 0)
 *   d_initial_states (batch, nheads, headdim, dstate) or NULL => not written
 * Pointers: x, B, C, dy, the state tensors, dx, dB, dC 16-byte aligned;
 * the workspace 256-byte aligned and at least
 * ssd_chunk_scan_bwd_workspace_size bytes.  No output may overlap an input,
 * the workspace or another output.  All checks happen before the first
 * launch; on error nothing is enqueued and the outputs are untouched.  The
 * call enqueues on `stream` and does not synchronise.  The result is
 * deterministic (fixed reduction orders, no atomics). */
size_t ssd_chunk_scan_bwd_workspace_size(const ssd_shape *shape, int64_t chunk_size);
ssd_status ssd_chunk_scan_bwd(const ssd_shape *shape,
                              const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              int64_t chunk_size, const float *initial_states,
                              const void *dy, const float *d_final_states,
                              float *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                              float *d_initial_states,
                              void *workspace, size_t workspace_bytes, void *stream);
/* As ssd_chunk_scan_bwd, with 2 * SSD_BWD_STAGES valid hipEvent_t recorded
 * by the stages' own dispatches (start, stop per stage), stages in order:
 * 0 cumsum, 1 chunk states, 2 state passing (the recomputed forward states),
 * 3 adjoint chunk terms, 4 reverse carry, 5 score tiles (the B . C tiles
 * of each group; for fp32 inputs also each head's decayed x . dy tiles, the
 * stage's two events then spanning two launches), 6 dx pass, 7 dB
 * pass, 8 dC pass, 9 the sums of the decay-gradient matrix, 10 per-token
 * finish (ddt), 11 reductions (dB, dC, dA, dD).  A stage with nothing to do
 * records both its events back to back. */
#define SSD_BWD_STAGES 12
ssd_status ssd_chunk_scan_bwd_profiled(const ssd_shape *shape,
                                       const void *x, const void *dt, const float *A,
                                       const void *B, const void *C, const float *D,
                                       int64_t chunk_size, const float *initial_states,
                                       const void *dy, const float *d_final_states,
                                       float *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                                       float *d_initial_states,
                                       void *workspace, size_t workspace_bytes, void *stream,
                                       void *const *stage_events);
/* As ssd_chunk_scan_bwd, reusing the chunk-start states h_c of a forward
 * call instead of recomputing them (the same gradients of the same section
 * of the pages; stages 1 and 2 launch nothing).
 *   fwd_workspace        the workspace of a forward call (an
 *                        ssd_chunk_scan_fwd entry point that takes the
 *                        caller's workspace, any plan) made on
 *                        the same x, dt, A, B, initial_states and chunk size,
 *                        with SSD_FLAG_KEEP_INTERMEDIATES in its shape's
 *                        flags, and not written since; 256-byte aligned.  Its
 *                        H region (ssd_chunk_scan_fwd_workspace_layout of
 *                        that shape) is read, nothing in it is written, and
 *                        it must not overlap an output or `workspace`.
 *                        NULL => SSD_ERROR_INVALID_VALUE.
 *   fwd_workspace_bytes  at least that layout's total, else
 *                        SSD_ERROR_WORKSPACE.
 *   stage_events         NULL, or 2 * SSD_BWD_STAGES events as in
 *                        ssd_chunk_scan_bwd_profiled (stages 1 and 2 record
 *                        their pairs back to back).
 * Everything else as ssd_chunk_scan_bwd, whose workspace it still takes.  The
 * library cannot check that fwd_workspace belongs to these inputs: states of
 * other inputs give the gradients of that other forward pass's states. */
ssd_status ssd_chunk_scan_bwd_saved(const ssd_shape *shape,
                                    const void *x, const void *dt, const float *A,
                                    const void *B, const void *C, const float *D,
                                    int64_t chunk_size, const float *initial_states,
                                    const void *dy, const float *d_final_states,
                                    const void *fwd_workspace, size_t fwd_workspace_bytes,
                                    float *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                                    float *d_initial_states,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *stage_events);

/* Static, human-readable description of a status code. */
const char *ssd_status_string(ssd_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */

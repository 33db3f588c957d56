/*
 * gdn.h -- C ABI of the gated-delta-rule (Gated DeltaNet) layer core for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  "Optimizing on-device inference for Apple Silicon" (Perplexity),
 * section "Qwen creates three distinct workload shapes", describes the Gated DeltaNet
 * layer: it packs past context into a fixed-size recurrent state, a learned gate sets
 * how much of the existing state is kept, a delta update writes in the current token,
 * and each token depends on the state the previous token left.  Per batch b and value
 * head h (which reads query/key head h / (Hv / Hk)), with the state S a dv x dk matrix:
 *
 *     a_t = exp(g_t)
 *     S_t = a_t * S_{t-1} * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S_t * q_t
 *
 * The same section says a prefill can evaluate this either by scanning tokens while
 * carrying the state, or by regrouping the updates into blocks that expose matrix
 * operations and token-level parallelism; gdn_prefill does the latter.  gdn_decode_step
 * is the one-token update used while generating ("Decode: minimise bytes moved per
 * token"; the fused "recurrent update" of "Reduce intermediate and state traffic").
 * Section "Keep the recurrent state on chip" fixes the precision: the state and the
 * gate are fp32, query/key activations bf16.  Section "Bound temporary memory with
 * prompt chunking" fixes the hand-off: a prompt split into segments that carry the
 * recurrent state gives the same output -- pass one call's state_out as the next
 * call's state_in.
 *
 * Conventions for every entry point
 *   - All tensor pointers are HIP DEVICE pointers owned by the caller; the library never
 *     allocates, frees or retains them.  Tensors are dense, contiguous, row-major.
 *   - q, k, v and o hold elements of type `dtype` (bf16 = 2-byte bfloat16, f32 = float);
 *     g, beta and the state are always float (fp32).
 *   - q, k, v, o, state pointers must be 16-byte aligned; g, beta 4-byte aligned.
 *   - No query scaling is applied.  gdn_prefill and gdn_decode_step use q, k as given;
 *     their _qknorm variants L2-normalise q and k first.  g must be finite (a_t > 0).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work on
 *     it and return without synchronising; argument errors are reported synchronously,
 *     before anything is enqueued.  Asynchronous kernel faults surface on the stream.
 *   - Shapes supported: dk, dv in {32, 64, 128}; Hk >= 1; Hv a multiple of Hk; B >= 1;
 *     chunk in {16, 32, 64}; any T >= 0 (a final chunk shorter than `chunk` is exact).
 *   - Thread safety: the only global state is a per-device cache of an occupancy query and
 *     of the scratch array's address (gdn_prefill_noalloc), each filled idempotently on first
 *     use; concurrent calls on different streams with disjoint buffers are safe, except
 *     overlapping gdn_prefill_noalloc calls on one GPU (see there).
 *   - Return value: a gdn_status; GDN_OK (0) on success.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                                  */
    GDN_ERR_SHAPE = 2,       /* a size is negative / zero where it may not be, or Hv % Hk != 0 */
    GDN_ERR_UNSUPPORTED = 3, /* dk, dv, chunk or dtype outside the supported set            */
    GDN_ERR_ALIGN = 4,       /* a pointer violates the alignment rules above                */
    GDN_ERR_ALIAS = 5,       /* an output overlaps another argument (state_out == state_in is allowed) */
    GDN_ERR_WORKSPACE = 6,   /* workspace NULL, or too small (see gdn_prefill)              */
    GDN_ERR_HIP = 7          /* the HIP runtime reported an error while enqueueing          */
} gdn_status;

/* Bytes of device workspace gdn_prefill needs to run these sizes in one pass (0 when
 * T == 0).  Returns 0 also for unsupported arguments (gdn_prefill then reports the reason).
 * The workspace holds the per-chunk blocks of the blockwise form between its two kernels;
 * its content on entry is irrelevant and on exit unspecified.  It grows linearly with B * T
 * (about 81 MiB at B = 1, T = 4096, Hk = 16, Hv = 32, dk = dv = 128, bf16). */
size_t gdn_prefill_workspace_bytes(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                   gdn_dtype dtype);

/* Blockwise (chunked) prefill over T tokens.
 *   q, k       [B, T, Hk, dk] dtype      v  [B, T, Hv, dv] dtype
 *   g, beta    [B, T, Hv] float          (log-gate, finite; update strength)
 *   state_in   [B, Hv, dv, dk] float, or NULL for a zero starting state
 *   o          [B, T, Hv, dv] dtype      (o_t = S_t q_t, the post-update state read with q_t)
 *   state_out  [B, Hv, dv, dk] float     (state after token T-1; may equal state_in, which
 *                                         is then updated in place)
 *   workspace  device buffer, 256-byte aligned; may be NULL only when T == 0.
 *              gdn_prefill_workspace_bytes(...) bytes hold the whole prompt.  The prompt
 *              runs in consecutive passes of whole chunks, of equal length, with the state
 *              carried from one to the next through state_out ("Optimizing on-device
 *              inference for Apple Silicon", section "Bound temporary memory with prompt
 *              chunking": segmenting a prompt and carrying the recurrent state leaves the
 *              output unchanged), when the workspace is smaller (it bounds the temporary
 *              memory) or when one pass's workspace and v rows would exceed the last-level
 *              cache (about 176 MB for bf16 operands, 600 MB for fp32; passes that stay in it
 *              run faster).  The result equals the one-pass result bit for bit.
 *              GDN_ERR_WORKSPACE if not even one chunk fits.
 * T == 0 copies state_in (or zeros) to state_out and touches nothing else.
 * Outputs must not overlap each other, the inputs or the workspace, except
 * state_out == state_in exactly. */
gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *state_in, void *o, float *state_out,
                       int B, int T, int Hk, int Hv, int dk, int dv, int chunk, gdn_dtype dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/* gdn_prefill with q and k L2-normalised per token and head inside the kernels: every
 * q_t and k_t above is replaced by x / sqrt(|x|^2 + 1e-6), computed in fp32 from the stored
 * elements, so that raw projections need no separate normalisation pass ("Optimizing
 * on-device inference for Apple Silicon", section "Reduce intermediate and state traffic":
 * the query/key preparation is fused rather than written out and read back).  The stored
 * q and k are not modified.  Arguments, workspace (size and segmentation), aliasing rules
 * and status codes are those of gdn_prefill. */
gdn_status gdn_prefill_qknorm(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *state_in, void *o,
                              float *state_out, int B, int T, int Hk, int Hv, int dk, int dv,
                              int chunk, gdn_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Flags of gdn_prefill_ex (bitwise or). */
#define GDN_QK_NORM 1u         /* L2-normalise q and k inside, as gdn_prefill_qknorm         */
#define GDN_PATH_SEQUENTIAL 2u /* token-sequential scan, state in registers (see below)     */
#define GDN_PATH_AUTO 4u       /* the decode step for T == 1 from a given state, else the
                                  sequential form when T <= gdn_prefill_sequential_max_tokens(),
                                  blockwise otherwise                                        */

/* Prefill with a choice of evaluation form ("Optimizing on-device inference for Apple
 * Silicon", section "Qwen creates three distinct workload shapes": the tokens can be scanned
 * directly while carrying the state, or the updates regrouped into blocks; which is faster
 * depends on the dimensions, the workload and the hardware).
 *   flags without a path bit: the blockwise form, exactly gdn_prefill (or gdn_prefill_qknorm
 *     with GDN_QK_NORM).
 *   GDN_PATH_SEQUENTIAL: the form of section "Keep the recurrent state on chip" -- each
 *     state row split over a few lanes, held in registers for all T tokens, reduced across
 *     lanes per token, written once at the end; one launch, fp32 throughout.  The workspace
 *     is not used (it may be NULL; when given it still takes part in the overlap checks).
 *   GDN_PATH_AUTO: for T == 1 with a start state, the decode step (gdn_decode_step or its
 *     _qknorm form: one read and one write of the state); otherwise the sequential form for
 *     T <= gdn_prefill_sequential_max_tokens(...), else the blockwise form.
 * Arguments, aliasing rules and status codes as gdn_prefill; chunk is validated whatever
 * the path.  GDN_ERR_UNSUPPORTED for unknown flag bits or both path bits. */
gdn_status gdn_prefill_ex(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *state_in, void *o, float *state_out,
                          int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                          gdn_dtype dtype, void *workspace, size_t workspace_bytes, void *stream,
                          unsigned flags);

/* Longest prompt for which GDN_PATH_AUTO picks the sequential form at these sizes: the
 * crossover of the two forms measured on MI355X, by operand type and head size (bf16: 43, 42,
 * 42 tokens at dk = dv = 32, 64, 128; fp32: 89, 96, 110), lowered when batch x value heads x
 * rows exceed what the sequential form runs in one wave per SIMD.  0 for unsupported sizes. */
int gdn_prefill_sequential_max_tokens(int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype);

/* The two stages of gdn_prefill, for callers that schedule them separately (for example
 * to overlap the state-independent stage of one segment with other work, or to time each
 * stage).  Same arguments and rules as gdn_prefill, except that they need the one-pass
 * workspace (gdn_prefill_workspace_bytes); gdn_prefill == prepare then scan on one stream
 * with one workspace.
 *   gdn_prefill_prepare: the state-independent per-chunk blocks (decay-masked Gram and its
 *     unit-triangular inverse, folded with the gates and beta into the blocks that update
 *     the state and form the output from the chunk's residual v - decayed prediction; k
 *     and q rearranged for the scan), written to the workspace.  Reads q, k, g, beta, and
 *     v only to bring it into the cache for the scan; ignores state_in, o and state_out
 *     (they still take part in the overlap checks).
 *   gdn_prefill_scan: carries the state across the chunks in order and writes o and
 *     state_out.  Reads state_in, v and what gdn_prefill_prepare left in the workspace
 *     for the same q, k, v, g, beta and sizes; the workspace must not be modified in
 *     between.  T == 0: state copy, as gdn_prefill. */
gdn_status gdn_prefill_prepare(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *state_in, void *o,
                               float *state_out, int B, int T, int Hk, int Hv, int dk, int dv,
                               int chunk, gdn_dtype dtype, void *workspace,
                               size_t workspace_bytes, void *stream);
gdn_status gdn_prefill_scan(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *state_in, void *o, float *state_out,
                            int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                            gdn_dtype dtype, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Size of the device array gdn_prefill_noalloc uses as its workspace (one per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdn_prefill for callers that cannot allocate device memory: code under HIP-graph capture,
 * tight serving loops, and harnesses that forbid hipMalloc.  Arguments, results, aliasing
 * rules and status codes are those of gdn_prefill, without the workspace: the blocks between
 * the two kernels go to a device array of GDN_NOALLOC_SCRATCH_BYTES inside the library, one
 * copy per GPU, held until the process ends.  Nothing is allocated or freed, by this call or
 * by the library.  A prompt whose one-pass workspace (gdn_prefill_workspace_bytes) exceeds the
 * array runs in segments of whole chunks, exactly as gdn_prefill with a smaller workspace, so
 * the result equals gdn_prefill's bit for bit.  GDN_ERR_WORKSPACE when even one chunk's blocks
 * do not fit (B * Hv too large at these head sizes); GDN_ERR_HIP if the array's device address
 * cannot be obtained (taken once per device, on the first call with that device current).
 * The array keeps the last call's contents, none of which a later call relies on (every
 * value the second kernel reads is written by the first in the same call).  All calls on one
 * GPU share the array: calls that overlap in time on that GPU (on different streams, or from
 * different host threads onto different streams) race and must be serialised by the caller;
 * calls in order on one stream are safe. */
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *state_in, void *o,
                               float *state_out, int B, int T, int Hk, int Hv, int dk, int dv,
                               int chunk, gdn_dtype dtype, void *stream);

/* One-token recurrent update (decode step), in place or out of place.
 *   q, k       [B, Hk, dk] dtype         v  [B, Hv, dv] dtype
 *   g, beta    [B, Hv] float
 *   state_in   [B, Hv, dv, dk] float (required)
 *   state_out  [B, Hv, dv, dk] float; may equal state_in (in-place update)
 *   o          [B, Hv, dv] dtype
 * Each state element is read once and written once; independent layers can be batched
 * through B when their states are laid out back to back. */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *state_in, float *state_out, void *o,
                           int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype, void *stream);

/* gdn_decode_step with q and k L2-normalised in registers first (x / sqrt(|x|^2 + 1e-6),
 * fp32), the decode-side fusion of the same section as gdn_prefill_qknorm.  Arguments and
 * status codes are those of gdn_decode_step. */
gdn_status gdn_decode_step_qknorm(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *state_in, float *state_out,
                                  void *o, int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype,
                                  void *stream);

/* One layer's tensors for gdn_decode_step_layers: exactly the arguments of gdn_decode_step.
 *   q, k [B, Hk, dk] dtype; v, o [B, Hv, dv] dtype; g, beta [B, Hv] float;
 *   state_in, state_out [B, Hv, dv, dk] float (state_out may equal state_in). */
typedef struct {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;
    float *state_out;
    void *o;
} gdn_decode_layer;

/* One decode token through nlayers independent layers whose tensors live anywhere in memory
 * ("Optimizing on-device inference for Apple Silicon", section "Overlap independent GPU work":
 * independent work of a decode step is dispatched together rather than one dependent stage
 * after another).  The same step as gdn_decode_step on every layer, with the same arguments
 * per layer (layers[l], a HOST array read during the call), the sizes and dtype shared; the
 * results are those of nlayers gdn_decode_step calls, bit for bit.  The pointer table travels
 * in the kernel arguments: one launch per 32 layers, no device memory used or allocated, and
 * the call may be captured in a HIP graph.  flags: 0 or GDN_QK_NORM (as
 * gdn_decode_step_qknorm).  Besides gdn_decode_step's checks on each layer: GDN_ERR_NULL if
 * layers is NULL, GDN_ERR_SHAPE if nlayers < 1, GDN_ERR_UNSUPPORTED for other flag bits, and
 * GDN_ERR_ALIAS if an output of one layer overlaps any tensor of another (the layers run
 * concurrently). */
gdn_status gdn_decode_step_layers(const gdn_decode_layer *layers, int nlayers, int B, int Hk,
                                  int Hv, int dk, int dv, gdn_dtype dtype, unsigned flags,
                                  void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

/*
 * titans_mem.h -- C ABI of the MI355X (gfx950) Titans neural long-term memory.
 *
 * One call runs the memory's whole hot path over a batch of independent
 * (batch, head) streams: the chunked test-time update and per-token retrieval
 * of "Titans: Learning to Memorize at Test Time" (mer.dev notes):
 *
 *   loss      l(M; x_t) = ||M(k_t) - v_t||^2          section 3.1, "Objective"
 *   surprise  S_t = eta_t S_{t-1} - theta_t grad l    section 3.1, "Learning
 *                                                      Process and Surprise Metric"
 *   write     M_t = (1 - alpha_t) M_{t-1} + S_t        section 3.1, "Forgetting
 *                                                      Mechanism"
 *   read      y_t = M*(q_t), no weight change          section 3.1, "Retrieving
 *                                                      a Memory"
 *   chunking  gradients of a chunk of b tokens taken at the chunk-start
 *             weights M_{t'}                           section 3.2, "How to
 *                                                      Parallelize ..."
 *
 * The memory M is a matrix W (n_layers == 1, M(k) = W k) or a bias-free MLP
 * (n_layers >= 2) d -> hidden -> ... -> hidden -> d with SiLU after every
 * layer but the last (section 3.1 "Memory Architecture"; block details in
 * section 4.4 use SiLU).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are contiguous and row-major.  Streams are indexed
 *   s = b * H + h.  Token rows are [N, d] per stream.
 * - Parameter layout per stream: layers 1..L concatenated, layer l stored
 *   row-major as [n_l x n_{l-1}] (column-vector convention M(k) = W k); S
 *   has the same layout.  P = sum_l n_l n_{l-1} (titans_mem_param_count).
 * - The gradient used is (M(k) - v) dM/dW, i.e. the gradient of
 *   0.5 ||M(k) - v||^2, the scale section 3.2 prints for the linear case.
 *   Pass 2*theta for the gradient of ||.||^2 itself (theta enters linearly).
 * - Tokens are 0-indexed; chunk c covers [c*chunk, min((c+1)*chunk, N)) and
 *   differentiates at the state left by the previous chunk.  N need not be
 *   a multiple of chunk: the last chunk is shorter.
 * - Gates are not range-checked; non-finite values propagate.
 * - Device pointers must be 16-byte aligned.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream): they return after enqueueing and never synchronise.  Argument
 *   errors (codes -1..-4) are detected on the host before anything is
 *   enqueued, so they can be tested without a GPU.
 * - The library allocates no device memory at run time; the caller owns
 *   every buffer.  (The scratch of titans_mem_forward_noalloc is a device
 *   array of the library's code object, present once per GPU from load.)
 * - Process-wide state: per device, one HIP stream of the library's own
 *   (default priority) and six events, created on the first call that needs
 *   them and kept until the process ends.  The shape-generic forward (when
 *   the state does not fit on chip) and the backward run part of their work
 *   there, forked from and joined back into the caller's `stream` with
 *   events, on every return path; a mutex serialises the enqueueing of such
 *   calls.  Calls are thread-safe.
 */
#ifndef TITANS_MEM_H
#define TITANS_MEM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TITANS_MEM_ABI_VERSION 1

/* status codes */
#define TM_OK               0
#define TM_ERR_INVALID     -1  /* null pointer, dimension <= 0, chunk <= 0, misaligned pointer, bad enum, wrong abi_version */
#define TM_ERR_UNSUPPORTED -2  /* shape / dtype / flag combination the library has no kernel for */
#define TM_ERR_WORKSPACE   -3  /* workspace smaller than titans_mem_workspace_bytes() */
#define TM_ERR_ALIAS       -4  /* illegal overlap between buffers */
#define TM_ERR_HIP         -5  /* the HIP runtime reported an error when launching */
#define TM_ERR_GAVE_UP     -6  /* titans_mem_workspace_status: the MFMA kernel's paired
                                  workgroups gave up waiting for each other; the call's
                                  y, W_out and S_out hold NaN */

/* dtype of k, v, q and y (the io tensors); state and gates are always fp32 */
#define TM_IO_F32  0
#define TM_IO_BF16 1

#define TM_ACT_SILU 0

/* which state retrieval reads (section 3.1 "Retrieving a Memory" has no
 * time index; the write-then-read memory view of section 2.1 reads M_t) */
#define TM_READ_AFTER_WRITE 0  /* y_t = M_{W_t}(q_t): the state after token t's write */
#define TM_READ_CHUNK_START 1  /* y_t = M_{W_t'}(q_t): the state at the start of t's chunk */

/* flags */
#define TM_FLAG_FORCE_GENERIC 1u  /* run the shape-generic fp32 kernel even where a specialised one exists */
#define TM_FLAG_CHUNK_GATES   2u  /* alpha, eta, theta hold one value per chunk, [B,H,ceil(N/chunk)],
                                     shared by the chunk's tokens ("Titans: Learning to Memorize at
                                     Test Time", mer.dev notes, section 3.2 "Parameters as the
                                     Function of Chunks": inside a chunk the update is then
                                     time-invariant) */
#define TM_FLAG_NO_WAIT       4u  /* test hook for the failure path of the MFMA kernel: its paired
                                     workgroups give up at their first wait for each other, so the
                                     call ends normally with NaN outputs and the give-up status
                                     (ignored by the other kernels) */

/* kernel paths reported by titans_mem_select_path */
#define TM_PATH_GENERIC_F32   0   /* any shape: fp32 (matrix instructions), state in global memory */
#define TM_PATH_MLP2_D64_H256 1   /* 2-layer, d=64, hidden=256, chunk<=64, bf16 io, either read mode:
                                     MFMA, register-resident state */
#define TM_PATH_DEEP_BF16     2   /* MLP (n_layers >= 2) with d and hidden multiples of 64, chunk<=256,
                                     bf16 io, N >= 1, either read mode: bf16 MFMA products with fp32
                                     sums, fp32 state in W_out/S_out; every step of a chunk one launch
                                     over all streams, the reads on the library's second stream */

typedef struct {
    int32_t abi_version;  /* must equal TITANS_MEM_ABI_VERSION */
    int32_t B, H, N;      /* batch, heads, tokens per stream (N >= 0) */
    int32_t d;            /* key = value = query width */
    int32_t hidden;       /* MLP width; ignored when n_layers == 1 */
    int32_t n_layers;     /* 1 = linear memory W (d x d); >= 2 = MLP */
    int32_t activation;   /* TM_ACT_SILU */
    int32_t io_dtype;     /* TM_IO_F32 or TM_IO_BF16 */
    int32_t read_mode;    /* TM_READ_AFTER_WRITE or TM_READ_CHUNK_START */
    uint32_t flags;       /* TM_FLAG_* */
} titans_mem_desc;

/* ABI version this library was built with. */
int32_t titans_mem_abi_version(void);

/* Parameters per stream (P), or a negative status for an invalid shape. */
int64_t titans_mem_param_count(const titans_mem_desc* desc);

/* Kernel path titans_mem_forward would run for (desc, chunk), or a negative
 * status (TM_ERR_INVALID / TM_ERR_UNSUPPORTED). */
int32_t titans_mem_select_path(const titans_mem_desc* desc, int32_t chunk);

/* Device workspace titans_mem_forward needs for (desc, chunk), in bytes
 * (0 when the selected kernel needs none), or a negative status. */
int64_t titans_mem_workspace_bytes(const titans_mem_desc* desc, int32_t chunk);

/*
 * titans_mem_forward -- chunked update plus retrieval over all B*H streams.
 *
 *   k, v, q    [B,H,N,d]  io dtype, device, read-only
 *   alpha, eta, theta  [B,H,N] fp32, device, read-only: forgetting gate,
 *              surprise decay, momentary-surprise weight
 *              ([B,H,ceil(N/chunk)] with TM_FLAG_CHUNK_GATES)
 *   W_in, S_in [B,H,P]  fp32, device, read-only: memory weights and
 *              surprise momentum before token 0
 *   chunk      b >= 1: tokens per chunk (gradients at the chunk-start state)
 *   y_out      [B,H,N,d]  io dtype, device, written: y_t per token
 *              (computed in fp32, rounded once to nearest-even)
 *   W_out, S_out [B,H,P] fp32, device, written: state after token N-1.
 *              W_out == W_in and/or S_out == S_in (exact in-place) is
 *              allowed; any other overlap among all buffers is TM_ERR_ALIAS.
 *   workspace  device scratch of at least titans_mem_workspace_bytes(desc,
 *              chunk) bytes (may be NULL when that is 0); its contents on
 *              entry do not matter and are undefined on return.
 *   stream     hipStream_t to enqueue on (NULL = default stream).  On the
 *              deep-memory path (TM_PATH_DEEP_BF16), and on the
 *              shape-generic kernel when the state does not fit on chip
 *              and chunk >= 16 (and the call is not in place), part of the
 *              work (the retrieval) runs on a second stream of the
 *              library's own (one per device, default priority), ordered
 *              against `stream` with events and joined back into it before
 *              the call's work ends.
 *
 * Returns TM_OK or a negative status.  Resuming: passing (W_out, S_out) of
 * a call as (W_in, S_in) of the next, with a split on a chunk boundary,
 * continues the same sequence.
 *
 * The MFMA path (TM_PATH_MLP2_D64_H256) runs each stream on two workgroups
 * that wait for each other every chunk.  Both must be resident at once; the
 * launch sizes its grid to half the device's CUs, but work that other
 * streams or processes keep on the CUs can hold one back.  A workgroup whose
 * partner does not arrive within a bounded wait (about 2^21 polls) gives up
 * instead of hanging: the call still completes, y, W_out and S_out of the
 * pair's streams hold NaN, and titans_mem_workspace_status reports
 * TM_ERR_GAVE_UP.
 */
int titans_mem_forward(const titans_mem_desc* desc,
                       const void* k, const void* v, const void* q,
                       const float* alpha, const float* eta, const float* theta,
                       const float* W_in, const float* S_in,
                       int32_t chunk,
                       void* y_out, float* W_out, float* S_out,
                       void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * titans_mem_forward_noalloc -- titans_mem_forward for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, results and asynchrony as titans_mem_forward without the
 * workspace, for the shapes of the MFMA path (TM_PATH_MLP2_D64_H256:
 * 2-layer, d = 64, hidden = 256, bf16 io, chunk <= 64; any B*H, N and read
 * mode); TM_ERR_UNSUPPORTED for every other shape.  Its scratch (the
 * workgroups' tagged exchange and hand-over words and the status word) is a
 * library-owned device array of 42,467,584 bytes (40.5 MiB + 256: enough for
 * the kernel's largest grids, 128 workgroup pairs or, with at most 64
 * streams, 64 groups of four workgroups; TM_ERR_WORKSPACE if a shape ever
 * needed more), one per GPU,
 * allocated with the library's code and held until the process ends.  The
 * call allocates nothing: it enqueues a small fill kernel and the memory
 * kernel on `stream`.  The first call on a device looks up the array's
 * address there.  All calls on one GPU share the array: calls that follow
 * one another on a stream are independent, calls that overlap in time on one
 * GPU (other streams, other threads) race and must not be issued.
 * titans_mem_workspace_status with workspace NULL reports on the last such
 * call on the current device.
 */
int titans_mem_forward_noalloc(const titans_mem_desc* desc,
                               const void* k, const void* v, const void* q,
                               const float* alpha, const float* eta, const float* theta,
                               const float* W_in, const float* S_in,
                               int32_t chunk,
                               void* y_out, float* W_out, float* S_out,
                               void* stream);

/*
 * titans_mem_workspace_status -- outcome of the last titans_mem_forward call
 * that used `workspace` (same desc and chunk).  Waits for `stream` to drain
 * (hipStreamSynchronize) and reads the status word the MFMA kernel keeps in
 * its workspace.
 *
 * Returns TM_OK when the call completed, TM_ERR_GAVE_UP when paired
 * workgroups of the MFMA kernel gave up waiting for each other (its outputs
 * hold NaN), an argument error (-1..-3) like titans_mem_forward's, or
 * TM_ERR_HIP when the copy or the synchronisation fails.  Paths without
 * cross-workgroup waits always report TM_OK.  workspace NULL stands for the
 * scratch of titans_mem_forward_noalloc on the current device.
 */
int titans_mem_workspace_status(const titans_mem_desc* desc, int32_t chunk,
                                const void* workspace, int64_t workspace_bytes,
                                void* stream);

/*
 * titans_mem_retrieve -- pure retrieval y = M*_W(q) at a fixed state
 * (section 3.1 "Retrieving a Memory": a forward pass without weight
 * adjustment), e.g. a lookup after a context has been consumed.
 *
 *   q      [B,H,N,d] io dtype, device
 *   W      [B,H,P]   fp32, device (the state to read)
 *   y_out  [B,H,N,d] io dtype, device, must not overlap q or W
 * Uses desc's shape fields; read_mode is ignored.  The 2-layer d=64
 * hidden=256 bf16 memory runs on the matrix cores (bf16 operands, fp32 sums);
 * every other shape, and any call with TM_FLAG_FORCE_GENERIC, on the
 * shape-generic fp32 kernel (widths up to 1024).
 */
int titans_mem_retrieve(const titans_mem_desc* desc, const void* q, const float* W,
                        void* y_out, void* stream);

/*
 * titans_mem_backward -- gradients through titans_mem_forward, for training
 * what produces the memory's inputs (section 3.1, "Objective": the memory's
 * weights are fitted in an inner loop at test time; the rest of the model
 * learns in an outer loop, through the memory).
 *
 * Returns the vector-Jacobian products of the forward map (same desc,
 * inputs and chunk as the forward call) with the output adjoints:
 *   dy               [B,H,N,d] fp32, device, or NULL (zero): dL/dy
 *   dW_out, dS_out   [B,H,P] fp32, device, or NULL (zero): dL/dW_out, dL/dS_out
 * into
 *   dk, dv, dq       [B,H,N,d] fp32, device, written
 *   dalpha, deta, dtheta  [B,H,N] fp32 ([B,H,ceil(N/chunk)] with
 *                    TM_FLAG_CHUNK_GATES), device, written
 *   dW_in, dS_in     [B,H,P] fp32, device, written
 * The derivative includes the second-order term of the chunk-start
 * gradients (each token's inner gradient depends on W at its chunk start).
 * Both read modes.  Arithmetic is fp32 whatever the io dtype (bf16 inputs
 * are read exactly).  Outputs must not overlap each other or any input.
 * Supported: every layer width a multiple of 4, at most 1024, N >= 1,
 * chunk <= 4096 (TM_ERR_UNSUPPORTED otherwise).
 * The workspace holds (W, S) at every chunk start and two chunks' token
 * vectors: titans_mem_backward_workspace_bytes(desc, chunk) bytes.
 * The work is ordered on `stream`; part of it runs on a second stream of
 * the library's own (one per device, created on the first call, default
 * priority), forked from and joined back into `stream` with events, so
 * work enqueued on `stream` after the call sees every result.
 */
int64_t titans_mem_backward_workspace_bytes(const titans_mem_desc* desc, int32_t chunk);

int titans_mem_backward(const titans_mem_desc* desc,
                        const void* k, const void* v, const void* q,
                        const float* alpha, const float* eta, const float* theta,
                        const float* W_in, const float* S_in, int32_t chunk,
                        const float* dy, const float* dW_out, const float* dS_out,
                        float* dk, float* dv, float* dq,
                        float* dalpha, float* deta, float* dtheta,
                        float* dW_in, float* dS_in,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * titans_mem_input -- the step before the memory: model activations x to
 * the memory's keys, values, queries and gates, for whole sequences.
 *
 * Per sequence b, token t, head h (mer.dev notes):
 *   projections  k = x W_K, v = x W_V      section 3.1, "Objective"
 *                q = x W_Q                 section 3.1, "Retrieving a Memory"
 *   convolution  causal depthwise over time after each projection, width w:
 *                u_t[c] = sum_{j<w} conv_w[c][j] * proj_{t-j}[c], tokens before
 *                the sequence start count as zero   section 4.4, "Convolution"
 *   activation   SiLU on k, v and q; k and q divided by their l2 norm over
 *                the head's d channels (floored at 1e-6)
 *                                          section 4.4, "Architectural Details"
 *   gates        alpha, eta, theta = scale_g * sigmoid(x . w_gate[g][h] +
 *                b_gate[g][h]): per token and head, input dependent
 *                                          section 3.1, "Learning Process and
 *                                          Surprise Metric"
 * There are no projection biases.  Arithmetic: bf16 x bf16 products, fp32
 * sums and epilogue, k, v, q rounded once to bf16 (nearest-even).
 *
 *   x          [B,N,D]     bf16, device, read-only
 *   w_proj     [3,H*d,D]   bf16, device: rows of W_K, then W_V, then W_Q;
 *              channel c of head h is row h*d + c (out = x . row)
 *   conv_w     [3,H*d,w]   fp32, device: tap j weighs the token j steps back
 *   w_gate     [3,H,D]     bf16, device: logit weights of alpha, eta, theta
 *   b_gate     [3,H]       fp32, device: logit biases
 *   *_scale    host scalars multiplying the three sigmoids
 *   k_out, v_out, q_out  [B,H,N,d] bf16, device, written (the layout
 *              titans_mem_forward reads)
 *   alpha_out, eta_out, theta_out  [B,H,N] fp32, device, written
 * Supported: D a positive multiple of 32, d in {16, 32, 64, 128}, H*d a
 * multiple of 128, 1 <= w <= 4 (else TM_ERR_UNSUPPORTED).  Outputs must not
 * overlap each other or any input (TM_ERR_ALIAS).  N == 0 enqueues nothing.
 */
typedef struct {
    int32_t abi_version;  /* must equal TITANS_MEM_ABI_VERSION */
    int32_t B, N;         /* sequences, tokens per sequence (N >= 0) */
    int32_t D;            /* model width */
    int32_t H, d;         /* heads, head width */
    int32_t conv_width;   /* w: causal depthwise taps */
    uint32_t flags;       /* must be 0 */
} titans_input_desc;

int titans_mem_input(const titans_input_desc* desc,
                     const void* x, const void* w_proj, const float* conv_w,
                     const void* w_gate, const float* b_gate,
                     float alpha_scale, float eta_scale, float theta_scale,
                     void* k_out, void* v_out, void* q_out,
                     float* alpha_out, float* eta_out, float* theta_out,
                     void* stream);

/* Static text for a status code. */
const char* titans_mem_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TITANS_MEM_H */

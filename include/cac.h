/* cac.h — C ABI of the cache-aware streaming Conformer chunk step on MI355X (gfx950).
 *
 * What one push computes (per stream, per chunk of n subsampled frames), following
 * "True streaming encode — implementation spec" (fluidaudio-web STREAMING.md), "Per-chunk flow"
 * steps 2-4, with the state of its "State" section:
 *   [optional front end: 3 causal stride-2 k=3 convs over [melTail || 16 new mel frames]]
 *   for each of n_layers Conformer blocks:
 *     x += 1/2 FF1(x); x += MHSA_relpos(LN(x)) against the layer's K/V cache (<= att_left rows)
 *     under the chunked-causal mask on absolute positions; x += ConvModule(x) with the layer's
 *     depthwise cache (dw_kernel-1 columns of GLU output); x += 1/2 FF2(x); x = LN_out(x)
 *   z = x Wj + bj  (the encoder-side joint projection, computed once per frame: "Fast
 *                   Accuracy-Preserving RNNT Beam Search on Apple Silicon", "Delete Repeated
 *                   Projection Work First")
 * The lookahead variant (same spec, "Status", Nemotron bullet) computes n_emit + n_lookahead
 * frames per pass with right context att_right, emits n_emit and caches only those.
 *
 * Conventions
 *   - Every function returns int32: >= 0 on success (a count where stated), < 0 an error code.
 *   - "d_" pointers are device memory (hipMalloc'd by the caller), "h_" pointers host memory.
 *   - All device work is enqueued on the HIP stream given at create time (or by
 *     cac_set_stream); no call synchronises the host except where stated. Outputs are valid
 *     once that stream has been synchronised.
 *   - The context calls never allocate device memory: the caller provides one workspace of
 *     cac_workspace_bytes() bytes that holds the repacked weights, every stream's state and
 *     all activations. The library keeps a pointer to it until cac_destroy. (The test-only
 *     cac_test_gemm is the one exception; it says so below.)
 *   - A call that enqueues device work first checks the context's stream for an asynchronous
 *     error left by earlier work (without waiting for it) and returns CAC_EHIP if there is one.
 *   - Arguments are validated on the host before any device work; on error nothing is
 *     enqueued and the context is unchanged. cac_last_error() then describes the failure.
 *   - One context is used by one host thread at a time; there is no internal locking.
 */
#ifndef CAC_H
#define CAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* error codes */
#define CAC_OK 0
#define CAC_EINVAL (-1)  /* bad config or argument: null pointer, id out of range, duplicate id
                            in one call, n not a multiple of att_chunk, too many frames */
#define CAC_ESTATE (-2)  /* stream state forbids the call: push to a flushed stream (reset it
                            first), state import that does not fit the config (a blob made
                            with another config, a position or pending count out of range) */
#define CAC_ENOMEM (-3)  /* workspace smaller than cac_workspace_bytes() */
#define CAC_EHIP (-4)    /* a HIP runtime call or a kernel launch failed, or an asynchronous
                            device error from earlier work was found on the context's stream */
#define CAC_ENODEV (-5)  /* the context was created with CAC_FLAG_DRY_RUN: no device work */

/* compute dtype of GEMM operands and caches (residual stream, LayerNorm, softmax, GLU and the
   depthwise conv always run in fp32) */
#define CAC_F32 0
#define CAC_BF16 1
/* float32 activations and caches with int8 dense weights: each matrix of the blocks (FF1/FF2
   w1 and w2, wq/wk/wv/wo, pw1, pw2) and the joint is stored as codes q[n][k] with one float32
   scale s[n] per output n, s = max_k |w[k][n]| / 127 and q = rint(w / s) clamped to +-127 (round
   half to even, float32 arithmetic), and computes with q * s. The compression the pages name
   for the weight-bandwidth-bound one-stream case ("Fast Accuracy-Preserving RNNT Beam Search on
   Apple Silicon", §1.3; "True streaming encode — implementation spec", "Status"); an
   approximation of the float32 encoder. No front end, no lookahead, d_model and d_ff multiples
   of 256; a push carries at most 2 rows (streams x frames), else CAC_EINVAL. */
#define CAC_F32_I8 2

/* config flags */
#define CAC_FLAG_DRY_RUN 1 /* host-only context: validation and stream bookkeeping, no device
                              calls (workspace may be NULL); pushes return CAC_ENODEV after
                              validating and updating host bookkeeping */
#define CAC_FLAG_POISON 2  /* reset fills cache slots with NaN instead of 0: a read of any slot
                              that does not hold a valid row shows up as NaN in the outputs */

typedef struct cac_ctx cac_ctx;

typedef struct {
  int32_t n_layers;      /* Conformer blocks (17; the model card's "Config" table) */
  int32_t d_model;       /* D (512), a multiple of 64, <= 1024 */
  int32_t n_heads;       /* H (8); head_dim = D/H must be 16, 32 or 64 */
  int32_t d_ff;          /* F (2048), a multiple of 64 */
  int32_t dw_kernel;     /* depthwise kernel width (9), <= 16; cache of dw_kernel-1 columns */
  int32_t att_left;      /* Lc: left attention context = K/V cache rows (70) */
  int32_t att_chunk;     /* c: attention chunk in frames (2); pushes are multiples of c */
  int32_t att_right;     /* right context of the lookahead variant (3), else 0 */
  int32_t n_emit;        /* frames emitted per pass (lookahead variant), else frames per push */
  int32_t n_lookahead;   /* provisional frames recomputed every pass (8), 0 = exact streaming */
  int32_t joint_dim;     /* P (640); 0 = no joint projection, outputs are the hidden rows */
  int32_t frontend;      /* 1 = inputs are log-mel chunks run through the conv front end;
                            2 = the same inputs through the 2-D time x frequency stack */
  int32_t mel_bins;      /* 128 */
  int32_t mel_per_chunk; /* 16 mel frames -> 2 subsampled frames */
  int32_t mel_tail;      /* 14 */
  int32_t dtype;         /* CAC_F32, CAC_BF16 or CAC_F32_I8 */
  int32_t max_streams;   /* stream ids are 0 .. max_streams-1 */
  int32_t max_push_frames; /* most frames one push may carry (exact variant), <= 16 */
  int32_t flags;         /* CAC_FLAG_* */
  int32_t fe_channels;   /* channels of the 2-D front end (frontend 2: a multiple of 64, <= 512),
                            else ignored */
} cac_config;

/* Number of float parameters cac_create_streams expects, in this order (all float32, host):
 *   for each layer l = 0 .. n_layers-1:
 *     ff1: ln_g[D] ln_b[D] w1[D][F] b1[F] w2[F][D] b2[D]
 *     att: ln_g[D] ln_b[D] wq[D][D] bq[D] wk[D][D] bk[D] wv[D][D] bv[D] wo[D][D] bo[D]
 *          pos_u[H][hd] pos_v[H][hd] wpos[D][D]
 *     conv: ln_g[D] ln_b[D] pw1[D][2D] pw1_b[2D] dw[D][dw_kernel] dw_b[D] pw2[D][D] pw2_b[D]
 *     ff2: ln_g[D] ln_b[D] w1[D][F] b1[F] w2[F][D] b2[D]
 *     out: ln_g[D] ln_b[D]
 *   if joint_dim: joint w[D][P] b[P]
 *   if frontend 1: c1 w[D][mel_bins][3] b[D]; c2 w[D][D][3] b[D]; c3 w[D][D][3] b[D]
 *   if frontend 2 (C = fe_channels, F8 = mel_bins / 8): c1 w[C][3][3] b[C]; dw2 w[C][3][3] b[C];
 *     pw2 w[C][C] ([out][in]) b[C]; dw3 w[C][3][3] b[C]; pw3 w[C][C] b[C];
 *     lin w[C * F8][D] (input index c * F8 + f) b[D]
 * Matrices are [in][out] row-major (y = x W + b); conv weights are [out][in][tap] (2-D:
 * [out][time tap][frequency tap]).
 * The 2-D front end (frontend 2): stage 1 is a 3 x 3 convolution from the mel map to C
 * channels, stages 2 and 3 a depthwise 3 x 3 then a pointwise C x C convolution, each stage
 * stride 2 in time and frequency with ReLU, causal in time exactly like the 1-D front end and
 * padded by one column in frequency; the C x F/8 map of each frame is projected to D by lin.
 * Returns 0 for an invalid config. */
size_t cac_param_count(const cac_config* cfg);

/* Bytes of device workspace a context needs (weights + state of max_streams streams +
 * activations for max_streams * frames-per-pass rows). Returns 0 for an invalid config. */
size_t cac_workspace_bytes(const cac_config* cfg);

/* Floats per stream in the canonical state blob of cac_export_state / cac_import_state:
 *   header[4]  four 32-bit words (not floats): magic 0x53434143, layout version 1 and a 64-bit
 *              hash of the config (cac_state_header); export writes it, import rejects a blob
 *              whose header differs from the context's with CAC_ESTATE
 *   K[n_layers][att_left][D], V[n_layers][att_left][D]   row r = position pos-att_left+r
 *   conv[n_layers][dw_kernel-1][D]                       column j = position pos-(K-1)+j
 *   mel_tail[mel_tail][mel_bins]                         (frontend only)
 *   x0[n_lookahead][D]  pending layer-0 inputs, row j = position pos+j (lookahead only)
 * Rows of positions before 0 are ignored on import and written as 0 on export. */
size_t cac_state_floats(const cac_config* cfg);

/* The 4-word state-blob header of cfg (h_out: 4 uint32, host): magic, version and the 64-bit
 * FNV-1a hash of every config field except max_streams, max_push_frames and flags. Callers
 * that build a state blob themselves put it in front of each stream's floats. Returns CAC_OK,
 * or CAC_EINVAL for an invalid config or a NULL h_out. */
int32_t cac_state_header(const cac_config* cfg, uint32_t* h_out);

/* Validate cfg, repack the float32 host parameters (h_params, cac_param_count floats) into the
 * workspace in the compute layout (bf16 rounding to nearest even for CAC_BF16), compute each
 * layer's projected position table once (streaming spec, "Per-chunk flow" step 3: the
 * projected position rows are a per-layer constant), reset every stream to position 0, and
 * return the context in *out. hip_stream is a
 * hipStream_t (NULL = default stream). Synchronises hip_stream before returning. The caller may
 * free h_params afterwards; d_workspace must stay allocated until cac_destroy. */
int32_t cac_create_streams(const cac_config* cfg, const float* h_params, size_t n_params,
                           void* d_workspace, size_t ws_bytes, void* hip_stream, cac_ctx** out);

/* Push one chunk for n_streams streams (1 <= n_streams <= max_streams; ids in h_stream_ids,
 * distinct, in [0, max_streams)); an empty call (n_streams 0) is CAC_EINVAL and changes nothing.
 *   exact variant: d_input is [n_streams][n_frames][D] (or [n_streams][mel_per_chunk][mel_bins]
 *     log-mel with the front end, n_frames = mel_per_chunk/8), in the compute dtype (float32 or
 *     bf16); n_frames a multiple of att_chunk, <= max_push_frames (front end: exactly 2).
 *     d_out receives [n_streams][n_frames][P] float32 (P = joint_dim, or D without joint).
 *   lookahead variant: n_frames must equal n_emit; the frames join each stream's pending
 *     inputs; streams with n_emit + n_lookahead pending run one pass and emit n_emit frames
 *     into d_out rows [i][0 .. n_emit) ; streams still warming up emit nothing.
 * d_input and d_out must be different buffers.
 * h_emitted (optional, n_streams int32) receives each stream's emitted frame count.
 * Returns the largest per-stream emitted count. Asynchronous (see Conventions). */
int32_t cac_push_chunk(cac_ctx* ctx, int32_t n_streams, const int32_t* h_stream_ids,
                       int32_t n_frames, const void* d_input, float* d_out, int32_t* h_emitted);

/* Return streams to the fresh state (streaming spec, "Engine + mic wiring": reset zeroes the
 * caches, mel tail and position). Returns n. */
int32_t cac_reset_stream(cac_ctx* ctx, int32_t n, const int32_t* h_stream_ids);

/* End streams (streaming spec, "Status": end-of-stream padding happens only at flush). The
 * lookahead variant runs a
 * final pass over each stream's pending frames and writes all of them to d_out
 * ([n][n_lookahead][P], first h_frames_out[i] rows of stream i); the exact variant has nothing
 * left to emit. Flushed streams reject pushes until reset. Returns the largest frame count. */
int32_t cac_flush(cac_ctx* ctx, int32_t n, const int32_t* h_stream_ids, float* d_out,
                  int32_t* h_frames_out);

/* Copy the state of n streams into / from the canonical float32 layout (cac_state_floats per
 * stream, d_state is [n][cac_state_floats] device memory). h_pos: stream positions (frames
 * emitted); h_pending: pending layer-0 inputs of the lookahead variant (ignored otherwise,
 * may be NULL then). Import requires 0 <= pending <= n_lookahead and the context's header in
 * front of every stream's blob; it reads those headers (one small device-to-host copy) and
 * rejects the whole call with CAC_ESTATE, changing nothing, if any differs. A dry-run context
 * reads d_state as host memory. Both calls synchronise the context's stream. */
int32_t cac_export_state(cac_ctx* ctx, int32_t n, const int32_t* h_stream_ids, int32_t* h_pos,
                         int32_t* h_pending, float* d_state);
int32_t cac_import_state(cac_ctx* ctx, int32_t n, const int32_t* h_stream_ids,
                         const int32_t* h_pos, const int32_t* h_pending, const float* d_state);

/* Host view of a stream: position, pending frames, flushed flag (no device access). */
int32_t cac_stream_info(const cac_ctx* ctx, int32_t stream_id, int32_t* pos, int32_t* pending,
                        int32_t* flushed);

/* Pushes are recorded once per call shape (stream count, frames, lookahead passes) into a HIP
 * graph of kernel nodes and replayed; only the nodes holding the caller's input and output
 * pointers are re-pointed between replays. enable = 0 launches every kernel directly (as
 * profiling always does). Default on. */
int32_t cac_set_graph(cac_ctx* ctx, int32_t enable);

/* Change the HIP stream later calls enqueue on. */
int32_t cac_set_stream(cac_ctx* ctx, void* hip_stream);

/* Synchronise the context's stream and report any asynchronous device error (CAC_EHIP). */
int32_t cac_synchronize(cac_ctx* ctx);

/* Per-kernel timing of later pushes and flushes (measurement aid). While on, pushes launch
 * directly (no graph replay) and every kernel is launched with a start and a stop HIP event
 * bound to its own dispatch on the context's stream (hipExtLaunchKernel), so each time is
 * that kernel's execution plus the event markers, without host submission gaps.
 * cac_profile(ctx, 1) clears and starts, 0 stops.
 * cac_profile_read synchronises the recorded events and fills, per kernel name (up to
 * max_entries; names is max_entries * name_len chars): launches, total milliseconds between
 * each launch's events, and the algorithmic bytes and flops the library attributes to those
 * launches (weights read once per launch, K/V and depthwise ring rows read and written,
 * inputs and outputs; activations that stay on chip are not counted). Returns the number of
 * kernel names recorded. */
int32_t cac_profile(cac_ctx* ctx, int32_t enable);
int32_t cac_profile_read(cac_ctx* ctx, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
                         double* total_ms, double* bytes, double* flops);

/* Back-to-back duration of one kernel family (measurement aid). Takes the kernel launches of
 * the most recently replayed push graph whose kernel names start with `prefix` (for example
 * "gemm_tworow_f32"), chains just those launches, in their order and with their arguments,
 * into a graph, replays it `reps` times on the context's stream between two HIP events, and
 * writes the mean time per launch in microseconds to *us_per_launch and the number of
 * launches per replay to *launches, plus their mean algorithmic bytes and flops per launch to
 * *bytes / *flops (any of the four pointers may be NULL). The kernels run on whatever the
 * workspace holds, so the state of the streams of that push is unspecified afterwards: reset
 * or re-import them before pushing them again. Returns CAC_OK, CAC_EINVAL (no recorded push
 * graph, no launch with that prefix, reps < 1) or CAC_EHIP. */
int32_t cac_profile_replay(cac_ctx* ctx, const char* prefix, int32_t reps, double* us_per_launch, int32_t* launches,
                           double* bytes, double* flops);

/* Free the host context (the workspace stays the caller's). Accepts NULL. */
int32_t cac_destroy(cac_ctx* ctx);

/* Description of the last error on ctx; with ctx == NULL, of the last failed
 * cac_create_streams (or test GEMM call) on this thread. Never NULL. */
const char* cac_last_error(const cac_ctx* ctx);

/* Test-only: C[M][N] (float32) = A[M][K] W[N][K]^T + bias through the library's dense kernels
 * (dtype selects bf16 or float32 operands for A and W; bias may be NULL). path: 0 = the
 * library's own choice, 1 = the small-M kernel, 2 = the MFMA tile kernel with its own tile
 * choice, 3..6 = the MFMA tile kernel with 128x128, 128x64, 64x128 or 64x64 block tiles
 * (MFMA paths: bf16 only, K a multiple of 64, N a multiple of 8), 9 / 10 = its 64x64 tile with the k-steps split
 * over 2 / 4 groups of waves in one block (K a multiple of 128 / 256), 11 / 12 = its 128x128 /
 * 128x96 tile over 2 groups (K a multiple of 128), 7 / 8 = the 64x64 MFMA kernel with K split in
 * 2 / 4 ranges whose float32 partials the residual row kernel sums with the bias (K a multiple
 * of 128 / 256, N a multiple of 256 up to 1024; allocates and frees a temporary partial buffer
 * with hipMalloc / hipFree, the one allocation in the library, and returns after the stream has
 * drained). Enqueued on hip_stream; CAC_EINVAL for shapes a path does not take. */
int32_t cac_test_gemm(int32_t dtype, int32_t path, int32_t M, int32_t N, int32_t K,
                      const void* d_A, const void* d_W, const float* d_bias, float* d_C,
                      void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): cac_test_gemm with the same arguments, shapes and
 * results, that calls no hipMalloc, hipFree or other allocating routine and does not
 * synchronise. The split-K paths (7, 8) keep their float32 partials in a device scratch array
 * of the library (4 Mi floats = 16 MiB, one per GPU, held until the process ends): a call whose
 * partials (ranges * M * N floats) do not fit returns CAC_ENOMEM before any device work. The
 * output is cleared by a kernel (no memset node). Every call on one GPU shares that GPU's
 * scratch and each call rewrites what it reads, so calls run one after another on one stream
 * are independent, but calls that overlap in time on one GPU (different streams or threads)
 * race on it. Errors are described by cac_last_error(NULL). */
int32_t cac_test_gemm_noalloc(int32_t dtype, int32_t path, int32_t M, int32_t N, int32_t K,
                              const void* d_A, const void* d_W, const float* d_bias, float* d_C,
                              void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* CAC_H */

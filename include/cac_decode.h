/* cac_decode.h — C ABI of greedy RNNT + EOU decoding on MI355X (gfx950), the consumer of the
 * chunk step's projected encoder frames (cac.h).
 *
 * What one call computes, per stream, over its n_frames new projected encoder frames z
 * ("Parakeet-EOU-120M — Streaming ASR Model", "Decoder" and "Joint"; "Fast Accuracy-Preserving
 * RNNT Beam Search on Apple Silicon", §3.2: the joint after projection; "True streaming
 * encode — implementation spec", "Decoder state carry"):
 *   - prediction network: token embedding, then pred_layers LSTM layers of width pred_hidden
 *     (gate order i, f, g, o), its top output projected to joint_dim once per update;
 *   - joint after projection: logits = ReLU(z + p) Wout + bout over vocab + 2 classes
 *     (tokens 0 .. vocab-1, blank = vocab, EOU = vocab + 1);
 *   - greedy: per frame, argmax (ties to the lowest class); blank moves to the next frame,
 *     any other class is emitted and the predictor advances on it before the same frame is
 *     scored again; after max_symbols emissions at one frame the decoder moves on;
 *   - the stream's LSTM state, projected predictor output and not yet consumed last token are
 *     carried to the next call; a fresh stream starts by predicting from blank.
 * All arithmetic is float32.
 *
 * Conventions as in cac.h: int32 returns (>= 0 success, < 0 error code, CAC_* codes of
 * cac.h), "d_" device pointers, "h_" host pointers, all device work on the stream given at
 * create time, arguments validated on the host before any device work (on error nothing is
 * enqueued and the context is unchanged), one host thread per context at a time. The caller
 * owns all device memory; the decoder calls never allocate device memory.
 */
#ifndef CAC_DECODE_H
#define CAC_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cac_dec cac_dec;

typedef struct {
  int32_t joint_dim;    /* P (640): width of the projected encoder frames and predictor output;
                           a multiple of 64, <= 4096 */
  int32_t pred_hidden;  /* H (640): embedding and LSTM width, a multiple of 64, <= 4096 */
  int32_t pred_layers;  /* LSTM layers (2), 1 .. 8 */
  int32_t vocab;        /* V (1024): classes are V + 2 (blank = V, EOU = V + 1) */
  int32_t max_symbols;  /* emissions per frame before moving on (4), 1 .. 16 */
  int32_t max_streams;  /* stream ids 0 .. max_streams-1, <= 65536 */
  int32_t max_frames;   /* most frames one call decodes, 1 .. 16 */
  int32_t flags;        /* CAC_FLAG_DRY_RUN (cac.h): host-only context */
} cac_dec_config;

/* Float parameters cac_dec_create expects, in this order (float32, host; matrices [in][out]):
 *   embed[V+2][H]
 *   for each layer l: w_ih[H][4H] w_hh[H][4H] b_ih[4H] b_hh[4H]   (gate blocks i, f, g, o)
 *   proj_w[H][P] proj_b[P]
 *   out_w[P][V+2] out_b[V+2]
 * Returns 0 for an invalid config. */
size_t cac_dec_param_count(const cac_dec_config* cfg);

/* Bytes of device workspace a decoder context needs (repacked weights, the state of
 * max_streams streams, per-call scratch for max_streams x max_frames rows). 0 if invalid. */
size_t cac_dec_workspace_bytes(const cac_dec_config* cfg);

/* Validate cfg, repack the parameters into the workspace (256-byte aligned, at least
 * cac_dec_workspace_bytes), reset every stream, synchronise hip_stream and return the context
 * in *out. Errors: CAC_EINVAL (config, counts, NULL), CAC_ENOMEM (workspace), CAC_EHIP. */
int32_t cac_dec_create(const cac_dec_config* cfg, const float* h_params, size_t n_params, void* d_workspace,
                       size_t ws_bytes, void* hip_stream, cac_dec** out);

/* Greedy decoding of n_frames (1 .. max_frames) new frames for n_streams distinct streams
 * (ids in h_stream_ids, 1 .. max_streams of them).
 *   d_z            [n_streams][n_frames][P] float32: the projected encoder frames (for example
 *                  the d_out of cac_push_chunk);
 *   d_tokens       [n_streams][n_frames * max_symbols] int32: emitted classes in order,
 *                  -1 after the last;
 *   d_token_frames [n_streams][n_frames * max_symbols] int32: the frame (0 .. n_frames-1)
 *                  each class was emitted at, -1 after the last (may be NULL);
 *   d_counts       [n_streams] int32: classes emitted per stream.
 * The call runs 1 + n_frames * max_symbols predictor / joint rounds (each round's kernels
 * return at once when no stream needs them). Asynchronous: outputs are valid once the stream
 * is synchronised. Returns 0. */
int32_t cac_dec_greedy(cac_dec* ctx, int32_t n_streams, const int32_t* h_stream_ids, int32_t n_frames,
                       const float* d_z, int32_t* d_tokens, int32_t* d_token_frames, int32_t* d_counts);

/* Decode calls are recorded once per call shape (streams, frames, whether token frames are
 * wanted) into a HIP graph of kernel nodes and replayed, the nodes holding the caller's
 * pointers re-pointed between replays; enable = 0 launches every kernel directly (as
 * profiling always does). Default on. */
int32_t cac_dec_set_graph(cac_dec* ctx, int32_t enable);

/* Per-kernel timing of later decode calls (measurement aid), as cac_profile in cac.h: each
 * kernel launched with start and stop HIP events bound to its dispatch. After each profiled
 * call the library reads back how many streams each round's lists held (a synchronisation)
 * and gives every launch its algorithmic flops (2 x rows x K x N of its tile product) and
 * weight bytes; launches whose list was empty are recorded as "<kernel>/idle".
 * cac_dec_profile(ctx, 1) clears and starts, 0 stops; cac_dec_profile_read synchronises and
 * fills, per kernel name (up to max_entries; names is max_entries * name_len chars): launches,
 * total milliseconds, bytes and flops. Returns the number of kernel names. */
int32_t cac_dec_profile(cac_dec* ctx, int32_t enable);
int32_t cac_dec_profile_read(cac_dec* ctx, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
                             double* total_ms, double* bytes, double* flops);

/* Return streams to the fresh state (zero LSTM state, next prediction from blank). Returns n. */
int32_t cac_dec_reset(cac_dec* ctx, int32_t n, const int32_t* h_stream_ids);

/* Free the host context (the workspace stays the caller's). Accepts NULL. */
int32_t cac_dec_destroy(cac_dec* ctx);

/* Description of the last error on ctx; with ctx == NULL, of the last failed cac_dec_create
 * on this thread. Never NULL. */
const char* cac_dec_last_error(const cac_dec* ctx);

#ifdef __cplusplus
}
#endif

#endif /* CAC_DECODE_H */

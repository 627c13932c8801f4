/* cac_beam.h — C ABI of batched MALSD beam search on MI355X (gfx950): the projected encoder
 * frames of many utterances in, the K best transcripts of each out.
 *
 * What one call computes, per utterance ("Fast Accuracy-Preserving RNNT Beam Search on Apple
 * Silicon", §2.2 "One pinned iteration", §2.3 "Equality and recombination", §2.4
 * "Configuration fields that can change output", §4.1 "Fixed storage"):
 *   A beam of K slots starts with one empty hypothesis (score 0, frame 0); the prediction
 *   network starts on the blank token from zero state. Every iteration moves each live
 *   hypothesis by one alignment step: log_softmax of the joint after projection,
 *   ReLU(z[t] + p) Wout + bout, over all classes; its K best classes become candidates (score +
 *   log-probability), or blank alone once it has emitted max_symbols labels at its frame (the
 *   blank's full log-probability); a hypothesis past its last frame offers itself unchanged.
 *   The K best candidates of the utterance survive (ranked by score, then slot, then class:
 *   ties go to the lower index). Blank moves to the next frame, a label extends the
 *   transcript. Survivors with the same transcript are then merged: the highest-scoring one
 *   (ties: lower slot) keeps its slot with the log-sum-exp of their scores, the others leave
 *   the beam. The predictor advances on new labels; blank keeps the parent's state. The loop
 *   ends when no live hypothesis has frames left.
 * Classes: vocab tokens 0 .. vocab-1, blank = vocab, EOU = vocab + 1 (a token like any other
 * here). The weights are those of cac_decode.h (same order and shapes). Arithmetic is float32.
 * Transcript equality is decided on the tokens themselves (a 64-bit hash of the transcript,
 * its length and last label only select the pairs to compare), so no two different
 * transcripts are ever merged.
 *
 * Conventions as in cac.h (int32 returns, CAC_* error codes, "d_" device / "h_" host pointers,
 * work on the create-time stream, validation before any device work, no device allocation).
 */
#ifndef CAC_BEAM_H
#define CAC_BEAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cac_beam cac_beam;

typedef struct {
  int32_t joint_dim;    /* P: width of the projected frames and predictor output (640), multiple of 64 */
  int32_t pred_hidden;  /* H: embedding and LSTM width (640), multiple of 64 */
  int32_t pred_layers;  /* LSTM layers (2), 1 .. 8 */
  int32_t vocab;        /* V (1024); classes C = V + 2 <= 2048 */
  int32_t beam;         /* K: 1 .. 8 */
  int32_t max_symbols;  /* labels per frame before blank is forced (10), 1 .. 16 */
  int32_t max_streams;  /* utterances per call, 1 .. 4096 */
  int32_t max_frames;   /* frames per utterance, 1 .. 4096 */
  int32_t score_norm;   /* 1: rank the final beam by score / (length + 1); 0: by score */
  int32_t flags;        /* CAC_FLAG_DRY_RUN (cac.h); CAC_BEAM_FLAG_WEAK_HASH */
} cac_beam_config;

/* Replace the transcript hash by 0, so every pair of hypotheses with equal length and last
 * label has its tokens compared (a test of the collision path; results do not change). */
#define CAC_BEAM_FLAG_WEAK_HASH 0x100

/* Number of float32 parameters (the greedy decoder's: cac_dec_param_count of the same sizes).
 * 0 for an invalid config. */
size_t cac_beam_param_count(const cac_beam_config* cfg);

/* Device workspace bytes: weights, the per-utterance beams (two copies of every slot's state
 * and transcript, whose stride is max_frames * max_symbols tokens), 2K predictor states per
 * utterance, the staged frames, the joint's logits and the work lists. 0 for an invalid config. */
size_t cac_beam_workspace_bytes(const cac_beam_config* cfg);

/* Validate cfg, repack the weights (order of cac_decode.h), compute the start state of the
 * prediction network, synchronise and return the context. CAC_EINVAL / CAC_ENOMEM / CAC_EHIP. */
int32_t cac_beam_create(const cac_beam_config* cfg, const float* h_params, size_t n_params, void* d_workspace,
                        size_t ws_bytes, void* hip_stream, cac_beam** out);

/* Beam search over n_streams utterances. d_z is [n_streams][n_frames][P] float32 (the
 * encoder's projected frames); h_lengths[i] (0 .. n_frames) is utterance i's frame count.
 * max_steps > 0 stops after that many iterations (the beam as it stands then, live
 * hypotheses included); 0 runs to the end. Outputs, per utterance, the K slots ranked best
 * first (score_norm), empty slots last:
 *   d_tokens  [n_streams][K][n_frames * max_symbols] int32, -1 past each transcript's end;
 *   d_lengths [n_streams][K] int32 transcript lengths, -1 for an empty slot;
 *   d_scores  [n_streams][K] float32 log-probability scores, -inf for an empty slot;
 *   d_frames  [n_streams][K] int32 the frame each hypothesis stands at (NULL: not written).
 * The call waits for the device between groups of iterations to learn whether any
 * hypothesis still has frames (it returns after the device has finished). Returns the number
 * of iterations the longest utterance took (>= 0), or a CAC_* error. */
int32_t cac_beam_decode(cac_beam* ctx, int32_t n_streams, const int32_t* h_lengths, int32_t n_frames,
                        const float* d_z, int32_t max_steps, int32_t* d_tokens, int32_t* d_lengths, float* d_scores,
                        int32_t* d_frames);

/* Graph replay of each group of iterations (default on). */
int32_t cac_beam_set_graph(cac_beam* ctx, int32_t enable);

/* Per-kernel timing as cac_dec_profile / cac_dec_profile_read (cac_decode.h): with profiling
 * on, calls launch their kernels one by one with events around each. */
int32_t cac_beam_profile(cac_beam* ctx, int32_t enable);
int32_t cac_beam_profile_read(cac_beam* ctx, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
                              double* total_ms, double* bytes, double* flops);

/* Free the host context. Accepts NULL. */
int32_t cac_beam_destroy(cac_beam* ctx);

/* Description of the last error on ctx; with NULL, of the last failed cac_beam_create on this
 * thread. Never NULL. */
const char* cac_beam_last_error(const cac_beam* ctx);

#ifdef __cplusplus
}
#endif

#endif /* CAC_BEAM_H */

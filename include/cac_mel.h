/* cac_mel.h — C ABI of the streaming log-mel front on MI355X (gfx950): raw 16 kHz audio of
 * many streams in, log-mel frames out (the input of cac.h's front end).
 *
 * Per stream and push of whole hops ("True streaming encode — implementation spec", "Per-chunk
 * flow" step 1: the mel frames of [melTail || chunk]; "Status": the streaming mel is exact
 * against the offline one), frame g of the push is computed from the win_length preemphasised
 * samples that end at that frame's hop boundary (causal frames; samples before the stream
 * start are 0):
 *   y[n] = x[n] - preemph * x[n-1]; periodic Hann window; n_fft-point DFT (zero padded);
 *   power |X[k]|^2, k = 0 .. n_fft/2; n_mels triangular filters on the Slaney mel scale
 *   between fmin and fmax, each of unit area; out = log(mel + 2^-24).
 * The stream carries its last win_length - hop + 1 raw samples between pushes, so chunked
 * pushes give exactly the frames of one push over the whole signal. The transform runs in
 * float64 from the float32 samples; only the output is rounded (to out_dtype).
 *
 * Conventions as in cac.h (int32 returns, CAC_* error codes, "d_" device / "h_" host pointers,
 * work on the create-time stream, validation before any device work, no device allocation).
 */
#ifndef CAC_MEL_H
#define CAC_MEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cac_mel cac_mel;

typedef struct {
  int32_t sample_rate;  /* 16000 */
  int32_t n_fft;        /* 512: 128, 256, 512 or 1024 */
  int32_t win_length;   /* 400: <= n_fft, > hop */
  int32_t hop;          /* 160 */
  int32_t n_mels;       /* 128, <= 256 */
  double fmin, fmax;    /* 0, 8000 (0 <= fmin < fmax <= sample_rate / 2) */
  double preemph;       /* 0.97 (0 = none) */
  int32_t out_dtype;    /* CAC_F32 or CAC_BF16 (cac.h) */
  int32_t max_streams;  /* stream ids 0 .. max_streams-1, <= 2^20 */
  int32_t max_hops;     /* most hops one push carries (16 = one 160 ms chunk), <= 64 */
  int32_t flags;        /* CAC_FLAG_DRY_RUN (cac.h) */
} cac_mel_config;

/* Device workspace bytes (window, twiddle and filter tables, every stream's sample tail).
 * 0 for an invalid config. */
size_t cac_mel_workspace_bytes(const cac_mel_config* cfg);

/* Validate cfg, build the window, twiddle and filter tables (on the host, in double), zero every stream's
 * tail, synchronise and return the context. CAC_EINVAL / CAC_ENOMEM / CAC_EHIP. */
int32_t cac_mel_create(const cac_mel_config* cfg, void* d_workspace, size_t ws_bytes, void* hip_stream,
                       cac_mel** out);

/* Log-mel frames of n_streams distinct streams (ids in h_stream_ids): d_audio is
 * [n_streams][n_samples] float32 (n_samples a multiple of hop, at most max_hops * hop),
 * d_mel receives [n_streams][n_samples / hop][n_mels] in out_dtype. Asynchronous. Returns the
 * frames per stream. */
int32_t cac_mel_push(cac_mel* ctx, int32_t n_streams, const int32_t* h_stream_ids, int32_t n_samples,
                     const float* d_audio, void* d_mel);

/* Zero the sample tails of n streams (a fresh stream). Returns n. */
int32_t cac_mel_reset(cac_mel* ctx, int32_t n, const int32_t* h_stream_ids);

/* Free the host context. Accepts NULL. */
int32_t cac_mel_destroy(cac_mel* ctx);

/* Description of the last error on ctx; with NULL, of the last failed cac_mel_create on this
 * thread. Never NULL. */
const char* cac_mel_last_error(const cac_mel* ctx);

#ifdef __cplusplus
}
#endif

#endif /* CAC_MEL_H */

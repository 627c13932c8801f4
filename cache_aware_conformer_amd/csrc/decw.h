// Parameters of the prediction network and the joint after projection as the greedy and beam
// decoders keep them on the device (host-side helpers, used at create time).
//
// Caller order (cac_decode.h): embed [C][H]; per LSTM layer w_ih [H][4H], w_hh [H][4H], b_ih
// [4H], b_hh [4H] (gate blocks i, f, g, o); proj_w [H][P], proj_b [P]; out_w [P][C], out_b [C].
// Device order: every matrix stored per output column, its K inputs contiguous ([N][K], the
// layout the tile loop reads): the same embedding; per LSTM layer one [4H][2H] matrix whose row
// n = 4u + g holds unit u's gate g (i, f, g, o) with the w_ih inputs first and the w_hh inputs
// after them, and the two biases summed in the same row order; the projection as [P][H]; the
// joint as [Cpad][P] with rows C .. Cpad-1 (and their bias) zero, Cpad a multiple of 64.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

struct DecWeights {
  size_t embed, lstm_w, lstm_b, proj_w, proj_b, out_w, out_b, end;
};

inline size_t dec_param_count(size_t C, size_t H, size_t L, size_t P) {
  return C * H + L * (2 * H * 4 * H + 2 * 4 * H) + H * P + P + P * C + C;
}

// Offsets of every region, each taken from take(bytes) (which aligns and advances).
template <class Take>
DecWeights dec_weight_offsets(Take take, size_t C, size_t H, size_t L, size_t P, size_t Cpad) {
  DecWeights w;
  w.embed = take(C * H * 4);
  w.lstm_w = take(L * 2 * H * 4 * H * 4);
  w.lstm_b = take(L * 4 * H * 4);
  w.proj_w = take(H * P * 4);
  w.proj_b = take(P * 4);
  w.out_w = take(P * Cpad * 4);
  w.out_b = take(Cpad * 4);
  w.end = take(0);
  return w;
}

// Repack the caller's parameters into buf (zeroed, at least w.end bytes) at the offsets of w.
inline void dec_repack(const float* params, const DecWeights& w, size_t C, size_t H, size_t L, size_t P, size_t Cpad,
                       uint8_t* buf) {
  const float* q = params;
  auto take = [&](size_t k) { const float* r = q; q += k; return r; };
  memcpy(buf + w.embed, take(C * H), C * H * 4);
  for (size_t l = 0; l < L; ++l) {
    const float* wih = take(H * 4 * H);
    const float* whh = take(H * 4 * H);
    const float* bih = take(4 * H);
    const float* bhh = take(4 * H);
    float* m = (float*)(buf + w.lstm_w) + l * 2 * H * 4 * H;
    float* b = (float*)(buf + w.lstm_b) + l * 4 * H;
    for (size_t g = 0; g < 4; ++g)
      for (size_t u = 0; u < H; ++u) {
        const size_t src = g * H + u, dst = 4 * u + g;
        b[dst] = bih[src] + bhh[src];
        float* row = m + dst * 2 * H;
        for (size_t k = 0; k < H; ++k) {
          row[k] = wih[k * 4 * H + src];
          row[H + k] = whh[k * 4 * H + src];
        }
      }
  }
  const float* pw = take(H * P);
  float* pd = (float*)(buf + w.proj_w);
  for (size_t k = 0; k < H; ++k)
    for (size_t n = 0; n < P; ++n) pd[n * H + k] = pw[k * P + n];
  memcpy(buf + w.proj_b, take(P), P * 4);
  const float* ow = take(P * C);
  float* od = (float*)(buf + w.out_w);
  for (size_t k = 0; k < P; ++k)
    for (size_t n = 0; n < C; ++n) od[n * P + k] = ow[k * C + n];
  memcpy(buf + w.out_b, take(C), C * 4);
}

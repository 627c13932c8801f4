// Streaming log-mel front (include/cac_mel.h): raw audio of many streams -> log-mel frames.
//
// One wave per (stream, frame), blocks on grid (stream, frame); the transform, power and filter
// sums run in float64 (a bin's float32 error would scale with the frame's energy, not the bin's,
// which the low bands after preemphasis hold a millionth of), the output is rounded once. The
// frame's win_length
// preemphasised, Hann-weighted samples are packed two to a complex value (even sample real,
// odd sample imaginary) into LDS in
// bit-reversed order, transformed by an n_fft/2-point radix-2 FFT, and split into the n_fft
// real DFT bins (X[k] = E[k] + W^k O[k] with E, O the transforms of the even and odd samples).
// The mel filters are sparse: each lane sums its filters' few bins from the power spectrum in
// LDS and takes the log. A second kernel, one block per stream, moves the stream's raw-sample
// tail forward once every frame of the push has read it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/cac.h"
#include "../../include/cac_mel.h"
#include "common.h"

void kernels_init();

namespace {

struct MelArgs {
  const int32_t* ids;    // [n] stream ids
  const float* audio;    // [n][ns] caller's samples
  const float* tail;     // [S][T] raw samples before this push
  void* out;             // [n][G][n_mels] caller's frames
  const double* win;     // [win_len] Hann window
  const double2* tw;     // [N2 / 2] exp(-2 pi i j / N2)
  const double2* tw2;    // [N2 + 1] exp(-2 pi i k / n_fft)
  const int32_t* fspan;  // [n_mels][2]: first bin, bin count
  const int32_t* foff;   // [n_mels] offset of the filter's weights in fw
  const double* fw;
  int n, ns, G, win_len, hop, T, N2, bits, n_mels, out_bf16;
  double preemph;
};

__global__ __launch_bounds__(64) void mel_kernel(MelArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int id = a.ids[s];
  extern __shared__ __attribute__((aligned(16))) double mlds[];
  double2* buf = (double2*)mlds;               // [N2]
  double* pw = mlds + 2 * a.N2;                // [N2 + 1]
  const float* tl = a.tail + (long)id * a.T;
  const float* au = a.audio + (long)s * a.ns;
  // raw sample q of tail || audio
  auto raw = [&](int q) { return (double)(q < a.T ? tl[q] : au[q - a.T]); };
  const double pre = a.preemph;
  const int p0 = g * a.hop;  // window sample j is preemph(raw[p0 + j + 1], raw[p0 + j])
  for (int m = lane; m < a.N2; m += 64) {
    double re = 0.0, im = 0.0;
    const int j = 2 * m;
    if (j + 1 < a.win_len) {
      re = (raw(p0 + j + 1) - pre * raw(p0 + j)) * a.win[j];
      im = (raw(p0 + j + 2) - pre * raw(p0 + j + 1)) * a.win[j + 1];
    }
    buf[__brev((unsigned)m) >> (32 - a.bits)] = make_double2(re, im);
  }
  __syncthreads();
  for (int len = 2; len <= a.N2; len <<= 1) {
    const int half = len >> 1, step = a.N2 / len;
    for (int b = lane; b < a.N2 / 2; b += 64) {
      const int grp = b / half, j = b - grp * half;
      const int i0 = grp * len + j, i1 = i0 + half;
      const double2 w = a.tw[j * step];
      const double2 u = buf[i0], v = buf[i1];
      const double2 t = make_double2(w.x * v.x - w.y * v.y, w.x * v.y + w.y * v.x);
      buf[i0] = make_double2(u.x + t.x, u.y + t.y);
      buf[i1] = make_double2(u.x - t.x, u.y - t.y);
    }
    __syncthreads();
  }
  // real split: Z[k] and conj(Z[N2 - k]) give the even-sample transform E and the odd one O
  for (int k = lane; k <= a.N2; k += 64) {
    const double2 zk = buf[k & (a.N2 - 1)], zc = buf[(a.N2 - k) & (a.N2 - 1)];
    const double er = 0.5 * (zk.x + zc.x), ei = 0.5 * (zk.y - zc.y);   // (Z[k] + conj Z[N2-k]) / 2
    const double orr = 0.5 * (zk.y + zc.y), oi = -0.5 * (zk.x - zc.x); // (Z[k] - conj Z[N2-k]) / 2i
    const double2 w = a.tw2[k];
    const double xr = er + w.x * orr - w.y * oi, xi = ei + w.x * oi + w.y * orr;
    pw[k] = xr * xr + xi * xi;
  }
  __syncthreads();
  for (int m = lane; m < a.n_mels; m += 64) {
    const int k0 = a.fspan[2 * m], nk = a.fspan[2 * m + 1];
    const double* w = a.fw + a.foff[m];
    double acc = 0.0;
    for (int k = 0; k < nk; ++k) acc += pw[k0 + k] * w[k];
    const float v = (float)log(acc + 5.9604644775390625e-8);  // 2^-24
    const long o = ((long)s * a.G + g) * a.n_mels + m;
    if (a.out_bf16) ((bf16_t*)a.out)[o] = f2bf(v);
    else ((float*)a.out)[o] = v;
  }
}

struct MelTailArgs {
  const int32_t* ids;
  const float* audio;
  float* tail;
  int ns, T;
};

// New tail = the last T raw samples of tail || audio; one block per stream (it alone touches
// that stream's tail in this kernel).
__global__ __launch_bounds__(256) void mel_tail_kernel(MelTailArgs a) {
  const int s = blockIdx.x, id = a.ids[s];
  float* tl = a.tail + (long)id * a.T;
  const float* au = a.audio + (long)s * a.ns;
  float v[4];
  int cnt = 0;
  for (int i = threadIdx.x; i < a.T && cnt < 4; i += 256, ++cnt) {
    const int q = a.ns + i;  // index in tail || audio
    v[cnt] = q < a.T ? tl[q] : au[q - a.T];
  }
  __syncthreads();
  cnt = 0;
  for (int i = threadIdx.x; i < a.T && cnt < 4; i += 256, ++cnt) tl[i] = v[cnt];
}

struct MelResetArgs {
  const int32_t* ids;
  float* tail;
  int T;
};

__global__ __launch_bounds__(256) void mel_reset_kernel(MelResetArgs a) {
  float* tl = a.tail + (long)a.ids[blockIdx.x] * a.T;
  for (int i = threadIdx.x; i < a.T; i += 256) tl[i] = 0.0f;
}

// ------------------------------------------------------------------------------- host side
struct MelDims {
  int sr, nfft, win, hop, nm, out_bf16, S, max_hops, flags, N2, bits, T;
  double fmin, fmax, pre;
};

bool mel_dims(const cac_mel_config* c, MelDims& d, std::string& why) {
  if (!c) { why = "config is NULL"; return false; }
  d.sr = c->sample_rate; d.nfft = c->n_fft; d.win = c->win_length; d.hop = c->hop; d.nm = c->n_mels;
  d.fmin = c->fmin; d.fmax = c->fmax; d.pre = c->preemph; d.S = c->max_streams; d.max_hops = c->max_hops;
  d.flags = c->flags;
  auto bad = [&](const char* m) { why = m; return false; };
  if (d.sr < 1000 || d.sr > 192000) return bad("sample_rate must be in [1000, 192000]");
  if (d.nfft != 128 && d.nfft != 256 && d.nfft != 512 && d.nfft != 1024) return bad("n_fft must be 128, 256, 512 or 1024");
  if (d.hop < 1 || d.win <= d.hop || d.win > d.nfft || d.win % 2) return bad("need hop < win_length <= n_fft, win_length even");
  if (d.nm < 1 || d.nm > 256) return bad("n_mels must be in [1, 256]");
  if (!(d.fmin >= 0.0) || !(d.fmax > d.fmin) || d.fmax > 0.5 * d.sr) return bad("need 0 <= fmin < fmax <= sample_rate / 2");
  if (!(d.pre >= 0.0) || d.pre > 1.0) return bad("preemph must be in [0, 1]");
  if (c->out_dtype != CAC_F32 && c->out_dtype != CAC_BF16) return bad("out_dtype must be CAC_F32 or CAC_BF16");
  if (d.S < 1 || d.S > (1 << 20)) return bad("max_streams must be in [1, 2^20]");
  if (d.max_hops < 1 || d.max_hops > 64) return bad("max_hops must be in [1, 64]");
  d.out_bf16 = c->out_dtype == CAC_BF16;
  d.N2 = d.nfft / 2;
  d.bits = 0;
  while ((1 << d.bits) < d.N2) ++d.bits;
  d.T = d.win - d.hop + 1;
  return true;
}

// Slaney mel scale: linear below 1 kHz (3 f / 200), logarithmic above (15 + 27 ln(f / 1000) / ln 6.4)
double slaney_mel(double f) { return f < 1000.0 ? 3.0 * f / 200.0 : 15.0 + 27.0 * std::log(f / 1000.0) / std::log(6.4); }
double slaney_hz(double m) { return m < 15.0 ? 200.0 * m / 3.0 : 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0); }

struct MelTables {
  std::vector<double> win, tw, tw2, fw;
  std::vector<int32_t> fspan, foff;
};

MelTables mel_tables(const MelDims& d) {
  MelTables t;
  const double pi = 3.14159265358979323846;
  t.win.resize(d.win);
  for (int i = 0; i < d.win; ++i) t.win[i] = 0.5 - 0.5 * std::cos(2.0 * pi * i / d.win);
  for (int j = 0; j < d.N2 / 2; ++j) {
    t.tw.push_back(std::cos(2.0 * pi * j / d.N2));
    t.tw.push_back(-std::sin(2.0 * pi * j / d.N2));
  }
  for (int k = 0; k <= d.N2; ++k) {
    t.tw2.push_back(std::cos(2.0 * pi * k / d.nfft));
    t.tw2.push_back(-std::sin(2.0 * pi * k / d.nfft));
  }
  const double m0 = slaney_mel(d.fmin), m1 = slaney_mel(d.fmax);
  for (int m = 0; m < d.nm; ++m) {
    const double lo = slaney_hz(m0 + (m1 - m0) * m / (d.nm + 1));
    const double mid = slaney_hz(m0 + (m1 - m0) * (m + 1) / (d.nm + 1));
    const double hi = slaney_hz(m0 + (m1 - m0) * (m + 2) / (d.nm + 1));
    int first = -1, count = 0;
    t.foff.push_back((int32_t)t.fw.size());
    for (int k = 0; k <= d.N2; ++k) {
      const double f = (double)k * d.sr / d.nfft;
      const double tri = std::max(0.0, std::min((f - lo) / (mid - lo), (hi - f) / (hi - mid)));
      if (tri <= 0.0) continue;
      if (first < 0) first = k;
      // the bins between first and k are inside the triangle too (it is convex in f)
      while (first + count < k) { t.fw.push_back(0.0); ++count; }
      t.fw.push_back(tri * 2.0 / (hi - lo));
      ++count;
    }
    t.fspan.push_back(first < 0 ? 0 : first);
    t.fspan.push_back(count);
  }
  return t;
}

struct MelLayout {
  size_t win, tw, tw2, fspan, foff, fw, tail, ids, total;
};

MelLayout mel_layout(const MelDims& d, const MelTables& t) {
  MelLayout y{};
  size_t off = 0;
  auto take = [&](size_t b) { off = (off + 255) & ~(size_t)255; size_t o = off; off += b; return o; };
  y.win = take(t.win.size() * 8);
  y.tw = take(t.tw.size() * 8);
  y.tw2 = take(t.tw2.size() * 8);
  y.fspan = take(t.fspan.size() * 4);
  y.foff = take(t.foff.size() * 4);
  y.fw = take(std::max<size_t>(t.fw.size(), 1) * 8);
  y.tail = take((size_t)d.S * d.T * 4);
  y.ids = take((size_t)d.S * 4);
  y.total = take(0);
  return y;
}

thread_local std::string g_mel_error;

}  // namespace

struct cac_mel {
  MelDims d;
  MelTables t;
  MelLayout lay;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  bool dry = false;
  std::vector<int32_t> stamp, dev_ids;
  int32_t stamp_gen = 0;
  std::string err;
  template <class T> T* P(size_t off) const { return (T*)(ws + off); }
  int fail(int code, const std::string& m) { err = m; return code; }
};

namespace {

int mel_check_ids(cac_mel* c, int32_t n, const int32_t* ids) {
  if (n < 1 || n > c->d.S) return c->fail(CAC_EINVAL, "stream count out of range");
  if (!ids) return c->fail(CAC_EINVAL, "stream id list is NULL");
  if (++c->stamp_gen == INT32_MAX) { std::fill(c->stamp.begin(), c->stamp.end(), 0); c->stamp_gen = 1; }
  for (int i = 0; i < n; ++i) {
    const int id = ids[i];
    if (id < 0 || id >= c->d.S) return c->fail(CAC_EINVAL, "stream id " + std::to_string(id) + " out of range");
    if (c->stamp[id] == c->stamp_gen) return c->fail(CAC_EINVAL, "stream id " + std::to_string(id) + " appears twice");
    c->stamp[id] = c->stamp_gen;
  }
  return CAC_OK;
}

hipError_t mel_upload_ids(cac_mel* c, const int32_t* ids, int n) {
  if ((int)c->dev_ids.size() == n && memcmp(c->dev_ids.data(), ids, (size_t)n * 4) == 0) return hipSuccess;
  c->dev_ids.assign(ids, ids + n);
  return hipMemcpyAsync(c->ws + c->lay.ids, c->dev_ids.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
}

}  // namespace

extern "C" {

size_t cac_mel_workspace_bytes(const cac_mel_config* cfg) {
  MelDims d;
  std::string why;
  if (!mel_dims(cfg, d, why)) return 0;
  return mel_layout(d, mel_tables(d)).total;
}

const char* cac_mel_last_error(const cac_mel* ctx) { return ctx ? ctx->err.c_str() : g_mel_error.c_str(); }

int32_t cac_mel_create(const cac_mel_config* cfg, void* d_workspace, size_t ws_bytes, void* hip_stream, cac_mel** out) {
  g_mel_error.clear();
  if (!out) { g_mel_error = "out is NULL"; return CAC_EINVAL; }
  *out = nullptr;
  MelDims d;
  if (!mel_dims(cfg, d, g_mel_error)) return CAC_EINVAL;
  MelTables t = mel_tables(d);
  const MelLayout lay = mel_layout(d, t);
  const bool dry = (d.flags & CAC_FLAG_DRY_RUN) != 0;
  if (!dry) {
    if (!d_workspace) { g_mel_error = "workspace is NULL"; return CAC_EINVAL; }
    if (((uintptr_t)d_workspace) & 255) { g_mel_error = "workspace must be 256-byte aligned"; return CAC_EINVAL; }
    if (ws_bytes < lay.total) { g_mel_error = "workspace too small: need " + std::to_string(lay.total) + " bytes"; return CAC_ENOMEM; }
  }
  cac_mel* c = new cac_mel();
  c->d = d; c->t = std::move(t); c->lay = lay; c->ws = (char*)d_workspace; c->stream = (hipStream_t)hip_stream;
  c->dry = dry;
  c->stamp.assign(d.S, 0);
  if (dry) { *out = c; return CAC_OK; }
  std::vector<int32_t> all(d.S);
  for (int i = 0; i < d.S; ++i) all[i] = i;
  hipError_t e = hipSuccess;
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (e == hipSuccess && bytes) e = hipMemcpyAsync(c->ws + off, src, bytes, hipMemcpyHostToDevice, c->stream);
  };
  put(lay.win, c->t.win.data(), c->t.win.size() * 8);
  put(lay.tw, c->t.tw.data(), c->t.tw.size() * 8);
  put(lay.tw2, c->t.tw2.data(), c->t.tw2.size() * 8);
  put(lay.fspan, c->t.fspan.data(), c->t.fspan.size() * 4);
  put(lay.foff, c->t.foff.data(), c->t.foff.size() * 4);
  put(lay.fw, c->t.fw.data(), c->t.fw.size() * 8);
  c->dev_ids = all;
  put(lay.ids, c->dev_ids.data(), (size_t)d.S * 4);
  if (e == hipSuccess) {
    Launcher L;
    L.stream = c->stream;
    MelResetArgs r{c->P<int32_t>(lay.ids), c->P<float>(lay.tail), d.T};
    L.tag("mel_reset", 0.0, 0.0);
    L.launch((const void*)&mel_reset_kernel, dim3(d.S), dim3(256), 0, &r);
    e = L.err;
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    g_mel_error = std::string("HIP error during create: ") + hipGetErrorString(e);
    delete c;
    return CAC_EHIP;
  }
  *out = c;
  return CAC_OK;
}

int32_t cac_mel_push(cac_mel* c, int32_t n, const int32_t* ids, int32_t ns, const float* d_audio, void* d_mel) {
  if (!c) return CAC_EINVAL;
  const MelDims& d = c->d;
  int rc = mel_check_ids(c, n, ids);
  if (rc) return rc;
  if (ns < d.hop || ns % d.hop || ns / d.hop > d.max_hops)
    return c->fail(CAC_EINVAL, "n_samples must be a multiple of hop, at most max_hops * hop");
  if (!d_audio || !d_mel) return c->fail(CAC_EINVAL, "audio or mel pointer is NULL");
  const int G = ns / d.hop;
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  const hipError_t pe = hipStreamQuery(c->stream);
  if (pe != hipSuccess && pe != hipErrorNotReady)
    return c->fail(CAC_EHIP, std::string("asynchronous device error from earlier work: ") + hipGetErrorString(pe));
  Launcher L;
  L.stream = c->stream;
  L.err = mel_upload_ids(c, ids, n);
  const MelLayout& y = c->lay;
  MelArgs a{};
  a.ids = c->P<int32_t>(y.ids); a.audio = d_audio; a.tail = c->P<float>(y.tail); a.out = d_mel;
  a.win = c->P<double>(y.win); a.tw = c->P<double2>(y.tw); a.tw2 = c->P<double2>(y.tw2);
  a.fspan = c->P<int32_t>(y.fspan); a.foff = c->P<int32_t>(y.foff); a.fw = c->P<double>(y.fw);
  a.n = n; a.ns = ns; a.G = G; a.win_len = d.win; a.hop = d.hop; a.T = d.T; a.N2 = d.N2; a.bits = d.bits;
  a.n_mels = d.nm; a.out_bf16 = d.out_bf16; a.preemph = d.pre;
  const size_t shm = ((size_t)2 * d.N2 + d.N2 + 1) * sizeof(double);
  // algorithmic bytes: the new samples read, the frames written
  L.tag("logmel", (double)n * ns * 4.0 + (double)n * G * d.nm * (d.out_bf16 ? 2 : 4), 0.0);
  L.launch((const void*)&mel_kernel, dim3(n, G), dim3(64), shm, &a);
  MelTailArgs ta{a.ids, d_audio, c->P<float>(y.tail), ns, d.T};
  L.tag("mel_tail", 0.0, 0.0);
  L.launch((const void*)&mel_tail_kernel, dim3(n), dim3(256), 0, &ta);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  return G;
}

int32_t cac_mel_reset(cac_mel* c, int32_t n, const int32_t* ids) {
  if (!c) return CAC_EINVAL;
  int rc = mel_check_ids(c, n, ids);
  if (rc) return rc;
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  Launcher L;
  L.stream = c->stream;
  L.err = mel_upload_ids(c, ids, n);
  MelResetArgs r{c->P<int32_t>(c->lay.ids), c->P<float>(c->lay.tail), c->d.T};
  L.tag("mel_reset", 0.0, 0.0);
  L.launch((const void*)&mel_reset_kernel, dim3(n), dim3(256), 0, &r);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  return n;
}

int32_t cac_mel_destroy(cac_mel* c) {
  delete c;
  return CAC_OK;
}

}  // extern "C"

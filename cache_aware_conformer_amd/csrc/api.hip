// C ABI of the chunk-step library (include/cac.h): validation, workspace layout, weight
// repacking, host-side stream bookkeeping and the per-push launch sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cac.h"
#include "common.h"

void kernels_init();

// Device scratch of the no-allocation test GEMM: the float32 split-K partials live in this
// file-scope array (one copy per GPU, held until the process ends) instead of a hipMalloc'd
// buffer. Host code never passes the array's name to a kernel: it takes the per-device address
// hipGetSymbolAddress returns.
constexpr size_t kScratchFloats = (size_t)4 << 20;  // 16 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

thread_local std::string g_create_error;

std::mutex g_scratch_mu;
std::vector<float*> g_scratch_ptr;  // device address of `scratch`, per device id

// Address of the current device's scratch array, looked up once per device.
hipError_t scratch_ptr(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------------------- dimensions
struct Dims {
  int L, D, H, hd, F, K, Kc, Lc, c, right, ne, nla, nc, P, fe, bins, mpc, tail, dt, S, npush, flags;
  int fc;             // channels of the 2-D front end (frontend 2), else 0
  bool lookahead;
  int nfmax;          // frames per stream a call runs through the layers
  int R, Rc, Rx;      // ring depths: K/V, depthwise input, pending inputs
  int rel_lo, nrel;   // relative offsets covered by the position table
  size_t esz;         // bytes per compute-dtype element
  int wq;             // dense weights are int8 codes + float32 row scales (CAC_F32_I8)
  int dtype_cfg;      // the config's dtype field (dt is the activation/cache dtype)
  size_t wsz(size_t rows, size_t cols) const {  // bytes of one dense matrix [rows][cols]
    return wq ? rows * cols + rows * 4 : rows * cols * esz;
  }
};

bool make_dims(const cac_config* c, Dims& d, std::string& why) {
  if (!c) { why = "config is NULL"; return false; }
  d.L = c->n_layers; d.D = c->d_model; d.H = c->n_heads; d.F = c->d_ff; d.K = c->dw_kernel;
  d.Lc = c->att_left; d.c = c->att_chunk; d.right = c->att_right; d.ne = c->n_emit;
  d.nla = c->n_lookahead; d.P = c->joint_dim; d.fe = c->frontend; d.bins = c->mel_bins;
  d.mpc = c->mel_per_chunk; d.tail = c->mel_tail; d.dt = c->dtype; d.S = c->max_streams;
  d.npush = c->max_push_frames; d.flags = c->flags;
  auto bad = [&](const char* m) { why = m; return false; };
  if (d.L < 1 || d.L > 64) return bad("n_layers must be in [1, 64]");
  if (d.D < 64 || d.D > 1024 || d.D % 64) return bad("d_model must be a multiple of 64 in [64, 1024]");
  if (d.H < 1 || d.D % d.H) return bad("n_heads must divide d_model");
  d.hd = d.D / d.H;
  if (d.hd != 16 && d.hd != 32 && d.hd != 64) return bad("head_dim must be 16, 32 or 64");
  if (d.F < 64 || d.F > 4096 || d.F % 64) return bad("d_ff must be a multiple of 64 in [64, 4096]");
  if (d.K < 1 || d.K > 16) return bad("dw_kernel must be in [1, 16]");
  d.Kc = d.K - 1;
  if (d.Lc < 0 || d.Lc > 512) return bad("att_left must be in [0, 512]");
  if (d.c < 1 || d.c > 16) return bad("att_chunk must be in [1, 16]");
  if (d.nla < 0 || d.ne < 1) return bad("n_emit must be >= 1 and n_lookahead >= 0");
  d.lookahead = d.nla > 0;
  if (!d.lookahead && d.right != 0) return bad("att_right needs the lookahead variant (n_lookahead > 0)");
  if (d.right < 0 || d.right > 64) return bad("att_right must be in [0, 64]");
  d.nc = d.ne + d.nla;
  if (d.nc > 16) return bad("n_emit + n_lookahead must be <= 16");
  if (d.P < 0 || d.P > 8192) return bad("joint_dim must be in [0, 8192]");
  if (d.dt != CAC_F32 && d.dt != CAC_BF16 && d.dt != CAC_F32_I8) return bad("dtype must be CAC_F32, CAC_BF16 or CAC_F32_I8");
  d.dtype_cfg = d.dt;
  d.wq = d.dt == CAC_F32_I8;
  if (d.wq) {
    d.dt = CAC_F32;  // activations and caches
    if (c->frontend || c->n_lookahead > 0) return bad("CAC_F32_I8 is the one-stream path: no front end, no lookahead");
    if (c->d_model % 256 || c->d_ff % 256) return bad("CAC_F32_I8 needs d_model and d_ff multiples of 256");
  }
  if (d.S < 1 || d.S > (1 << 20)) return bad("max_streams must be in [1, 2^20]");
  d.fc = 0;
  if (d.fe != 0 && d.fe != 1 && d.fe != 2) return bad("frontend must be 0, 1 or 2");
  if (d.fe == 2) {
    d.fc = c->fe_channels;
    if (d.fc < 64 || d.fc > 512 || d.fc % 64) return bad("fe_channels must be a multiple of 64 in [64, 512]");
    if (d.dt != CAC_BF16) return bad("the 2-D front end runs in bf16 (CAC_BF16)");
    if (c->mel_bins % 64) return bad("the 2-D front end needs mel_bins a multiple of 64");
  }
  if (d.fe) {
    if (d.lookahead) return bad("the front end is supported with the exact variant only");
    if (d.mpc != 16 || d.tail != 14) return bad("the front end needs mel_per_chunk 16 and mel_tail 14");
    if (d.bins < 32 || d.bins > 1024 || d.bins % 32) return bad("mel_bins must be a multiple of 32 in [32, 1024]");
  } else {
    d.bins = 0; d.tail = 0; d.mpc = 0;
  }
  if (d.lookahead) {
    d.nfmax = d.nc;
  } else {
    if (d.npush < d.c || d.npush > 16 || d.npush % d.c) return bad("max_push_frames must be a multiple of att_chunk in [att_chunk, 16]");
    if (d.fe && d.npush < 2) return bad("the front end pushes 2 frames per chunk");
    d.nfmax = d.npush;
  }
  d.R = d.Lc + d.nfmax;
  d.Rc = d.Kc + d.nfmax;
  d.Rx = d.lookahead ? d.nc : 0;
  if (d.lookahead) { d.rel_lo = -d.right; d.nrel = d.Lc + d.right + 1; }
  else { d.rel_lo = -(d.c - 1); d.nrel = d.Lc + 2 * d.c - 1; }
  d.esz = d.dt == CAC_BF16 ? 2 : 4;
  if (d.R > 256) return bad("att_left + frames per call must be at most 256 (K/V ring slots)");
  if (attention_shmem(d.nfmax, d.R, d.nrel, d.hd, d.esz) > 160 * 1024) return bad("attention tile exceeds LDS: reduce att_left or frames per call");
  return true;
}

// ------------------------------------------------------------------------------- layout
struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) { off = (off + 255) & ~(size_t)255; size_t o = off; off += bytes; return o; }
};

struct LayerOff {
  size_t ln[10];  // ff1 g,b  att g,b  conv g,b  ff2 g,b  out g,b
  size_t b_ff1_1, b_ff1_2, b_qkv, b_o, b_pw1, b_dw, b_pw2, b_ff2_1, b_ff2_2, pos_u, pos_v, dw_w, wpos;
  size_t w_ff1_1, w_ff1_2, w_qkv, w_o, w_pw1, w_pw2, w_ff2_1, w_ff2_2;
  // bf16 weights: the products after the attention, conv and FF2 LayerNorms once more with the
  // LayerNorm folded in (gain-scaled rows, and per output column c1 = sum of the row, c2 = sum
  // of shift x weight + bias; pw1's c1, c2 in the bias order) for the rows that carry the
  // LayerNorm through the products
  size_t wg_qkv, c1_qkv, c2_qkv, wg_pw1, c1_pw1, c2_pw1, wg_ff2, c1_ff2, c2_ff2;
  size_t size;
};

struct Layout {
  LayerOff lo;
  size_t layers, wj, bj, fe_w[3], fe_b[3], weights_end;
  size_t f2_c1w, f2_c1b, f2_dw2w, f2_dw2b, f2_pw2w, f2_pw2b, f2_dw3w, f2_dw3b, f2_pw3w, f2_pw3b, f2_linw, f2_linb;
  size_t f2_a1, f2_d2, f2_a2, f2_d3, f2_a3;
  size_t posproj, posproj_bf, kring, vring, cring, tail, x0, pos, pend;
  size_t ids, cids, cidx, sids, spos, spend, cpos, ccpos;
  size_t x, x2, y, q, h, o, e, part, lns_a, lns_b, lnm_a, lnm_b, win, fe1, fe2;
  size_t total;
};

// bf16 weights in the compute dtype with D in 64-column tiles (at most 16): the LayerNorms
// before qkv, pw1 and FF2 up can ride on the products (see Pass::ln_carry)
bool ln_fold(const Dims& d) { return d.dt == CAC_BF16 && !d.wq && d.D % 64 == 0 && d.D / 64 <= 16; }

Layout make_layout(const Dims& d) {
  Layout t{};
  const size_t D = d.D, F = d.F, f4 = 4, e = d.esz;
  Bump b;
  LayerOff& lo = t.lo;
  for (int i = 0; i < 10; ++i) lo.ln[i] = b.take(D * f4);
  lo.b_ff1_1 = b.take(F * f4); lo.b_ff1_2 = b.take(D * f4); lo.b_qkv = b.take(3 * D * f4);
  lo.b_o = b.take(D * f4); lo.b_pw1 = b.take(2 * D * f4); lo.b_dw = b.take(D * f4);
  lo.b_pw2 = b.take(D * f4); lo.b_ff2_1 = b.take(F * f4); lo.b_ff2_2 = b.take(D * f4);
  lo.pos_u = b.take(D * f4); lo.pos_v = b.take(D * f4); lo.dw_w = b.take((size_t)d.K * D * f4);
  lo.wpos = b.take(D * D * f4);
  // dense matrices [N][K] (int8 weights: the codes, then the N row scales)
  lo.w_ff1_1 = b.take(d.wsz(F, D)); lo.w_ff1_2 = b.take(d.wsz(D, F)); lo.w_qkv = b.take(d.wsz(3 * D, D));
  lo.w_o = b.take(d.wsz(D, D)); lo.w_pw1 = b.take(d.wsz(2 * D, D)); lo.w_pw2 = b.take(d.wsz(D, D));
  lo.w_ff2_1 = b.take(d.wsz(F, D)); lo.w_ff2_2 = b.take(d.wsz(D, F));
  const bool lnw = ln_fold(d);
  lo.wg_qkv = b.take(lnw ? 3 * D * D * e : 0); lo.c1_qkv = b.take(lnw ? 3 * D * f4 : 0); lo.c2_qkv = b.take(lnw ? 3 * D * f4 : 0);
  lo.wg_pw1 = b.take(lnw ? 2 * D * D * e : 0); lo.c1_pw1 = b.take(lnw ? 2 * D * f4 : 0); lo.c2_pw1 = b.take(lnw ? 2 * D * f4 : 0);
  lo.wg_ff2 = b.take(lnw ? F * D * e : 0); lo.c1_ff2 = b.take(lnw ? F * f4 : 0); lo.c2_ff2 = b.take(lnw ? F * f4 : 0);
  lo.size = (b.take(0) + 255) & ~(size_t)255;

  Bump w;
  t.layers = w.take(lo.size * d.L);
  if (d.P) { t.wj = w.take(d.wsz(d.P, D)); t.bj = w.take((size_t)d.P * f4); }
  if (d.fe == 1) {
    const size_t kin[3] = {(size_t)3 * d.bins, 3 * D, 3 * D};
    for (int i = 0; i < 3; ++i) { t.fe_w[i] = w.take(D * kin[i] * e); t.fe_b[i] = w.take(D * f4); }
  } else if (d.fe == 2) {
    const size_t C = d.fc, K8 = (size_t)d.fc * (d.bins / 8);
    t.f2_c1w = w.take(9 * C * f4); t.f2_c1b = w.take(C * f4);
    t.f2_dw2w = w.take(9 * C * f4); t.f2_dw2b = w.take(C * f4);
    t.f2_pw2w = w.take(C * C * e); t.f2_pw2b = w.take(C * f4);
    t.f2_dw3w = w.take(9 * C * f4); t.f2_dw3b = w.take(C * f4);
    t.f2_pw3w = w.take(C * C * e); t.f2_pw3b = w.take(C * f4);
    t.f2_linw = w.take(D * K8 * e); t.f2_linb = w.take(D * f4);
  }
  t.weights_end = w.take(0);
  const size_t S = d.S, L = d.L, M = S * d.nfmax;
  t.posproj = w.take(L * d.H * d.nrel * d.hd * f4);
  // bf16 copy of the position table (operand of the bf16 MFMA attention kernel)
  if (d.dt == CAC_BF16) t.posproj_bf = w.take(L * d.H * d.nrel * d.hd * 2);
  t.kring = w.take(L * S * d.H * d.R * d.hd * e);
  t.vring = w.take(L * S * d.H * d.R * d.hd * e);
  t.cring = w.take(L * S * d.Rc * D * e);
  t.tail = w.take(S * d.tail * d.bins * e);
  t.x0 = w.take(S * d.Rx * D * e);
  t.pos = w.take(S * 4); t.pend = w.take(S * 4);
  t.ids = w.take(S * 4); t.cids = w.take(S * 4); t.cidx = w.take(S * 4);
  t.sids = w.take(S * 4); t.spos = w.take(S * 4); t.spend = w.take(S * 4);
  t.cpos = w.take(S * 4); t.ccpos = w.take(S * 4);
  t.x = w.take(M * D * f4); t.x2 = w.take(M * D * f4); t.y = w.take(M * D * e); t.q = w.take(M * D * f4);
  t.h = w.take(M * F * e); t.o = w.take(M * D * e); t.e = w.take(M * D * e);
  // split-K partials of the residual products (bf16 MFMA path): up to 4 k-ranges
  if (d.dt == CAC_BF16) t.part = w.take(4 * M * D * f4);
  // LayerNorm statistics carried through the products: two sets of [D / 64][M] (mean, M2)
  if (ln_fold(d)) {
    t.lns_a = w.take(D / 64 * M * 8); t.lns_b = w.take(D / 64 * M * 8);
    t.lnm_a = w.take(M * f4); t.lnm_b = w.take(M * f4);
  }
  if (d.fe) t.win = w.take(S * (d.tail + d.mpc) * d.bins * e);
  if (d.fe == 1) {
    t.fe1 = w.take(S * 11 * D * e);
    t.fe2 = w.take(S * 5 * D * e);
  } else if (d.fe == 2) {  // channels-last stage maps: 11, 5 and 2 rows of F/2, F/4 and F/8 columns
    const size_t C = d.fc, B = d.bins;
    t.f2_a1 = w.take(S * 11 * (B / 2) * C * e);
    t.f2_d2 = w.take(S * 5 * (B / 4) * C * e);
    t.f2_a2 = w.take(S * 5 * (B / 4) * C * e);
    t.f2_d3 = w.take(S * 2 * (B / 8) * C * e);
    t.f2_a3 = w.take(S * 2 * (B / 8) * C * e);
  }
  t.total = w.take(0);
  return t;
}

size_t param_count(const Dims& d) {
  const size_t D = d.D, F = d.F, H = d.H, hd = d.hd;
  size_t per = 0;
  per += 2 * D + D * F + F + F * D + D;                        // ff1
  per += 2 * D + 4 * (D * D + D) + 2 * H * hd + D * D;         // att
  per += 2 * D + D * 2 * D + 2 * D + D * d.K + D + D * D + D;  // conv
  per += 2 * D + D * F + F + F * D + D;                        // ff2
  per += 2 * D;                                                // out
  size_t n = per * d.L;
  if (d.P) n += D * d.P + d.P;
  if (d.fe == 1) n += D * d.bins * 3 + D + 2 * (D * D * 3 + D);
  if (d.fe == 2) {
    const size_t C = d.fc;
    n += 3 * (9 * C + C) + 2 * (C * C + C) + C * (d.bins / 8) * D + D;
  }
  return n;
}

size_t state_floats(const Dims& d) {
  return STATE_HDR + 2 * (size_t)d.L * d.Lc * d.D + (size_t)d.L * d.Kc * d.D + (size_t)d.tail * d.bins +
         (size_t)d.nla * d.D;
}

// Header of a stream's state blob: magic, layout version, and a 64-bit FNV-1a hash of every
// config field that defines the model and the state's meaning (all but max_streams,
// max_push_frames and flags), taken after make_dims' normalisation.
void state_header(const Dims& d, uint32_t out[STATE_HDR]) {
  const int32_t f[] = {d.L, d.D, d.H, d.F, d.K, d.Lc, d.c, d.right, d.ne, d.nla, d.P, d.fe, d.bins, d.mpc, d.tail, d.dtype_cfg, d.fc};
  uint64_t h = 1469598103934665603ull;
  for (int32_t v : f)
    for (int b = 0; b < 4; ++b) {
      h ^= (uint64_t)(((uint32_t)v >> (8 * b)) & 0xffu);
      h *= 1099511628211ull;
    }
  out[0] = STATE_MAGIC;
  out[1] = STATE_VERSION;
  out[2] = (uint32_t)h;
  out[3] = (uint32_t)(h >> 32);
}

// ------------------------------------------------------------------------------- host packing
uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

struct Packer {
  std::vector<uint8_t>& buf;
  int dt;
  int wq = 0;          // dense matrices as int8 codes + row scales
  size_t rows = 0;     // rows of the dense matrix being packed (its scales follow the codes)
  void f32(size_t off, const float* src, size_t n) { memcpy(buf.data() + off, src, n * 4); }
  void op(size_t off, size_t idx, float v) {
    if (dt == CAC_BF16) ((uint16_t*)(buf.data() + off))[idx] = to_bf16(v);
    else ((float*)(buf.data() + off))[idx] = v;
  }
  // column n of in [K][N] as row `row` of a dense matrix [rows][K] at off. int8: the column's
  // scale s = max |w| / 127 and codes rint(w / s) clamped to [-127, 127] (0 for a zero
  // column), in float32 arithmetic, round half to even
  void column(size_t off, const float* in, size_t K, size_t N, size_t n, size_t row) {
    if (!wq) {
      for (size_t k = 0; k < K; ++k) op(off, row * K + k, in[k * N + n]);
      return;
    }
    float m = 0.0f;
    for (size_t k = 0; k < K; ++k) m = std::max(m, std::fabs(in[k * N + n]));
    const float sc = m / 127.0f;
    int8_t* q = (int8_t*)(buf.data() + off) + row * K;
    for (size_t k = 0; k < K; ++k) {
      float v = sc > 0.0f ? std::nearbyint(in[k * N + n] / sc) : 0.0f;
      v = std::min(127.0f, std::max(-127.0f, v));
      q[k] = (int8_t)v;
    }
    ((float*)(buf.data() + off + rows * K))[row] = sc;
  }
  // in [K][N] row-major -> rows row0 .. row0+N-1 of the [rows][K] matrix at off
  void transpose(size_t off, const float* in, size_t K, size_t N, size_t row0 = 0) {
    for (size_t n = 0; n < N; ++n) column(off, in, K, N, n, row0 + n);
  }
  // LayerNorm (gains g, shifts b) folded into column n of in [K][N]: row `row` of the bf16
  // matrix at off holds g[k] in[k][n] rounded; c1[ci] = the sum of that row as rounded,
  // c2[ci] = sum_k b[k] in[k][n] + bias (float64 sums)
  void ln_column(size_t off, size_t c1off, size_t c2off, const float* in, size_t K, size_t N, size_t n, size_t row,
                 size_t ci, const float* g, const float* b, float bias) {
    uint16_t* w = (uint16_t*)(buf.data() + off) + row * K;
    double s1 = 0.0, s2 = bias;
    for (size_t k = 0; k < K; ++k) {
      w[k] = to_bf16(g[k] * in[k * N + n]);
      s1 += (double)from_bf16(w[k]);
      s2 += (double)b[k] * in[k * N + n];
    }
    ((float*)(buf.data() + c1off))[ci] = (float)s1;
    ((float*)(buf.data() + c2off))[ci] = (float)s2;
  }
};


}  // namespace

// ------------------------------------------------------------------------------- context
struct cac_ctx {
  Dims d;
  Layout lay;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  bool dry = false;
  std::vector<int32_t> hpos, hpend;
  std::vector<uint8_t> flushed;
  std::vector<int32_t> dev_ids, dev_cids, dev_cidx;  // contents last uploaded
  std::vector<int32_t> stamp;
  int32_t stamp_gen = 0;
  std::string err;
  bool profiling = false;
  Profiler prof;
  // recorded push graphs, one per call shape
  struct Graph {
    hipGraph_t g = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<NodeRec> nodes;
    std::vector<std::vector<size_t>> in_offs, out_offs;  // per node: offsets of the caller pointers
    const void* in = nullptr;
    void* out = nullptr;
  };
  bool use_graph = true;
  std::map<uint64_t, Graph> graphs;
  Graph* last_graph = nullptr;  // graph of the most recent replayed push
  ~cac_ctx() {
    for (auto& kv : graphs) {
      if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
      if (kv.second.g) (void)hipGraphDestroy(kv.second.g);
    }
  }

  template <class T> T* P(size_t off) const { return (T*)(ws + off); }
  int fail(int code, const std::string& m) { err = m; return code; }
};

namespace {

int check_ids(cac_ctx* c, int32_t n, const int32_t* ids, bool need_open) {
  if (n < 1 || n > c->d.S) return c->fail(CAC_EINVAL, "stream count out of range");
  if (!ids) return c->fail(CAC_EINVAL, "stream id list is NULL");
  if (++c->stamp_gen == INT32_MAX) { std::fill(c->stamp.begin(), c->stamp.end(), 0); c->stamp_gen = 1; }
  for (int i = 0; i < n; ++i) {
    const int id = ids[i];
    if (id < 0 || id >= c->d.S) return c->fail(CAC_EINVAL, "stream id " + std::to_string(id) + " out of range");
    if (c->stamp[id] == c->stamp_gen) return c->fail(CAC_EINVAL, "stream id " + std::to_string(id) + " appears twice");
    c->stamp[id] = c->stamp_gen;
    if (need_open && c->flushed[id]) return c->fail(CAC_ESTATE, "stream " + std::to_string(id) + " was flushed; reset it first");
  }
  return CAC_OK;
}

hipError_t upload(cac_ctx* c, std::vector<int32_t>& cache, size_t off, const int32_t* src, int n) {
  if ((int)cache.size() == n && memcmp(cache.data(), src, n * 4) == 0) return hipSuccess;
  cache.assign(src, src + n);
  return hipMemcpyAsync(c->ws + off, cache.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
}

// ------------------------------------------------------------------------------- layer pass
// The launch sequence of the Conformer blocks for the rows of one call (cv.n_streams streams x
// cv.nf frames, row m = stream m / nf, frame m % nf), starting from float32 rows in x.
struct Pass {
  cac_ctx* c;
  Launcher& L;
  CallView cv;
  int M;
  double kv_rows;  // sum over the call's streams of the K/V rows attention reads (fill + new)

  EpiArgs epi0() const {
    EpiArgs e{};
    e.cv = cv;
    e.D = c->d.D; e.H = c->d.H; e.hd = c->d.hd; e.R = c->d.R; e.Rc = c->d.Rc;
    return e;
  }
  // weight dtype of the dense products (int8 codes + row scales, or the compute dtype)
  int wdt() const { return c->d.wq ? DT_I8W : c->d.dt; }
  void gemm_plain(const void* A, int lda, const void* W, int N, int K, const EpiArgs& e) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.A = A; g.W = W; g.epi = e;
    g.amap = RowMap{INT_MAX, 0, lda};
    launch_gemm(L, g, wdt(), 0);
  }

  // few rows (float32 workloads, or <= 8 rows): every dense product runs in the small-M kernel
  // with its prologue fusions: the previous block's ln_out is applied by its consumers (FF1 up
  // as an extra LayerNorm, FF1 down as the LayerNorm'ed residual base written to the other x
  // buffer), and the depthwise conv + SiLU is pw2's A operand.
  bool fused() const { return c->d.dt == CAC_F32 || M <= 8; }
  // many rows with D a multiple of 256 (<= 1024): each residual product is followed by one row
  // kernel that adds it to the residual stream and writes the next product's LayerNorm'ed
  // operand to y, so the products read y as plain compute-dtype rows
  bool row_kernels() const { return !fused() && c->d.D % 256 == 0 && c->d.D <= 1024; }
  float* cur = nullptr;  // buffer holding the residual stream (fused path: before ln_out)

  // k-ranges of a residual product (MFMA path): enough 64x64 tiles x ranges for a block per
  // CU, each range at least 128 deep; 1: no split
  int ksplit_for(int N, int K) const {
    const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
    int s = 1;
    while (s < 4 && tiles * s < 256 && K % (64 * 2 * s) == 0 && K / (2 * s) >= 128) s *= 2;
    return s;
  }
  // From 2048 rows the residual rows stay in the L2 of the XCD that owns them: the residual
  // product writes x back (EPI_RESID_KEEP), the row kernel works on the same XCD's eighth of the
  // rows and writes y back, and the next product reads its A rows there (measured: 1024 streams
  // 2.817 -> 2.700 ms per step, lookahead 4.353 -> 4.151 ms; at 512 rows, where the residual
  // products write split-K partials, 0.35% slower, so it stays off there).
  bool keep_rows() const { return M >= 2048; }
  void row_kernel(const ResLnArgs& r0) {
    ResLnArgs r = r0;
    r.keep = keep_rows();
    if (!launch_resid_ln(L, r, c->d.dt) && L.err == hipSuccess) L.err = hipErrorInvalidValue;
  }
  // cur += alpha (A W^T + bias), then cur = LN(cur; go, bo) when go, then y = LN(cur; gn, bn)
  // (y = cur when gn is null): split-K partials summed by the row kernel, or the product's
  // residual epilogue followed by the row kernel
  void resid_rows(const char* role, const void* A, int lda, const void* W, int K, float alpha, const float* bias,
                  const float* go, const float* bo, const float* gn, const float* bn, float* mean = nullptr) {
    const Dims& d = c->d;
    const int ks = ksplit_for(d.D, K);
    GemmArgs g{};
    g.M = M; g.N = d.D; g.K = K; g.A = A; g.W = W; g.amap = RowMap{INT_MAX, 0, lda};
    EpiArgs e = epi0();
    ResLnArgs r{};
    if (ks > 1) {
      e.kind = EPI_PART; e.out = c->P<void>(c->lay.part); e.ldo = d.D; e.pstride = (long)M * d.D;
      g.ksplit = ks;
      r.part = c->P<float>(c->lay.part); r.pstride = e.pstride; r.nparts = ks; r.bias = bias; r.alpha = alpha;
    } else {
      e.kind = keep_rows() ? EPI_RESID_KEEP : EPI_RESID; e.bias = bias; e.out = cur; e.ldo = d.D; e.alpha = alpha;
    }
    g.epi = e;
    L.role = role;
    launch_gemm(L, g, d.dt, 0);
    r.x = cur; r.go = go; r.bo = bo; r.gn = gn; r.bn = bn; r.y = c->P<void>(c->lay.y); r.M = M; r.D = d.D;
    r.mean = mean;
    L.role = role;
    row_kernel(r);
  }

  // The LayerNorms before qkv, pw1 and FF2 up ride on the products (bf16 weights, from 2048
  // rows, where the residual products run without split-K), which drops the three row kernels
  // in front of them. The residual product before each (FF1 down, wo, pw2) updates x and also
  // writes, per row, the (mean, M2) of each 64-column tile and the row centred on a shift s (the
  // mean its previous statistics give) in bf16; the consumer multiplies those centred rows by
  // the gain-scaled weights and finishes the LayerNorm in its epilogue:
  //   LN(x) W^T + bias = rstd ((x - s) W'^T - (mean - s) c1) + c2.
  // Rounding x - s rather than x keeps the operand's rounding error relative to the row's
  // spread, as when the normalised row is rounded.
  bool ln_carry() const {
    const Dims& d = c->d;
    return row_kernels() && keep_rows() && ln_fold(d) && ksplit_for(d.D, d.D) == 1 && ksplit_for(d.D, d.F) == 1;
  }
  // x += alpha (A W^T + bias), its tile statistics into st, the rows centred on the shifts to y
  void resid_carry(const char* role, const void* A, int lda, const void* W, int K, float alpha, const float* bias,
                   float2* st, const float* shift) {
    const Dims& d = c->d;
    GemmArgs g{};
    g.M = M; g.N = d.D; g.K = K; g.A = A; g.W = W; g.amap = RowMap{INT_MAX, 0, lda};
    EpiArgs e = epi0();
    e.kind = EPI_RESID_LNS; e.bias = bias; e.out = cur; e.ldo = d.D; e.alpha = alpha;
    e.lns = st; e.lns_shift = shift; e.lns_ld = M; e.lns_ntl = d.D / 64; e.xc = c->P<void>(c->lay.y);
    g.epi = e;
    L.role = role;
    launch_gemm(L, g, d.dt, 0);
  }
  // The depthwise conv + SiLU runs in pw1's GLU epilogue (MFMA kernel) when the kernel size is
  // at most 9 (it reads 8 older ring rows), the frames per call are at most 64, and the conv
  // ring's byte offsets fit 31 bits; the streams whose rows cross a multiple of 64 rows (none
  // when the frames per call divide 64) are left to a small kernel after pw1. Measured at 1024
  // streams: the separate kernel cost ~7 us per layer.
  bool dw_in_pw1() const {
    const Dims& d = c->d;
    return !d.wq && d.K <= 9 && cv.nf <= 64 && d.D % 32 == 0 &&
           (double)d.S * d.Rc * d.D * d.esz < 2147483648.0 - 4096.0;
  }
  // a consumer of centred rows: LayerNorm finished from st (statistics) and shift; the rows'
  // means go to mean (the next residual product's shifts)
  EpiArgs carried(EpiArgs e, const float* c1, const float* c2, const float2* st, const float* shift, float* mean) const {
    e.kind |= EPI_LNC; e.bias = nullptr; e.lnc_c1 = c1; e.lnc_c2 = c2;
    e.lns = const_cast<float2*>(st); e.lns_shift = shift; e.lns_mean = mean; e.lns_ld = M; e.lns_ntl = c->d.D / 64;
    return e;
  }

  void layers() {
    const Dims& d = c->d;
    const LayerOff& lo = c->lay.lo;
    cur = c->P<float>(c->lay.x);
    float* other = c->P<float>(c->lay.x2);
    const bool fz = fused(), rk = row_kernels();
    const float *pre_g = nullptr, *pre_b = nullptr;  // previous block's ln_out (fused path)
    if (rk) {  // y = LN(x) for the first block's FF1
      const char* l0 = c->ws + c->lay.layers;
      ResLnArgs r{};
      r.x = cur; r.gn = (const float*)(l0 + lo.ln[0]); r.bn = (const float*)(l0 + lo.ln[1]);
      r.y = c->P<void>(c->lay.y); r.M = M; r.D = d.D;
      if (ln_carry()) r.mean = c->P<float>(c->lay.lnm_a);
      L.role = "ln_in";
      row_kernel(r);
    }
    for (int l = 0; l < d.L; ++l) {
      char* lb = c->ws + c->lay.layers + (size_t)l * lo.size;
      const size_t kvl = (size_t)d.S * d.H * d.R * d.hd * d.esz;
      char* kr = c->ws + c->lay.kring + l * kvl;
      char* vr = c->ws + c->lay.vring + l * kvl;
      char* cr = c->ws + c->lay.cring + (size_t)l * d.S * d.Rc * d.D * d.esz;
      if (rk) {
        rows_layer(l, lb, kr, vr, cr);
        continue;
      }
      auto F32 = [&](size_t off) { return (const float*)(lb + off); };
      auto gemm_x = [&](const float* lng, const float* lnb, const void* W, int N, const EpiArgs& e, bool with_pre) {
        GemmArgs g{};
        g.M = M; g.N = N; g.K = d.D; g.W = W; g.epi = e;
        g.A = cur; g.amap = RowMap{INT_MAX, 0, d.D};
        g.a_f32 = 1; g.ln_g = lng; g.ln_b = lnb; g.a_scratch = c->P<void>(c->lay.y);
        if (with_pre) { g.pre_g = pre_g; g.pre_b = pre_b; }
        launch_gemm(L, g, wdt(), 0);
      };
      auto resid = [&](float alpha, const float* bias) {
        EpiArgs e = epi0();
        e.kind = EPI_RESID; e.bias = bias; e.out = cur; e.ldo = d.D; e.alpha = alpha;
        return e;
      };
      // ---- FF1 (macaron half step)
      {
        EpiArgs up = epi0();
        up.kind = EPI_SILU; up.bias = F32(lo.b_ff1_1); up.out = c->P<void>(c->lay.h); up.ldo = d.F;
        L.role = "ff1_up";
        gemm_x(F32(lo.ln[0]), F32(lo.ln[1]), lb + lo.w_ff1_1, d.F, up, fz);
        EpiArgs dn = resid(0.5f, F32(lo.b_ff1_2));
        GemmArgs g{};
        g.M = M; g.N = d.D; g.K = d.F; g.W = lb + lo.w_ff1_2;
        g.A = c->P<void>(c->lay.h); g.amap = RowMap{INT_MAX, 0, d.F};
        if (fz) {  // out = ln_out_prev(cur) + 1/2 FF(...) into the other buffer
          dn.out = other;
          g.res_src = cur; g.res_g = pre_g; g.res_b = pre_b;
        }
        g.epi = dn;
        L.role = "ff1_down";
        launch_gemm(L, g, wdt(), 0);
        if (fz) std::swap(cur, other);
      }
      // ---- MHSA: q to a buffer, k and v straight into the ring slots of their positions
      EpiArgs qkv = epi0();
      qkv.kind = EPI_QKV; qkv.bias = F32(lo.b_qkv); qkv.qbuf = c->P<float>(c->lay.q);
      qkv.kring = kr; qkv.vring = vr;
      L.role = "qkv";
      gemm_x(F32(lo.ln[2]), F32(lo.ln[3]), lb + lo.w_qkv, 3 * d.D, qkv, false);
      attention(l, lb, kr, vr);
      L.role = "wo";
      gemm_plain(c->P<void>(c->lay.o), d.D, lb + lo.w_o, d.D, d.D, resid(1.0f, F32(lo.b_o)));
      // ---- conv module: LN -> pw1 -> GLU into the ring; depthwise + SiLU; pw2 + residual
      EpiArgs glu = epi0();
      glu.kind = EPI_GLU; glu.bias = F32(lo.b_pw1); glu.cring = cr;
      // two rows: the depthwise conv + SiLU runs in pw1's epilogue (the rows of the call sit on
      // neighbouring lanes there), pw2 reads its output as a plain operand
      GemmArgs pw1{};
      pw1.M = M; pw1.N = 2 * d.D; pw1.K = d.D; pw1.W = lb + lo.w_pw1;
      pw1.A = cur; pw1.amap = RowMap{INT_MAX, 0, d.D};
      pw1.a_f32 = 1; pw1.ln_g = F32(lo.ln[4]); pw1.ln_b = F32(lo.ln[5]); pw1.a_scratch = c->P<void>(c->lay.y);
      pw1.epi = glu;
      pw1.epi.kind = EPI_GLU_DW; pw1.epi.out = c->P<void>(c->lay.e); pw1.epi.ldo = d.D;
      pw1.dw_w = F32(lo.dw_w); pw1.dw_b = F32(lo.b_dw); pw1.dw_taps = d.K; pw1.dw_Rc = d.Rc;
      L.role = "pw1";
      if (fz && rowdot_supported(pw1, wdt())) {
        launch_gemm(L, pw1, wdt(), 0);
        L.role = "pw2";
        gemm_plain(c->P<void>(c->lay.e), d.D, lb + lo.w_pw2, d.D, d.D, resid(1.0f, F32(lo.b_pw2)));
      } else if (fz) {
        gemm_x(F32(lo.ln[4]), F32(lo.ln[5]), lb + lo.w_pw1, 2 * d.D, glu, false);
        GemmArgs g{};
        g.M = M; g.N = d.D; g.K = d.D; g.W = lb + lo.w_pw2; g.epi = resid(1.0f, F32(lo.b_pw2));
        g.a_dw = 1; g.dw_ring = cr; g.dw_w = F32(lo.dw_w); g.dw_b = F32(lo.b_dw); g.dw_taps = d.K; g.dw_Rc = d.Rc;
        g.amap = RowMap{INT_MAX, 0, d.D};
        L.role = "pw2";
        launch_gemm(L, g, wdt(), 0);
      } else {
        gemm_x(F32(lo.ln[4]), F32(lo.ln[5]), lb + lo.w_pw1, 2 * d.D, glu, false);
        DwArgs dw{cv, cr, F32(lo.dw_w), F32(lo.b_dw), c->P<void>(c->lay.e), d.D, d.K, d.Rc};
        L.tag("dwconv", (double)cv.n_streams * (d.Kc + cv.nf) * d.D * d.esz, 2.0 * d.K * d.D * M);
        launch_dwconv(L, dw, d.dt);
        L.role = "pw2";
        gemm_plain(c->P<void>(c->lay.e), d.D, lb + lo.w_pw2, d.D, d.D, resid(1.0f, F32(lo.b_pw2)));
      }
      // ---- FF2 (macaron half step)
      {
        EpiArgs up = epi0();
        up.kind = EPI_SILU; up.bias = F32(lo.b_ff2_1); up.out = c->P<void>(c->lay.h); up.ldo = d.F;
        L.role = "ff2_up";
        gemm_x(F32(lo.ln[6]), F32(lo.ln[7]), lb + lo.w_ff2_1, d.F, up, false);
        L.role = "ff2_down";
        gemm_plain(c->P<void>(c->lay.h), d.F, lb + lo.w_ff2_2, d.D, d.F, resid(0.5f, F32(lo.b_ff2_2)));
      }
      // ---- the block's own LayerNorm: in place, or left to the consumers (fused path)
      if (fz) {
        pre_g = F32(lo.ln[8]); pre_b = F32(lo.ln[9]);
      } else {
        LnArgs lo_out{cur, cur, F32(lo.ln[8]), F32(lo.ln[9]), M, d.D, 1};
        launch_ln(L, lo_out, d.dt);
      }
    }
    last_g = pre_g; last_b = pre_b;
    rows_y = rk;
  }
  const float *last_g = nullptr, *last_b = nullptr;  // ln_out still to apply (fused path)
  bool rows_y = false;  // y holds the final rows in the compute dtype (row-kernel path)

  // rel-pos attention of layer l over the rings (q rows in q, output rows to o)
  void attention(int l, const char* lb, char* kr, char* vr) {
    const Dims& d = c->d;
    const LayerOff& lo = c->lay.lo;
    AttnArgs at{};
    at.cv = cv; at.q = c->P<float>(c->lay.q); at.kring = kr; at.vring = vr;
    at.posproj = c->P<float>(c->lay.posproj) + (size_t)l * d.H * d.nrel * d.hd;
    if (d.dt == CAC_BF16) at.posproj_bf = c->P<bf16_t>(c->lay.posproj_bf) + (size_t)l * d.H * d.nrel * d.hd;
    at.pos_u = (const float*)(lb + lo.pos_u); at.pos_v = (const float*)(lb + lo.pos_v);
    at.o = c->P<void>(c->lay.o);
    at.D = d.D; at.H = d.H; at.R = d.R; at.Lc = d.Lc; at.chunk = d.c; at.right = d.right;
    at.lookahead = d.lookahead; at.rel_lo = d.rel_lo; at.nrel = d.nrel;
    at.scale = 1.0f / sqrtf((float)d.hd);
    const double nrows = (double)cv.n_streams * cv.nf;
    const double bytes = kv_rows * 2.0 * d.D * d.esz + (double)d.H * d.nrel * d.hd * 4.0;
    const double flops = 6.0 * nrows * (kv_rows / cv.n_streams) * d.D;
    L.tag("attention", bytes, flops);
    L.tag_kv(kv_rows, 2.0 * d.D * d.esz, 6.0 * cv.nf * d.D);
    launch_attention(L, at, d.dt, d.hd);
  }

  // One Conformer block on the row-kernel path: on entry y holds LN_ff1(cur); every product
  // reads y (or h, o, e) as plain rows and every residual product ends in the row kernel that
  // writes the next LayerNorm'ed operand; the last one applies the block's ln_out to cur and
  // writes the next block's FF1 operand (after the last block: y = cur rounded, for the joint).
  void rows_layer(int l, const char* lb, char* kr, char* vr, char* cr) {
    const Dims& d = c->d;
    const LayerOff& lo = c->lay.lo;
    auto F32 = [&](size_t off) { return (const float*)(lb + off); };
    void* y = c->P<void>(c->lay.y);
    // with the LayerNorms carried: tile statistics sets sa / sb and row-mean sets ma / mb
    // alternate (on entry ma holds the row means the last row kernel wrote)
    const bool lc = ln_carry();
    float2* sa = lc ? c->P<float2>(c->lay.lns_a) : nullptr;
    float2* sb = lc ? c->P<float2>(c->lay.lns_b) : nullptr;
    float* ma = lc ? c->P<float>(c->lay.lnm_a) : nullptr;
    float* mb = lc ? c->P<float>(c->lay.lnm_b) : nullptr;
    // ---- FF1 (macaron half step)
    EpiArgs up = epi0();
    up.kind = EPI_SILU; up.bias = F32(lo.b_ff1_1); up.out = c->P<void>(c->lay.h); up.ldo = d.F;
    // the hidden rows stay in L2 for FF down from 4096 rows on, where FF down is bound by reading
    // them and its tiles run the same rows on the same XCD (measured: lookahead workload, 5120
    // rows, 4.49 -> 4.34 ms per step; at 2048 rows the write-back cost FF up 1% of the step)
    if (M >= 4096) up.kind = EPI_SILU_KEEP;
    L.role = "ff1_up";
    gemm_plain(y, d.D, lb + lo.w_ff1_1, d.F, d.D, up);
    if (lc) resid_carry("ff1_down", c->P<void>(c->lay.h), d.F, lb + lo.w_ff1_2, d.F, 0.5f, F32(lo.b_ff1_2), sb, ma);
    else resid_rows("ff1_down", c->P<void>(c->lay.h), d.F, lb + lo.w_ff1_2, d.F, 0.5f, F32(lo.b_ff1_2), nullptr, nullptr,
                    F32(lo.ln[2]), F32(lo.ln[3]));
    // ---- MHSA
    EpiArgs qkv = epi0();
    qkv.kind = EPI_QKV; qkv.bias = F32(lo.b_qkv); qkv.qbuf = c->P<float>(c->lay.q);
    qkv.kring = kr; qkv.vring = vr;
    L.role = "qkv";
    if (lc) gemm_plain(y, d.D, lb + lo.wg_qkv, 3 * d.D, d.D, carried(qkv, F32(lo.c1_qkv), F32(lo.c2_qkv), sb, ma, mb));
    else gemm_plain(y, d.D, lb + lo.w_qkv, 3 * d.D, d.D, qkv);
    attention(l, lb, kr, vr);
    if (lc) resid_carry("wo", c->P<void>(c->lay.o), d.D, lb + lo.w_o, d.D, 1.0f, F32(lo.b_o), sa, mb);
    else resid_rows("wo", c->P<void>(c->lay.o), d.D, lb + lo.w_o, d.D, 1.0f, F32(lo.b_o), nullptr, nullptr, F32(lo.ln[4]),
                    F32(lo.ln[5]));
    // ---- conv module: pw1 -> GLU into the ring; depthwise + SiLU (in pw1's epilogue, or its own
    // kernel); pw2
    const bool dwf = dw_in_pw1();
    EpiArgs glu = epi0();
    glu.kind = dwf ? EPI_GLU_DW : EPI_GLU; glu.bias = F32(lo.b_pw1); glu.cring = cr;
    if (dwf) { glu.out = c->P<void>(c->lay.e); glu.ldo = d.D; }
    GemmArgs g1{};
    g1.M = M; g1.N = 2 * d.D; g1.K = d.D; g1.A = y; g1.amap = RowMap{INT_MAX, 0, d.D};
    g1.W = lb + (lc ? lo.wg_pw1 : lo.w_pw1);
    g1.epi = lc ? carried(glu, F32(lo.c1_pw1), F32(lo.c2_pw1), sa, mb, ma) : glu;
    g1.dw_w = F32(lo.dw_w); g1.dw_b = F32(lo.b_dw); g1.dw_taps = d.K; g1.dw_Rc = d.Rc;
    L.role = "pw1";
    launch_gemm(L, g1, wdt(), 0);
    DwArgs dw{cv, cr, F32(lo.dw_w), F32(lo.b_dw), c->P<void>(c->lay.e), d.D, d.K, d.Rc};
    if (!dwf) {
      L.tag("dwconv", (double)cv.n_streams * (d.Kc + cv.nf) * d.D * d.esz, 2.0 * d.K * d.D * M);
      launch_dwconv(L, dw, d.dt);
    } else if (64 % cv.nf) {  // the streams across 64-row boundaries
      const int nx = (M - 1) / 64;
      L.role = "dw_straddle";
      L.tag("dwconv", (double)nx * (d.Kc + cv.nf) * d.D * d.esz, 2.0 * d.K * d.D * nx * cv.nf);
      launch_dwconv_straddle(L, dw);
    }
    if (lc) resid_carry("pw2", c->P<void>(c->lay.e), d.D, lb + lo.w_pw2, d.D, 1.0f, F32(lo.b_pw2), sb, ma);
    else resid_rows("pw2", c->P<void>(c->lay.e), d.D, lb + lo.w_pw2, d.D, 1.0f, F32(lo.b_pw2), nullptr, nullptr,
                    F32(lo.ln[6]), F32(lo.ln[7]));
    // ---- FF2 (macaron half step), then ln_out
    up.bias = F32(lo.b_ff2_1);
    L.role = "ff2_up";
    if (lc) gemm_plain(y, d.D, lb + lo.wg_ff2, d.F, d.D, carried(up, F32(lo.c1_ff2), F32(lo.c2_ff2), sb, ma, mb));
    else gemm_plain(y, d.D, lb + lo.w_ff2_1, d.F, d.D, up);
    const bool last = l + 1 == d.L;
    const char* nb = lb + lo.size;  // next block's parameters
    resid_rows("ff2_down", c->P<void>(c->lay.h), d.F, lb + lo.w_ff2_2, d.F, 0.5f, F32(lo.b_ff2_2), F32(lo.ln[8]),
               F32(lo.ln[9]), last ? nullptr : (const float*)(nb + lo.ln[0]), last ? nullptr : (const float*)(nb + lo.ln[1]),
               lc && !last ? ma : nullptr);
  }

  // encoder-side joint projection of the rows picked by amap into d_out (rows remapped by omap)
  void joint(float* d_out, int rows, RowMap amap, const int32_t* omap, int ogroup, int ostride) {
    const Dims& d = c->d;
    if (d.P == 0) {
      if (last_g) {  // apply the last ln_out before handing out the hidden rows
        LnArgs ln{cur, cur, last_g, last_b, M, d.D, 1};
        launch_ln(L, ln, d.dt);
      }
      CopyRowsArgs cp{cur, amap, d_out, omap, ogroup, ostride, rows, d.D};
      launch_copy_rows(L, cp);
      return;
    }
    EpiArgs e = epi0();
    e.kind = EPI_F32; e.out = d_out; e.ldo = d.P; e.bias = c->P<float>(c->lay.bj);
    e.omap = omap; e.ogroup = ogroup; e.ostride = ostride;
    GemmArgs g{};
    g.M = rows; g.N = d.P; g.K = d.D; g.A = cur; g.amap = amap;
    g.W = c->P<void>(c->lay.wj); g.epi = e; g.a_f32 = 1; g.a_scratch = c->P<void>(c->lay.y);
    g.ln_g = last_g; g.ln_b = last_b;
    if (rows_y) {  // the last row kernel left y = cur in the compute dtype
      g.A = c->P<void>(c->lay.y);
      g.a_f32 = 0;
      g.a_scratch = nullptr;
    }
    L.role = "joint";
    launch_gemm(L, g, wdt(), 0);
  }
};

StateArgs state_args(cac_ctx* c, int n) {
  const Dims& d = c->d;
  const Layout& lay = c->lay;
  StateArgs sa{};
  sa.ids = c->P<int32_t>(lay.sids); sa.hpos = c->P<int32_t>(lay.spos); sa.hpend = c->P<int32_t>(lay.spend);
  sa.pos = c->P<int32_t>(lay.pos); sa.pend = c->P<int32_t>(lay.pend);
  sa.kring = c->ws + lay.kring; sa.vring = c->ws + lay.vring; sa.cring = c->ws + lay.cring;
  sa.tail = c->ws + lay.tail; sa.x0 = c->ws + lay.x0;
  sa.n = n; sa.S = d.S; sa.L = d.L; sa.D = d.D; sa.H = d.H; sa.hd = d.hd; sa.R = d.R; sa.Rc = d.Rc;
  sa.Lc = d.Lc; sa.Kc = d.Kc; sa.tail_rows = d.tail; sa.bins = d.bins; sa.nla = d.nla; sa.Rx = d.Rx;
  sa.state_floats = (long)state_floats(d);
  sa.dtype = d.dt; sa.poison = (d.flags & CAC_FLAG_POISON) ? 1 : 0;
  state_header(d, sa.hdr);
  return sa;
}

// An asynchronous device error left on the context's stream by earlier work is reported at the
// next call that enqueues work (the query does not wait for the stream).
int pending_error(cac_ctx* c) {
  if (c->dry) return CAC_OK;
  const hipError_t e = hipStreamQuery(c->stream);
  if (e == hipSuccess || e == hipErrorNotReady) return CAC_OK;
  return c->fail(CAC_EHIP, std::string("asynchronous device error from earlier work: ") + hipGetErrorString(e));
}

int finish(cac_ctx* c, Launcher& L, int ok_value) {
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  return ok_value;
}

}  // namespace

// =============================================================================== C ABI
extern "C" {

size_t cac_param_count(const cac_config* cfg) {
  Dims d;
  std::string why;
  return make_dims(cfg, d, why) ? param_count(d) : 0;
}

size_t cac_workspace_bytes(const cac_config* cfg) {
  Dims d;
  std::string why;
  return make_dims(cfg, d, why) ? make_layout(d).total : 0;
}

size_t cac_state_floats(const cac_config* cfg) {
  Dims d;
  std::string why;
  return make_dims(cfg, d, why) ? state_floats(d) : 0;
}

int32_t cac_state_header(const cac_config* cfg, uint32_t* h_out) {
  Dims d;
  std::string why;
  if (!h_out || !make_dims(cfg, d, why)) return CAC_EINVAL;
  state_header(d, h_out);
  return CAC_OK;
}

const char* cac_last_error(const cac_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_create_error.c_str();
}

int32_t cac_create_streams(const cac_config* cfg, const float* h_params, size_t n_params,
                           void* d_workspace, size_t ws_bytes, void* hip_stream, cac_ctx** out) {
  g_create_error.clear();
  if (!out) { g_create_error = "out is NULL"; return CAC_EINVAL; }
  *out = nullptr;
  Dims d;
  if (!make_dims(cfg, d, g_create_error)) return CAC_EINVAL;
  const size_t np = param_count(d);
  if (!h_params) { g_create_error = "parameter array is NULL"; return CAC_EINVAL; }
  if (n_params != np) {
    g_create_error = "expected " + std::to_string(np) + " parameters, got " + std::to_string(n_params);
    return CAC_EINVAL;
  }
  const bool dry = (d.flags & CAC_FLAG_DRY_RUN) != 0;
  Layout lay = make_layout(d);
  if (!dry) {
    if (!d_workspace) { g_create_error = "workspace is NULL"; return CAC_EINVAL; }
    if (((uintptr_t)d_workspace) & 255) { g_create_error = "workspace must be 256-byte aligned"; return CAC_EINVAL; }
    if (ws_bytes < lay.total) {
      g_create_error = "workspace too small: need " + std::to_string(lay.total) + " bytes";
      return CAC_ENOMEM;
    }
  }
  cac_ctx* c = new cac_ctx();
  c->d = d; c->lay = lay; c->ws = (char*)d_workspace; c->stream = (hipStream_t)hip_stream; c->dry = dry;
  c->hpos.assign(d.S, 0); c->hpend.assign(d.S, 0); c->flushed.assign(d.S, 0); c->stamp.assign(d.S, 0);
  if (dry) { *out = c; return CAC_OK; }

  kernels_init();
  // repack the parameters on the host, then one copy into the workspace
  std::vector<uint8_t> wbuf(lay.weights_end, 0);
  Packer pk{wbuf, d.dt, d.wq};
  const float* p = h_params;
  const size_t D = d.D, F = d.F;
  auto take = [&](size_t n) { const float* r = p; p += n; return r; };
  const bool lnw = ln_fold(d);
  for (int l = 0; l < d.L; ++l) {
    const size_t base = lay.layers + (size_t)l * lay.lo.size;
    const LayerOff& lo = lay.lo;
    auto ffp = [&](int lnidx, size_t b1, size_t b2, size_t w1, size_t w2) {
      pk.f32(base + lo.ln[lnidx], take(D), D); pk.f32(base + lo.ln[lnidx + 1], take(D), D);
      pk.rows = F; pk.transpose(base + w1, take(D * F), D, F); pk.f32(base + b1, take(F), F);
      pk.rows = D; pk.transpose(base + w2, take(F * D), F, D); pk.f32(base + b2, take(D), D);
    };
    ffp(0, lo.b_ff1_1, lo.b_ff1_2, lo.w_ff1_1, lo.w_ff1_2);
    const float* g_att = take(D);
    const float* b_att = take(D);
    pk.f32(base + lo.ln[2], g_att, D); pk.f32(base + lo.ln[3], b_att, D);
    pk.rows = 3 * D;
    for (int m = 0; m < 3; ++m) {  // wq, wk, wv stacked as rows of [3D][D]
      const float* w = take(D * D);
      const float* bias = take(D);
      pk.transpose(base + lo.w_qkv, w, D, D, (size_t)m * D);
      pk.f32(base + lo.b_qkv + (size_t)m * D * 4, bias, D);
      if (lnw)
        for (size_t n = 0; n < D; ++n)
          pk.ln_column(base + lo.wg_qkv, base + lo.c1_qkv, base + lo.c2_qkv, w, D, D, n, m * D + n, m * D + n, g_att,
                       b_att, bias[n]);
    }
    pk.rows = D; pk.transpose(base + lo.w_o, take(D * D), D, D); pk.f32(base + lo.b_o, take(D), D);
    pk.f32(base + lo.pos_u, take(D), D); pk.f32(base + lo.pos_v, take(D), D);
    pk.f32(base + lo.wpos, take(D * D), D * D);
    const float* g_conv = take(D);
    const float* b_conv = take(D);
    pk.f32(base + lo.ln[4], g_conv, D); pk.f32(base + lo.ln[5], b_conv, D);
    {  // pw1 [D][2D] -> GLU-packed rows: value channel c at glu_a_col(c), its gate 32 rows later
      const float* w = take(D * 2 * D);
      const float* bias = take(2 * D);
      pk.rows = 2 * D;
      for (size_t ch = 0; ch < D; ++ch) {
        const size_t ra = glu_a_col((int)ch), rb = ra + 32;
        pk.column(base + lo.w_pw1, w, D, 2 * D, ch, ra);
        pk.column(base + lo.w_pw1, w, D, 2 * D, D + ch, rb);
        if (lnw) {
          pk.ln_column(base + lo.wg_pw1, base + lo.c1_pw1, base + lo.c2_pw1, w, D, 2 * D, ch, ra, ch, g_conv, b_conv,
                       bias[ch]);
          pk.ln_column(base + lo.wg_pw1, base + lo.c1_pw1, base + lo.c2_pw1, w, D, 2 * D, D + ch, rb, D + ch, g_conv,
                       b_conv, bias[D + ch]);
        }
      }
      pk.f32(base + lo.b_pw1, bias, 2 * D);
    }
    {  // dw [D][K] -> taps [K][D]
      const float* w = take(D * d.K);
      float* dst = (float*)(wbuf.data() + base + lo.dw_w);
      for (size_t ch = 0; ch < D; ++ch)
        for (int k = 0; k < d.K; ++k) dst[(size_t)k * D + ch] = w[ch * d.K + k];
      pk.f32(base + lo.b_dw, take(D), D);
    }
    pk.rows = D; pk.transpose(base + lo.w_pw2, take(D * D), D, D); pk.f32(base + lo.b_pw2, take(D), D);
    if (lnw) {  // FF2 up with its LayerNorm folded in: its parameters come next in the array
      const float* g_ff2 = p;
      const float* b_ff2 = p + D;
      const float* w = p + 2 * D;
      const float* bias = w + D * F;
      for (size_t n = 0; n < F; ++n)
        pk.ln_column(base + lo.wg_ff2, base + lo.c1_ff2, base + lo.c2_ff2, w, D, F, n, n, n, g_ff2, b_ff2, bias[n]);
    }
    ffp(6, lo.b_ff2_1, lo.b_ff2_2, lo.w_ff2_1, lo.w_ff2_2);
    pk.f32(base + lo.ln[8], take(D), D); pk.f32(base + lo.ln[9], take(D), D);
  }
  if (d.P) {
    pk.rows = d.P;
    pk.transpose(lay.wj, take(D * d.P), D, d.P);
    pk.f32(lay.bj, take(d.P), d.P);
  }
  pk.wq = 0;  // the front end keeps the compute dtype
  if (d.fe == 2) {
    const size_t C = d.fc, F8 = d.bins / 8;
    auto taps = [&](size_t off) {  // [C][3][3] -> [9][C] float32
      const float* w = take(C * 9);
      float* dst = (float*)(wbuf.data() + off);
      for (size_t ch = 0; ch < C; ++ch)
        for (int tp = 0; tp < 9; ++tp) dst[tp * C + ch] = w[ch * 9 + tp];
    };
    taps(lay.f2_c1w); pk.f32(lay.f2_c1b, take(C), C);
    taps(lay.f2_dw2w); pk.f32(lay.f2_dw2b, take(C), C);
    {  // pointwise [out][in] is already [N][K]
      const float* w = take(C * C);
      for (size_t i = 0; i < C * C; ++i) pk.op(lay.f2_pw2w, i, w[i]);
      pk.f32(lay.f2_pw2b, take(C), C);
    }
    taps(lay.f2_dw3w); pk.f32(lay.f2_dw3b, take(C), C);
    {
      const float* w = take(C * C);
      for (size_t i = 0; i < C * C; ++i) pk.op(lay.f2_pw3w, i, w[i]);
      pk.f32(lay.f2_pw3b, take(C), C);
    }
    {  // lin [c * F8 + f][D] -> [D][f * C + c] (the maps are channels-last)
      const float* w = take(C * F8 * D);
      for (size_t ch = 0; ch < C; ++ch)
        for (size_t f = 0; f < F8; ++f)
          for (size_t o = 0; o < D; ++o) pk.op(lay.f2_linw, o * C * F8 + f * C + ch, w[(ch * F8 + f) * D + o]);
      pk.f32(lay.f2_linb, take(D), D);
    }
  }
  if (d.fe == 1) {  // conv [out][in][tap] -> [out][tap * in + c_in] (matches a window of 3 rows)
    const size_t cin[3] = {(size_t)d.bins, D, D};
    for (int i = 0; i < 3; ++i) {
      const float* w = take(D * cin[i] * 3);
      for (size_t o = 0; o < D; ++o)
        for (size_t ci = 0; ci < cin[i]; ++ci)
          for (int t = 0; t < 3; ++t) pk.op(lay.fe_w[i], o * 3 * cin[i] + t * cin[i] + ci, w[(o * cin[i] + ci) * 3 + t]);
      pk.f32(lay.fe_b[i], take(D), D);
    }
  }
  hipError_t e = hipMemcpyAsync(c->ws, wbuf.data(), wbuf.size(), hipMemcpyHostToDevice, c->stream);
  Launcher L;
  L.stream = c->stream;
  if (e == hipSuccess) {
    // the position tables read the float32 Wpos copy of every layer (strided by layer block)
    for (int l = 0; l < d.L && L.err == hipSuccess; ++l) {
      PosProjArgs pa{c->P<float>(lay.layers + (size_t)l * lay.lo.size + lay.lo.wpos),
                     c->P<float>(lay.posproj) + (size_t)l * d.H * d.nrel * d.hd, 1, d.D, d.H, d.hd, d.rel_lo, d.nrel};
      launch_posproj(L, pa);
    }
    if (d.dt == CAC_BF16) {
      CvtArgs cv{c->P<float>(lay.posproj), RowMap{INT_MAX, 0, d.hd}, c->ws + lay.posproj_bf, d.L * d.H * d.nrel, d.hd};
      launch_cvt(L, cv);
    }
    e = L.err;
  }
  std::vector<int32_t> all(d.S);
  for (int i = 0; i < d.S; ++i) all[i] = i;
  if (e == hipSuccess) {
    e = hipMemcpyAsync(c->ws + lay.sids, all.data(), (size_t)d.S * 4, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) {
      StateArgs sa = state_args(c, d.S);
      launch_state(L, sa, 0);
      e = L.err;
    }
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  }
  if (e != hipSuccess) {
    g_create_error = std::string("HIP error during create: ") + hipGetErrorString(e);
    delete c;
    return CAC_EHIP;
  }
  *out = c;
  return CAC_OK;
}


}  // extern "C"

namespace {

// The K/V rows a push's attention reads, summed over the streams that run a pass: each one's
// cache fill before the push plus the rows the pass computes (host positions, before the push
// commits them).
double call_kv_rows(const cac_ctx* c, int n, const int32_t* ids, int n_frames, const std::vector<int32_t>& cids) {
  const Dims& d = c->d;
  double kvr = 0;
  if (!d.lookahead)
    for (int i = 0; i < n; ++i) kvr += std::min(c->hpos[ids[i]], d.Lc) + n_frames;
  else
    for (int id : cids) kvr += std::min(c->hpos[id], d.Lc) + d.nc;
  return kvr;
}

// Everything one push enqueues after the id lists are on the device.
void enqueue_push(cac_ctx* c, Launcher& L, int n, const int32_t* ids, int n_frames, const void* d_input, float* d_out,
                  const std::vector<int32_t>& cids) {
  const Dims& d = c->d;
  const int32_t* dids = c->P<int32_t>(c->lay.ids);
  int32_t* dpos = c->P<int32_t>(c->lay.pos);
  int32_t* dpend = c->P<int32_t>(c->lay.pend);
  if (!d.lookahead) {
    CallView cv{dids, dpos, n_frames, n, c->P<int32_t>(c->lay.cpos)};
    const int M = n * n_frames;
    if (d.fe == 2) {
      FeWindowArgs fw{cv, d_input, c->ws + c->lay.tail, c->ws + c->lay.win, d.bins, d.tail, d.mpc};
      launch_fe_window(L, fw, d.dt);
      // stage 1 (11 rows: positions 8c-6 .. 8c+4 of the chunk's subsampled-by-2 grid; the first
      // 6 lie before a fresh stream's start), then depthwise + pointwise twice (5 rows, 2 of
      // them before the start; 2 rows), then the projection of each frame's C x F/8 map
      const int C = d.fc, B = d.bins, wrows = d.tail + d.mpc;
      // stage 1 and the first depthwise stage in one launch where the stage-1 map fits on chip
      Fe2dS1DwArgs sd{cv, c->ws + c->lay.win, c->ws + c->lay.f2_d2, c->P<float>(c->lay.f2_c1w), c->P<float>(c->lay.f2_c1b),
                      c->P<float>(c->lay.f2_dw2w), c->P<float>(c->lay.f2_dw2b), wrows, B, 11, B / 2, 5, B / 4, C, 6};
      const bool s1dw = launch_fe2d_s1dw(L, sd);
      if (!s1dw) {
        Fe2dArgs s1{cv, c->ws + c->lay.win, c->ws + c->lay.f2_a1, c->P<float>(c->lay.f2_c1w), c->P<float>(c->lay.f2_c1b),
                    wrows, B, 11, B / 2, C, 1, 6};
        launch_fe2d(L, s1);
      }
      struct { size_t in, dw, dwb, mid, pw, pwb, out; int Tin, Fin, Tout, Fout, neg; const char* role; } st2[2] = {
          {c->lay.f2_a1, c->lay.f2_dw2w, c->lay.f2_dw2b, c->lay.f2_d2, c->lay.f2_pw2w, c->lay.f2_pw2b, c->lay.f2_a2, 11, B / 2, 5,
           B / 4, 2, "fe2d_pw2"},
          {c->lay.f2_a2, c->lay.f2_dw3w, c->lay.f2_dw3b, c->lay.f2_d3, c->lay.f2_pw3w, c->lay.f2_pw3b, c->lay.f2_a3, 5, B / 4, 2,
           B / 8, 0, "fe2d_pw3"}};
      for (int i = 0; i < 2; ++i) {
        Fe2dArgs dw{cv, c->ws + st2[i].in, c->ws + st2[i].mid, c->P<float>(st2[i].dw), c->P<float>(st2[i].dwb),
                    st2[i].Tin, st2[i].Fin, st2[i].Tout, st2[i].Fout, C, 0, 0};
        if (i > 0 || !s1dw) launch_fe2d(L, dw);
        EpiArgs e{};
        e.cv = cv; e.bias = c->P<float>(st2[i].pwb);
        e.kind = EPI_RELU_FE; e.out = c->ws + st2[i].out; e.ldo = C;
        e.fe_rows_per_stream = st2[i].Tout * st2[i].Fout; e.fe_neg_rows = st2[i].neg * st2[i].Fout;
        GemmArgs g{};
        g.M = n * st2[i].Tout * st2[i].Fout; g.N = C; g.K = C; g.A = c->ws + st2[i].mid; g.amap = RowMap{INT_MAX, 0, C};
        g.W = c->ws + st2[i].pw; g.epi = e;
        L.role = st2[i].role;
        launch_gemm(L, g, d.dt, 0);
      }
      EpiArgs e{};
      e.cv = cv; e.bias = c->P<float>(c->lay.f2_linb); e.kind = EPI_F32; e.out = c->ws + c->lay.x; e.ldo = d.D;
      GemmArgs g{};
      const int K8 = C * (B / 8);
      g.M = n * 2; g.N = d.D; g.K = K8; g.A = c->ws + c->lay.f2_a3; g.amap = RowMap{INT_MAX, 0, K8};
      g.W = c->ws + c->lay.f2_linw; g.epi = e;
      L.role = "fe2d_lin";
      launch_gemm(L, g, d.dt, 0);
    } else if (d.fe) {
      FeWindowArgs fw{cv, d_input, c->ws + c->lay.tail, c->ws + c->lay.win, d.bins, d.tail, d.mpc};
      launch_fe_window(L, fw, d.dt);
      const int wrows = d.tail + d.mpc;
      struct { int rows, neg; size_t in, out; int K; RowMap m; } st3[3] = {
          {11, 6, c->lay.win, c->lay.fe1, 3 * d.bins, RowMap{11, wrows * d.bins, 2 * d.bins}},
          {5, 2, c->lay.fe1, c->lay.fe2, 3 * d.D, RowMap{5, 11 * d.D, 2 * d.D}},
          {2, 0, c->lay.fe2, c->lay.x, 3 * d.D, RowMap{2, 5 * d.D, 2 * d.D}}};
      for (int i = 0; i < 3; ++i) {
        EpiArgs e{};
        e.cv = cv; e.bias = c->P<float>(c->lay.fe_b[i]);
        if (i < 2) { e.kind = EPI_RELU_FE; e.out = c->ws + st3[i].out; e.ldo = d.D; e.fe_rows_per_stream = st3[i].rows; e.fe_neg_rows = st3[i].neg; }
        else { e.kind = EPI_F32; e.out = c->ws + c->lay.x; e.ldo = d.D; }
        GemmArgs g{};
        g.M = n * st3[i].rows; g.N = d.D; g.K = st3[i].K; g.A = c->ws + st3[i].in; g.amap = st3[i].m;
        g.W = c->ws + c->lay.fe_w[i]; g.epi = e;
        L.role = i == 0 ? "fe_conv1" : (i == 1 ? "fe_conv2" : "fe_conv3");
        launch_gemm(L, g, d.dt, 0);
      }
    } else {  // the input kernel also advances the positions (every later kernel reads cpos)
      InputArgs ia{cv, d_input, c->P<float>(c->lay.x), M, d.D, dpos, n_frames};
      launch_input(L, ia, d.dt);
    }
    Pass ps{c, L, cv, M, call_kv_rows(c, n, ids, n_frames, cids)};
    ps.layers();
    ps.joint(d_out, M, RowMap{INT_MAX, 0, d.D}, nullptr, 1, 0);
    if (d.fe) {  // the front-end window kernel reads the positions from every thread of a stream
      AdvanceArgs ad{dids, dpos, dpend, n, n_frames, 0};
      launch_advance(L, ad);
    }
  } else {
    CallView pv{dids, dpos, d.ne, n, c->P<int32_t>(c->lay.cpos)};
    LaStoreArgs ls{pv, dpend, d_input, c->ws + c->lay.x0, d.D, d.Rx};
    launch_la_store(L, ls, d.dt);
    AdvanceArgs a1{dids, dpos, dpend, n, 0, d.ne};
    launch_advance(L, a1);
    const int nC = (int)cids.size();
    if (nC > 0) {
      const int32_t* dcids = c->P<int32_t>(c->lay.cids);
      CallView cv{dcids, dpos, d.nc, nC, c->P<int32_t>(c->lay.ccpos)};
      LaGatherArgs lg{cv, c->ws + c->lay.x0, c->P<float>(c->lay.x), d.D, d.Rx};
      launch_la_gather(L, lg, d.dt);
      Pass ps{c, L, cv, nC * d.nc, call_kv_rows(c, n, ids, n_frames, cids)};
      ps.layers();
      ps.joint(d_out, nC * d.ne, RowMap{d.ne, d.nc * d.D, d.D}, c->P<int32_t>(c->lay.cidx), d.ne, d.ne);
      AdvanceArgs a2{dcids, dpos, dpend, nC, d.ne, -d.ne};
      launch_advance(L, a2);
    }
  }
}

// Offsets of 8-byte fields holding exactly the value p.
std::vector<size_t> find_ptr(const std::vector<char>& args, const void* p) {
  std::vector<size_t> offs;
  const uint64_t v = (uint64_t)(uintptr_t)p;
  for (size_t o = 0; o + 8 <= args.size(); o += 8) {
    uint64_t w;
    memcpy(&w, args.data() + o, 8);
    if (w == v) offs.push_back(o);
  }
  return offs;
}

// Replay the recorded graph of this call shape (recording it on first use), re-pointing the
// nodes that hold the caller's input and output pointers.
hipError_t push_graph(cac_ctx* c, int n, const int32_t* ids, int n_frames, const void* d_input, float* d_out,
                      const std::vector<int32_t>& cids) {
  // 21 bits per field: stream counts up to 2^20 (make_dims' limit), frames up to 16
  const uint64_t key = ((uint64_t)n << 42) | ((uint64_t)n_frames << 21) | (uint64_t)cids.size();
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    cac_ctx::Graph gr;
    hipError_t e = hipGraphCreate(&gr.g, 0);
    if (e != hipSuccess) return e;
    Launcher L;
    L.stream = c->stream;
    L.graph = gr.g;
    L.rec = &gr.nodes;
    enqueue_push(c, L, n, ids, n_frames, d_input, d_out, cids);
    if (L.err != hipSuccess) { (void)hipGraphDestroy(gr.g); return L.err; }
    e = hipGraphInstantiate(&gr.exec, gr.g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(gr.g); return e; }
    for (const NodeRec& r : gr.nodes) {
      gr.in_offs.push_back(find_ptr(r.args, d_input));
      gr.out_offs.push_back(find_ptr(r.args, d_out));
    }
    gr.in = d_input;
    gr.out = d_out;
    it = c->graphs.emplace(key, std::move(gr)).first;
  }
  cac_ctx::Graph& gr = it->second;
  c->last_graph = &gr;
  // the nodes' algorithmic work as of this push (attention's grows with the cache fill, which
  // differs from the push that recorded the graph)
  const double kvr = call_kv_rows(c, n, ids, n_frames, cids);
  for (NodeRec& r : gr.nodes)
    if (r.kv_bytes > 0.0 || r.kv_flops > 0.0) {
      r.bytes += (kvr - r.kv_rows) * r.kv_bytes;
      r.flops += (kvr - r.kv_rows) * r.kv_flops;
      r.kv_rows = kvr;
    }
  if (gr.in != d_input || gr.out != d_out) {
    for (size_t i = 0; i < gr.nodes.size(); ++i) {
      if (gr.in_offs[i].empty() && gr.out_offs[i].empty()) continue;
      NodeRec& r = gr.nodes[i];
      for (size_t o : gr.in_offs[i]) memcpy(r.args.data() + o, &d_input, 8);
      for (size_t o : gr.out_offs[i]) memcpy(r.args.data() + o, &d_out, 8);
      hipKernelNodeParams p = r.p;
      void* kp[1] = {r.args.data()};
      p.kernelParams = kp;
      hipError_t e = hipGraphExecKernelNodeSetParams(gr.exec, r.node, &p);
      if (e != hipSuccess) return e;
    }
    gr.in = d_input;
    gr.out = d_out;
  }
  return hipGraphLaunch(gr.exec, c->stream);
}

}  // namespace

extern "C" {

int32_t cac_push_chunk(cac_ctx* c, int32_t n, const int32_t* ids, int32_t n_frames, const void* d_input,
                       float* d_out, int32_t* h_emitted) {
  if (!c) return CAC_EINVAL;
  const Dims& d = c->d;
  int rc = check_ids(c, n, ids, true);
  if (rc) return rc;
  if (d.lookahead) {
    if (n_frames != d.ne) return c->fail(CAC_EINVAL, "the lookahead variant takes n_emit frames per push");
  } else if (d.fe) {
    if (n_frames != 2) return c->fail(CAC_EINVAL, "with the front end a push is one 16-frame mel chunk (2 frames)");
  } else if (n_frames < d.c || n_frames > d.npush || n_frames % d.c) {
    return c->fail(CAC_EINVAL, "n_frames must be a multiple of att_chunk in [att_chunk, max_push_frames]");
  }
  if (!d_input || !d_out) return c->fail(CAC_EINVAL, "input or output pointer is NULL");
  if ((const void*)d_out == d_input) return c->fail(CAC_EINVAL, "input and output must be different buffers");
  if (d.wq && (long)n * n_frames > 2) return c->fail(CAC_EINVAL, "with int8 weights a push carries at most 2 rows (streams x frames)");
  if ((rc = pending_error(c))) return rc;

  // host bookkeeping decides who runs a pass (lookahead: streams whose pending frames reach
  // n_emit + n_lookahead after this push)
  std::vector<int32_t> cids, cidx;
  if (d.lookahead) {
    for (int i = 0; i < n; ++i)
      if (c->hpend[ids[i]] + d.ne >= d.nc) { cids.push_back(ids[i]); cidx.push_back(i); }
  }
  const int emitted = d.lookahead ? (cids.empty() ? 0 : d.ne) : n_frames;
  auto commit = [&]() {
    for (int i = 0; i < n; ++i) {
      const int id = ids[i];
      if (d.lookahead) c->hpend[id] += d.ne;
      else c->hpos[id] += n_frames;
      if (h_emitted) h_emitted[i] = 0;
    }
    if (d.lookahead) {
      for (size_t j = 0; j < cids.size(); ++j) {
        c->hpos[cids[j]] += d.ne;
        c->hpend[cids[j]] -= d.ne;
        if (h_emitted) h_emitted[cidx[j]] = d.ne;
      }
    } else if (h_emitted) {
      for (int i = 0; i < n; ++i) h_emitted[i] = n_frames;
    }
  };
  if (c->dry) { commit(); return c->fail(CAC_ENODEV, "dry-run context: no device work"); }

  hipError_t e = upload(c, c->dev_ids, c->lay.ids, ids, n);
  if (e == hipSuccess && !cids.empty()) e = upload(c, c->dev_cids, c->lay.cids, cids.data(), (int)cids.size());
  if (e == hipSuccess && !cids.empty()) e = upload(c, c->dev_cidx, c->lay.cidx, cidx.data(), (int)cidx.size());
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("id upload failed: ") + hipGetErrorString(e));
  if (c->use_graph && !c->profiling) {
    e = push_graph(c, n, ids, n_frames, d_input, d_out, cids);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("graph replay failed: ") + hipGetErrorString(e));
    rc = emitted;
  } else {
    Launcher L;
    L.stream = c->stream;
    if (c->profiling) L.prof = &c->prof;
    enqueue_push(c, L, n, ids, n_frames, d_input, d_out, cids);
    rc = finish(c, L, emitted);
  }
  if (rc >= 0) commit();
  return rc;
}

int32_t cac_set_graph(cac_ctx* c, int32_t enable) {
  if (!c) return CAC_EINVAL;
  c->use_graph = enable != 0;
  return CAC_OK;
}

int32_t cac_reset_stream(cac_ctx* c, int32_t n, const int32_t* ids) {
  if (!c) return CAC_EINVAL;
  int rc = check_ids(c, n, ids, false);
  if (rc) return rc;
  if (!c->dry) {
    Launcher L;
    L.stream = c->stream;
    L.err = hipMemcpyAsync(c->ws + c->lay.sids, ids, (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
    StateArgs sa = state_args(c, n);
    launch_state(L, sa, 0);
    rc = finish(c, L, n);
    if (rc < 0) return rc;
  }
  for (int i = 0; i < n; ++i) { c->hpos[ids[i]] = 0; c->hpend[ids[i]] = 0; c->flushed[ids[i]] = 0; }
  return c->dry ? c->fail(CAC_ENODEV, "dry-run context: no device work") : n;
}

int32_t cac_flush(cac_ctx* c, int32_t n, const int32_t* ids, float* d_out, int32_t* h_frames_out) {
  if (!c) return CAC_EINVAL;
  const Dims& d = c->d;
  int rc = check_ids(c, n, ids, true);
  if (rc) return rc;
  int maxm = 0;
  if (d.lookahead)
    for (int i = 0; i < n; ++i) maxm = std::max(maxm, c->hpend[ids[i]]);
  if (maxm > 0 && !d_out) return c->fail(CAC_EINVAL, "output pointer is NULL");
  if ((rc = pending_error(c))) return rc;
  auto commit = [&]() {
    for (int i = 0; i < n; ++i) {
      const int id = ids[i];
      if (h_frames_out) h_frames_out[i] = d.lookahead ? c->hpend[id] : 0;
      if (d.lookahead) { c->hpos[id] += c->hpend[id]; c->hpend[id] = 0; }
      c->flushed[id] = 1;
    }
  };
  if (c->dry || maxm == 0) {
    commit();
    return c->dry ? c->fail(CAC_ENODEV, "dry-run context: no device work") : 0;
  }
  Launcher L;
  L.stream = c->stream;
  if (c->profiling) L.prof = &c->prof;
  // one final pass per distinct pending count; pending frames see keys up to their own end
  for (int m = 1; m <= d.nla && L.err == hipSuccess; ++m) {
    std::vector<int32_t> cids, cidx;
    for (int i = 0; i < n; ++i)
      if (c->hpend[ids[i]] == m) { cids.push_back(ids[i]); cidx.push_back(i); }
    if (cids.empty()) continue;
    const int nC = (int)cids.size();
    L.err = upload(c, c->dev_cids, c->lay.cids, cids.data(), nC);
    if (L.err == hipSuccess) L.err = upload(c, c->dev_cidx, c->lay.cidx, cidx.data(), nC);
    const int32_t* dcids = c->P<int32_t>(c->lay.cids);
    int32_t* dpos = c->P<int32_t>(c->lay.pos);
    CallView cv{dcids, dpos, m, nC, c->P<int32_t>(c->lay.ccpos)};
    LaGatherArgs lg{cv, c->ws + c->lay.x0, c->P<float>(c->lay.x), d.D, d.Rx};
    launch_la_gather(L, lg, d.dt);
    double kvr = 0;
    for (int id : cids) kvr += std::min(c->hpos[id], d.Lc) + m;
    Pass ps{c, L, cv, nC * m, kvr};
    ps.layers();
    ps.joint(d_out, nC * m, RowMap{INT_MAX, 0, d.D}, c->P<int32_t>(c->lay.cidx), m, d.nla);
    AdvanceArgs ad{dcids, dpos, c->P<int32_t>(c->lay.pend), nC, m, -m};
    launch_advance(L, ad);
    // the cached id lists must not be reused by a later push with stale contents
  }
  rc = finish(c, L, maxm);
  if (rc >= 0) commit();
  return rc;
}

int32_t cac_export_state(cac_ctx* c, int32_t n, const int32_t* ids, int32_t* h_pos, int32_t* h_pending, float* d_state) {
  if (!c) return CAC_EINVAL;
  int rc = check_ids(c, n, ids, false);
  if (rc) return rc;
  if (!h_pos || !d_state) return c->fail(CAC_EINVAL, "position or state pointer is NULL");
  if (c->d.lookahead && !h_pending) return c->fail(CAC_EINVAL, "pending pointer is NULL");
  std::vector<int32_t> pos(n), pend(n);
  for (int i = 0; i < n; ++i) { pos[i] = c->hpos[ids[i]]; pend[i] = c->hpend[ids[i]]; }
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  Launcher L;
  L.stream = c->stream;
  L.err = hipMemcpyAsync(c->ws + c->lay.sids, ids, (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  if (L.err == hipSuccess) L.err = hipMemcpyAsync(c->ws + c->lay.spos, pos.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  if (L.err == hipSuccess) L.err = hipMemcpyAsync(c->ws + c->lay.spend, pend.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  StateArgs sa = state_args(c, n);
  sa.blob = d_state;
  launch_state(L, sa, 2);
  if (L.err == hipSuccess) L.err = hipStreamSynchronize(c->stream);
  rc = finish(c, L, n);
  if (rc < 0) return rc;
  for (int i = 0; i < n; ++i) { h_pos[i] = pos[i]; if (h_pending) h_pending[i] = pend[i]; }
  return n;
}

int32_t cac_import_state(cac_ctx* c, int32_t n, const int32_t* ids, const int32_t* h_pos, const int32_t* h_pending, const float* d_state) {
  if (!c) return CAC_EINVAL;
  const Dims& d = c->d;
  int rc = check_ids(c, n, ids, false);
  if (rc) return rc;
  if (!h_pos || !d_state) return c->fail(CAC_EINVAL, "position or state pointer is NULL");
  std::vector<int32_t> pend(n, 0);
  for (int i = 0; i < n; ++i) {
    if (h_pos[i] < 0) return c->fail(CAC_ESTATE, "negative stream position");
    if (!d.lookahead && h_pos[i] % d.c) return c->fail(CAC_ESTATE, "stream position off the attention chunk grid");
    if (d.lookahead) {
      if (!h_pending) return c->fail(CAC_EINVAL, "pending pointer is NULL");
      if (h_pending[i] < 0 || h_pending[i] > d.nla) return c->fail(CAC_ESTATE, "pending count out of [0, n_lookahead]");
      pend[i] = h_pending[i];
    }
  }
  // every stream's blob must carry this config's header (dry-run contexts read it from host
  // memory, since they make no device calls)
  const size_t sf = state_floats(d);
  std::vector<uint32_t> hdrs((size_t)n * STATE_HDR);
  if (c->dry) {
    for (int i = 0; i < n; ++i) memcpy(&hdrs[(size_t)i * STATE_HDR], d_state + (size_t)i * sf, STATE_HDR * 4);
  } else {
    hipError_t e = hipMemcpy2DAsync(hdrs.data(), STATE_HDR * 4, d_state, sf * 4, STATE_HDR * 4, n,
                                    hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("reading the state headers failed: ") + hipGetErrorString(e));
  }
  uint32_t want[STATE_HDR];
  state_header(d, want);
  for (int i = 0; i < n; ++i) {
    const uint32_t* h = &hdrs[(size_t)i * STATE_HDR];
    if (h[0] != want[0] || h[1] != want[1])
      return c->fail(CAC_ESTATE, "state blob " + std::to_string(i) + " has no state header of this layout version");
    if (h[2] != want[2] || h[3] != want[3])
      return c->fail(CAC_ESTATE, "state blob " + std::to_string(i) + " was made with a different config");
  }
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  Launcher L;
  L.stream = c->stream;
  L.err = hipMemcpyAsync(c->ws + c->lay.sids, ids, (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  if (L.err == hipSuccess) L.err = hipMemcpyAsync(c->ws + c->lay.spos, h_pos, (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  if (L.err == hipSuccess) L.err = hipMemcpyAsync(c->ws + c->lay.spend, pend.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  StateArgs sa = state_args(c, n);
  sa.blob = const_cast<float*>(d_state);
  launch_state(L, sa, 0);
  launch_state(L, sa, 1);
  if (L.err == hipSuccess) L.err = hipStreamSynchronize(c->stream);
  rc = finish(c, L, n);
  if (rc < 0) return rc;
  for (int i = 0; i < n; ++i) { c->hpos[ids[i]] = h_pos[i]; c->hpend[ids[i]] = pend[i]; c->flushed[ids[i]] = 0; }
  return n;
}

int32_t cac_stream_info(const cac_ctx* c, int32_t id, int32_t* pos, int32_t* pending, int32_t* flushed) {
  if (!c || id < 0 || id >= c->d.S) return CAC_EINVAL;
  if (pos) *pos = c->hpos[id];
  if (pending) *pending = c->hpend[id];
  if (flushed) *flushed = c->flushed[id];
  return CAC_OK;
}

int32_t cac_set_stream(cac_ctx* c, void* s) {
  if (!c) return CAC_EINVAL;
  c->stream = (hipStream_t)s;
  return CAC_OK;
}

int32_t cac_synchronize(cac_ctx* c) {
  if (!c) return CAC_EINVAL;
  if (c->dry) return CAC_OK;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("device error: ") + hipGetErrorString(e));
  return CAC_OK;
}

int32_t cac_profile(cac_ctx* c, int32_t enable) {
  if (!c) return CAC_EINVAL;
  if (enable) {
    c->prof.clear();
    c->profiling = true;
  } else {
    c->prof.drain();
    c->profiling = false;
  }
  return c->prof.err == hipSuccess ? CAC_OK : c->fail(CAC_EHIP, std::string("profiling: ") + hipGetErrorString(c->prof.err));
}

int32_t cac_profile_read(cac_ctx* c, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
                         double* total_ms, double* bytes, double* flops) {
  if (!c || max_entries < 0 || name_len < 1) return CAC_EINVAL;
  c->prof.drain();
  if (c->prof.err != hipSuccess) return c->fail(CAC_EHIP, std::string("profiling: ") + hipGetErrorString(c->prof.err));
  const int n = (int)c->prof.names.size();
  for (int i = 0; i < n && i < max_entries; ++i) {
    if (names) {
      strncpy(names + (size_t)i * name_len, c->prof.names[i].c_str(), name_len - 1);
      names[(size_t)i * name_len + name_len - 1] = 0;
    }
    if (launches) launches[i] = c->prof.launches[i];
    if (total_ms) total_ms[i] = c->prof.ms[i];
    if (bytes) bytes[i] = c->prof.bytes[i];
    if (flops) flops[i] = c->prof.flops[i];
  }
  return n;
}

int32_t cac_profile_replay(cac_ctx* c, const char* prefix, int32_t reps, double* us_per_launch, int32_t* launches,
                           double* bytes, double* flops) {
  if (!c) return CAC_EINVAL;
  if (!prefix || reps < 1) return c->fail(CAC_EINVAL, "profile_replay: prefix and reps >= 1 required");
  if (!c->last_graph) return c->fail(CAC_EINVAL, "profile_replay: no push graph has been replayed yet");
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  const size_t pl = strlen(prefix);
  std::vector<const NodeRec*> sel;
  for (const NodeRec& r : c->last_graph->nodes)
    if (r.name.compare(0, pl, prefix) == 0) sel.push_back(&r);
  if (sel.empty()) return c->fail(CAC_EINVAL, std::string("profile_replay: no launch named ") + prefix + "*");
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipGraphCreate(&g, 0);
  hipGraphNode_t last = nullptr;
  double sb = 0.0, sf = 0.0;
  for (const NodeRec* r : sel) {
    if (e != hipSuccess) break;
    hipKernelNodeParams p = r->p;
    std::vector<char> args = r->args;
    void* kp[1] = {args.data()};
    p.kernelParams = kp;
    hipGraphNode_t n;
    e = hipGraphAddKernelNode(&n, g, last ? &last : nullptr, last ? 1 : 0, &p);
    last = n;
    sb += r->bytes;
    sf += r->flops;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipGraphLaunch(ge, c->stream);  // warm
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipEventRecord(e0, c->stream);
  for (int i = 0; i < reps && e == hipSuccess; ++i) e = hipGraphLaunch(ge, c->stream);
  if (e == hipSuccess) e = hipEventRecord(e1, c->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (ge) (void)hipGraphExecDestroy(ge);
  if (g) (void)hipGraphDestroy(g);
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("profile_replay: ") + hipGetErrorString(e));
  const double n = (double)sel.size();
  if (us_per_launch) *us_per_launch = (double)ms * 1e3 / ((double)reps * n);
  if (launches) *launches = (int32_t)sel.size();
  if (bytes) *bytes = sb / n;
  if (flops) *flops = sf / n;
  return CAC_OK;
}

int32_t cac_destroy(cac_ctx* c) {
  delete c;
  return CAC_OK;
}

}  // extern "C"

namespace {

// Shape checks shared by the test GEMM entry points; returns the k-range count (>= 1) or an
// error code.
int test_gemm_ranges(int32_t dtype, int32_t path, int32_t M, int32_t N, int32_t K, const void* d_A,
                     const void* d_W, float* d_C) {
  g_create_error.clear();
  auto bad = [](const char* m) { g_create_error = m; return CAC_EINVAL; };
  if (dtype != CAC_F32 && dtype != CAC_BF16) return bad("dtype must be CAC_F32 or CAC_BF16");
  if (M < 1 || N < 1 || K < 1 || !d_A || !d_W || !d_C) return bad("empty shape or NULL pointer");
  if (path < 0 || path > 12 || (path >= 2 && dtype != CAC_BF16)) return bad("path out of range for this dtype");
  if (path >= 9 && K % (path == 10 ? 256 : 128)) return bad("paths 9, 11, 12 / 10 need K a multiple of 128 / 256");
  if (path >= 2 && K % 64) return bad("MFMA paths need K a multiple of 64");  // MFMA tiles step K by 64
  if (path >= 2 && N % 8) return bad("MFMA paths need N a multiple of 8");   // 8-column epilogue items
  if ((size_t)8 * K * 4 > 160 * 1024 && path < 2) return bad("K too large for the small-M kernel");
  const int ks = path == 7 ? 2 : path == 8 ? 4 : 1;
  if (ks > 1 && (K % (64 * ks) || N % 256 || N > 1024)) return bad("split-K paths need K a multiple of 64 * ranges and N a multiple of 256 up to 1024");
  return ks;
}

// C = A W^T + bias as the ks > 1 paths compute it: zero C, the split-K partials into part,
// then the residual row kernel adds them (in k-range order) and the bias to C.
void enqueue_split_gemm(Launcher& L, int32_t dtype, int ks, int32_t M, int32_t N, int32_t K, const void* d_A,
                        const void* d_W, const float* d_bias, float* d_C, float* part) {
  EpiArgs e{};
  e.kind = EPI_PART; e.out = part; e.ldo = N; e.pstride = (long)M * N;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.A = d_A; g.W = d_W; g.amap = RowMap{INT_MAX, 0, K}; g.epi = e; g.ksplit = ks;
  FillArgs z{d_C, (long)M * N, 0.0f};
  launch_fill(L, z);
  launch_gemm(L, g, dtype, 0);
  ResLnArgs r{};
  r.part = part; r.pstride = (long)M * N; r.nparts = ks; r.bias = d_bias; r.alpha = 1.0f; r.x = d_C; r.M = M; r.D = N;
  if (L.err == hipSuccess && !launch_resid_ln(L, r, dtype)) L.err = hipErrorInvalidValue;
}

}  // namespace

extern "C" {

int32_t cac_test_gemm(int32_t dtype, int32_t path, int32_t M, int32_t N, int32_t K, const void* d_A, const void* d_W,
                      const float* d_bias, float* d_C, void* hip_stream) {
  const int ks = test_gemm_ranges(dtype, path, M, N, K, d_A, d_W, d_C);
  if (ks < 0) return ks;
  kernels_init();
  Launcher L;
  L.stream = (hipStream_t)hip_stream;
  EpiArgs e{};
  e.kind = EPI_F32; e.bias = d_bias; e.out = d_C; e.ldo = N;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.A = d_A; g.W = d_W; g.amap = RowMap{INT_MAX, 0, K}; g.epi = e;
  if (ks == 1) {
    launch_gemm(L, g, dtype, path);
    return L.err == hipSuccess ? CAC_OK : CAC_EHIP;
  }
  // split-K: partials in a temporary buffer, summed with the bias into the zeroed output by
  // the residual row kernel
  float* part = nullptr;
  if (hipMalloc((void**)&part, (size_t)ks * M * N * sizeof(float)) != hipSuccess) return CAC_EHIP;
  hipError_t err = hipMemsetAsync(d_C, 0, (size_t)M * N * sizeof(float), L.stream);
  g.epi.kind = EPI_PART; g.epi.bias = nullptr; g.epi.out = part; g.epi.pstride = (long)M * N; g.ksplit = ks;
  if (err == hipSuccess) {
    launch_gemm(L, g, dtype, 0);
    ResLnArgs r{};
    r.part = part; r.pstride = (long)M * N; r.nparts = ks; r.bias = d_bias; r.alpha = 1.0f; r.x = d_C; r.M = M; r.D = N;
    if (L.err == hipSuccess && !launch_resid_ln(L, r, dtype)) L.err = hipErrorInvalidValue;
    err = L.err;
  }
  const hipError_t se = hipStreamSynchronize(L.stream);
  (void)hipFree(part);
  return err == hipSuccess && se == hipSuccess ? CAC_OK : CAC_EHIP;
}

int32_t cac_test_gemm_noalloc(int32_t dtype, int32_t path, int32_t M, int32_t N, int32_t K, const void* d_A,
                              const void* d_W, const float* d_bias, float* d_C, void* hip_stream) {
  const int ks = test_gemm_ranges(dtype, path, M, N, K, d_A, d_W, d_C);
  if (ks < 0) return ks;
  if (ks > 1 && (size_t)ks * M * N > kScratchFloats) {
    g_create_error = "split-K partials of " + std::to_string((size_t)ks * M * N) + " floats exceed the " +
                     std::to_string(kScratchFloats) + "-float device scratch";
    return CAC_ENOMEM;
  }
  kernels_init();
  Launcher L;
  L.stream = (hipStream_t)hip_stream;
  if (ks == 1) {
    EpiArgs e{};
    e.kind = EPI_F32; e.bias = d_bias; e.out = d_C; e.ldo = N;
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.A = d_A; g.W = d_W; g.amap = RowMap{INT_MAX, 0, K}; g.epi = e;
    launch_gemm(L, g, dtype, path);
  } else {
    float* part = nullptr;
    L.err = scratch_ptr(&part);
    if (L.err == hipSuccess) enqueue_split_gemm(L, dtype, ks, M, N, K, d_A, d_W, d_bias, d_C, part);
  }
  if (L.err != hipSuccess) {
    g_create_error = std::string("HIP error: ") + hipGetErrorString(L.err);
    return CAC_EHIP;
  }
  return CAC_OK;
}

}  // extern "C"

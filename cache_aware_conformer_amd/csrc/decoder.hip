// Greedy RNNT + EOU decoding (include/cac_decode.h): the prediction network (embedding + LSTM
// stack + projection), the joint after projection with an argmax epilogue, and the per-stream
// greedy state machine, all in float32.
//
// One call runs a fixed sequence of rounds, so it can be launched without knowing on the host
// how many symbols the streams will emit. Round j:
//   1. predictor step for the call slots on list P_j (streams that emitted at round j-1, or
//      whose stream carried a token into the call): LSTM layer 0 .. L-1, then the projection;
//   2. joint for the call slots on list A_j (streams with frames left), every frame of the
//      call at once (the predictor output does not change across blank frames);
//   3. decision per slot on A_j: scan its frames from its cursor; the first frame whose
//      argmax is not blank emits that class (the slot joins P_{j+1}, and A_{j+1} while it has
//      frames left), earlier frames were blank; no emission ends the slot.
// Each slot emits at most max_symbols per frame, so 1 + frames * max_symbols rounds finish
// every slot. Kernels of a round whose list is empty return at once.
//
// The dense parts are one tile kernel on v_mfma_f32_32x32x2f32: 64 x 64 output tiles of four
// waves (32 x 32 each), k-steps of 16 through two LDS buffers, the accumulator tile through LDS
// to a mode-specific epilogue (LSTM cell update, projection store, joint argmax).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/cac.h"
#include "../../include/cac_decode.h"
#include "common.h"
#include "decw.h"
#include "f32tile.h"

void kernels_init();

namespace {

typedef f32x4_t f32x4_d;

// DM_LSTM0: the first LSTM layer, whose input half embed[token] W_ih + biases is a per-token
// table (DM_TABLE, computed once at create), so its product covers only h W_hh.
enum DecMode { DM_LSTM0 = 0, DM_LSTM = 1, DM_PROJ = 2, DM_JOINT = 3, DM_TABLE = 4 };

struct DecTileArgs {
  int K, N;                 // contraction length, output columns (a multiple of 64)
  const float* W;           // [N][ldw]: output column n's K weights at W + n * ldw
  int ldw;
  const float* bias;        // [N]
  const int32_t* ids;       // [n] call slot -> stream id
  const int32_t* list;      // rows: P list (predictor modes) or A list (joint: row = a * nf + f)
  const int32_t* count;     // entries on the list
  const int32_t* slot_tok;  // [n] token a slot's predictor step consumes
  const float* embed;       // [C][H]
  float* h;                 // [S][L][H] state
  float* c;                 // [S][L][H] state
  float* hn;                // [L][n][H] new h of the round's P-list rows
  float* p;                 // [S][P] state: projected predictor output
  int32_t* need;            // [n] slot still has to consume slot_tok
  const float* z;           // [n][nf][P] caller's projected encoder frames
  float2* part;             // [n * nf][ntiles] joint argmax per 64-column tile (value, index)
  float* table;             // [C][4H] embed[token] W_ih + b_ih + b_hh (first layer's input half)
  int layer, L, H, P, C, nf, ntiles, n;
};

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// Where the A row of list row r (r < rows) comes from, resolved once per block: element k is
// ReLU(s0[k] + s1[k]) for the joint, s0[k] for k < split and s1[k - split] after it for the
// LSTM layers above the first, s0[k] otherwise.
struct ARow {
  const float* s0;
  const float* s1;
  int split;
};

template <int MODE>
__device__ __forceinline__ ARow dec_arow(const DecTileArgs& a, int r) {
  if constexpr (MODE == DM_JOINT) {
    const int slot = a.list[r / a.nf], f = r - (r / a.nf) * a.nf;
    return {a.z + ((long)slot * a.nf + f) * a.P, a.p + (long)a.ids[slot] * a.P, 0};
  } else if constexpr (MODE == DM_PROJ) {
    return {a.hn + ((long)(a.L - 1) * a.n + r) * a.H, nullptr, 0};
  } else if constexpr (MODE == DM_TABLE) {
    return {a.embed + (long)r * a.H, nullptr, 0};
  } else if constexpr (MODE == DM_LSTM0) {
    return {a.h + (long)a.ids[a.list[r]] * a.L * a.H, nullptr, 0};
  } else {
    const int id = a.ids[a.list[r]];
    return {a.hn + ((long)(a.layer - 1) * a.n + r) * a.H, a.h + ((long)id * a.L + a.layer) * a.H, a.H};
  }
}

template <int MODE>
__device__ __forceinline__ f32x4_d dec_a4(const ARow& src, int k) {
  if constexpr (MODE == DM_JOINT) {
    f32x4_d v = *(const f32x4_d*)(src.s0 + k) + *(const f32x4_d*)(src.s1 + k);
    v.x = fmaxf(v.x, 0.0f); v.y = fmaxf(v.y, 0.0f); v.z = fmaxf(v.z, 0.0f); v.w = fmaxf(v.w, 0.0f);
    return v;
  } else if constexpr (MODE == DM_LSTM) {
    return k < src.split ? *(const f32x4_d*)(src.s0 + k) : *(const f32x4_d*)(src.s1 + (k - src.split));
  } else {
    return *(const f32x4_d*)(src.s0 + k);
  }
}

// The thread's A row for the shared tile loop.
template <int MODE>
struct DecSrc {
  ARow r;
  __device__ __forceinline__ f32x4_d operator()(int k) const { return dec_a4<MODE>(r, k); }
};

template <int MODE>
__global__ __launch_bounds__(256) void dec_tile_kernel(DecTileArgs a) {
  const int cnt = *a.count;
  const int rows = MODE == DM_JOINT ? cnt * a.nf : cnt;
  const int row0 = blockIdx.y * 64, col0 = blockIdx.x * 64;
  if (row0 >= rows) return;  // the whole block: nothing on the list for these rows
  extern __shared__ __attribute__((aligned(16))) float dlds[];
  const int tid = threadIdx.x;
  // slot, stream id and token of every row of the tile, looked up once
  __shared__ int rslot[64], rid[64], rtok[64];
  if constexpr (MODE == DM_LSTM0 || MODE == DM_LSTM || MODE == DM_PROJ) {
    if (tid < 64) {
      const int r = min(row0 + tid, rows - 1), slot = a.list[r];
      rslot[tid] = slot;
      rid[tid] = a.ids[slot];
      rtok[tid] = MODE == DM_LSTM0 ? a.slot_tok[slot] : 0;
    }
  }
  // rows past the end reload the last one
  const DecSrc<MODE> src{dec_arow<MODE>(a, min(row0 + (tid >> 2), rows - 1))};
  f32_tile(src, a.W, a.ldw, a.K, col0, dlds);
  float (*Ct)[65] = (float (*)[65])dlds;

  if constexpr (MODE == DM_LSTM0 || MODE == DM_LSTM) {
    // packed gate columns: unit u's gates i, f, g, o are columns 4u .. 4u+3
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, rr = idx >> 4, u = idx & 15;
      const int r = row0 + rr;
      if (r >= rows) continue;
      const int col = col0 + 4 * u, U = col >> 2;
      const int id = rid[rr];
      // first layer: the token's row of the input table; other layers: the summed biases
      const float* add = MODE == DM_LSTM0 ? a.table + (long)rtok[rr] * a.N + col : a.bias + col;
      const float gi = Ct[rr][4 * u] + add[0], gf = Ct[rr][4 * u + 1] + add[1];
      const float gg = Ct[rr][4 * u + 2] + add[2], go = Ct[rr][4 * u + 3] + add[3];
      float* cp = a.c + ((long)id * a.L + a.layer) * a.H + U;
      const float cn = sigm(gf) * *cp + sigm(gi) * tanhf(gg);
      *cp = cn;
      a.hn[((long)a.layer * a.n + r) * a.H + U] = sigm(go) * tanhf(cn);
    }
  } else if constexpr (MODE == DM_TABLE) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q, rr = idx >> 6, j = idx & 63;
      if (row0 + rr < rows) a.table[(long)(row0 + rr) * a.N + col0 + j] = Ct[rr][j] + a.bias[col0 + j];
    }
  } else if constexpr (MODE == DM_PROJ) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q, rr = idx >> 6, j = idx & 63;
      if (row0 + rr < rows) a.p[(long)rid[rr] * a.P + col0 + j] = Ct[rr][j] + a.bias[col0 + j];
    }
    // the new h of every layer goes back to the stream state (nothing reads it any more in
    // this round): block column c copies units [64c, 64c + 64) (and every further
    // gridDim.x * 64), four threads per row, 16 units each
    {
      const int rr = tid >> 2, u0 = (tid & 3) * 16, r = row0 + rr;
      if (r < rows) {
        const long id = rid[rr];
        for (int l = 0; l < a.L; ++l)
          for (int ub = blockIdx.x * 64; ub < a.H; ub += gridDim.x * 64)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *(f32x4_d*)(a.h + (id * a.L + l) * a.H + ub + u0 + 4 * q) =
                  *(const f32x4_d*)(a.hn + ((long)l * a.n + r) * a.H + ub + u0 + 4 * q);
      }
    }
    // the slot's token has been consumed
    if (blockIdx.x == 0 && tid < 64 && row0 + tid < rows) a.need[rslot[tid]] = 0;
  } else {
    // joint: argmax of the row over this tile's columns (bias added, columns past C ignored),
    // ties to the lowest column; four threads per row
    const int rr = tid >> 2, part4 = tid & 3;
    float best = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int cc = part4 * 16 + j, col = col0 + cc;
      if (col >= a.C) break;
      const float v = Ct[rr][cc] + a.bias[col];
      if (v > best || bi == INT_MAX) { best = v; bi = col; }
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi != INT_MAX && (bi == INT_MAX || ov > best || (ov == best && oi < bi))) { best = ov; bi = oi; }
    }
    const int r = row0 + rr;
    if (part4 == 0 && r < rows) a.part[(long)r * a.ntiles + blockIdx.x] = make_float2(best, __int_as_float(bi));
  }
}

struct DecRoundArgs {
  const int32_t* ids;
  int32_t* slot_t;      // [n] frame cursor
  int32_t* slot_sym;    // [n] emissions at the cursor frame
  int32_t* slot_tok;    // [n]
  int32_t* slot_ntok;   // [n]
  int32_t* need;        // [n]
  int32_t* plist;       // [rounds + 1][n]
  int32_t* pcnt;        // [rounds + 1]
  int32_t* alist;       // [rounds + 1][n]
  int32_t* acnt;        // [rounds + 1]
  const float2* part;   // [n * nf][ntiles]
  int32_t* tokbuf;      // [n][nf * m] workspace: emitted classes
  int32_t* frmbuf;      // [n][nf * m] workspace: their frames
  int32_t* tokens;      // [n][nf * m] caller's (end kernel only)
  int32_t* tframes;     // [n][nf * m] caller's or null (end kernel only)
  int32_t* counts;      // [n] caller's (end kernel only)
  int32_t* pend;        // [S] token carried to the next call, -1 none
  int n, nf, m, ntiles, blank, round, rounds;
};

// One block: per-call slot state, round lists and output padding.
__global__ __launch_bounds__(256) void dec_begin_kernel(DecRoundArgs a) {
  __shared__ int pc;
  const int tid = threadIdx.x;
  if (tid == 0) pc = 0;
  for (int j = tid; j <= a.rounds; j += 256) { a.pcnt[j] = 0; a.acnt[j] = 0; }
  __syncthreads();
  for (int s = tid; s < a.n; s += 256) {
    const int tok = a.pend[a.ids[s]];
    a.slot_t[s] = 0; a.slot_sym[s] = 0; a.slot_ntok[s] = 0;
    a.slot_tok[s] = tok; a.need[s] = tok >= 0;
    if (tok >= 0) a.plist[atomicAdd(&pc, 1)] = s;
    a.alist[s] = s;
  }
  const int tot = a.n * a.nf * a.m;
  for (int i = tid; i < tot; i += 256) {
    a.tokbuf[i] = -1;
    a.frmbuf[i] = -1;
  }
  __syncthreads();
  if (tid == 0) { a.pcnt[0] = pc; a.acnt[0] = a.n; }
}

// Greedy decision of round `round` for every slot on its A list (see the file comment).
__global__ __launch_bounds__(256) void dec_decide_kernel(DecRoundArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int j = a.round;
  if (e >= a.acnt[j]) return;
  const int s = a.alist[(long)j * a.n + e];
  int t = a.slot_t[s], sym = a.slot_sym[s];
  for (int f = t; f < a.nf; ++f) {
    const float2* pr = a.part + ((long)e * a.nf + f) * a.ntiles;
    float best = pr[0].x;
    int bi = __float_as_int(pr[0].y);
    for (int q = 1; q < a.ntiles; ++q) {     // tiles in column order: strict > keeps the lower index
      const float v = pr[q].x;
      if (v > best) { best = v; bi = __float_as_int(pr[q].y); }
    }
    if (bi == a.blank) { sym = 0; continue; }
    if (f != t) sym = 0;
    const int k = a.slot_ntok[s];
    a.tokbuf[(long)s * a.nf * a.m + k] = bi;
    a.frmbuf[(long)s * a.nf * a.m + k] = f;
    a.slot_ntok[s] = k + 1;
    ++sym;
    t = f;
    if (sym == a.m) { t = f + 1; sym = 0; }
    a.slot_t[s] = t; a.slot_sym[s] = sym;
    a.slot_tok[s] = bi; a.need[s] = 1;
    a.plist[(long)(j + 1) * a.n + atomicAdd(&a.pcnt[j + 1], 1)] = s;
    if (t < a.nf) a.alist[(long)(j + 1) * a.n + atomicAdd(&a.acnt[j + 1], 1)] = s;
    return;
  }
  a.slot_t[s] = a.nf; a.slot_sym[s] = 0;
}

// Carry the unconsumed token of each slot to its stream; emitted classes, their frames and the
// counts out to the caller.
__global__ __launch_bounds__(256) void dec_end_kernel(DecRoundArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.n) return;
  a.pend[a.ids[s]] = a.need[s] ? a.slot_tok[s] : -1;
  a.counts[s] = a.slot_ntok[s];
  const long w = (long)a.nf * a.m, o = (long)s * w;
  for (long i = 0; i < w; ++i) {
    a.tokens[o + i] = a.tokbuf[o + i];
    if (a.tframes) a.tframes[o + i] = a.frmbuf[o + i];
  }
}

// The caller's projected frames into the workspace (so the joint nodes never hold a caller
// pointer and a replayed call re-points only this node and the end kernel's).
struct DecStageArgs {
  const f32x4_d* z;
  f32x4_d* zbuf;
  long n4;
};

__global__ __launch_bounds__(256) void dec_stage_kernel(DecStageArgs a) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.n4; i += (long)gridDim.x * 256) a.zbuf[i] = a.z[i];
}

struct DecResetArgs {
  const int32_t* ids;
  float* h; float* c; float* p; int32_t* pend;
  int n, L, H, P, blank;
};

// One block per stream.
__global__ __launch_bounds__(256) void dec_reset_kernel(DecResetArgs a) {
  const int id = a.ids[blockIdx.x];
  const long hs = (long)a.L * a.H;
  for (long i = threadIdx.x; i < hs; i += 256) {
    a.h[id * hs + i] = 0.0f;
    a.c[id * hs + i] = 0.0f;
  }
  for (long i = threadIdx.x; i < a.P; i += 256) a.p[(long)id * a.P + i] = 0.0f;
  if (threadIdx.x == 0) a.pend[id] = a.blank;
}

// ------------------------------------------------------------------------------- host side
struct DecDims {
  int P, H, L, V, C, Cpad, m, S, nfmax, flags, rounds_max;
};

bool dec_dims(const cac_dec_config* c, DecDims& d, std::string& why) {
  if (!c) { why = "config is NULL"; return false; }
  d.P = c->joint_dim; d.H = c->pred_hidden; d.L = c->pred_layers; d.V = c->vocab; d.m = c->max_symbols;
  d.S = c->max_streams; d.nfmax = c->max_frames; d.flags = c->flags;
  auto bad = [&](const char* msg) { why = msg; return false; };
  if (d.P < 64 || d.P > 4096 || d.P % 64) return bad("joint_dim must be a multiple of 64 in [64, 4096]");
  if (d.H < 64 || d.H > 4096 || d.H % 64) return bad("pred_hidden must be a multiple of 64 in [64, 4096]");
  if (d.L < 1 || d.L > 8) return bad("pred_layers must be in [1, 8]");
  if (d.V < 1 || d.V > (1 << 20)) return bad("vocab must be in [1, 2^20]");
  if (d.m < 1 || d.m > 16) return bad("max_symbols must be in [1, 16]");
  if (d.S < 1 || d.S > (1 << 16)) return bad("max_streams must be in [1, 65536]");
  if (d.nfmax < 1 || d.nfmax > 16) return bad("max_frames must be in [1, 16]");
  d.C = d.V + 2;
  d.Cpad = (d.C + 63) / 64 * 64;
  d.rounds_max = 1 + d.nfmax * d.m;
  return true;
}

size_t dec_params(const DecDims& d) { return dec_param_count(d.C, d.H, d.L, d.P); }

struct DecLayout {
  DecWeights w;
  size_t table, ccount;
  size_t h, c, p, pend;
  size_t ids, slot_t, slot_sym, slot_tok, slot_ntok, need, plist, pcnt, alist, acnt, hn, part, zbuf, tokbuf, frmbuf;
  size_t total;
};

DecLayout dec_layout(const DecDims& d) {
  DecLayout t{};
  size_t off = 0;
  auto take = [&](size_t bytes) { off = (off + 255) & ~(size_t)255; size_t o = off; off += bytes; return o; };
  const size_t H = d.H, P = d.P, S = d.S, n = d.S, R = (size_t)d.rounds_max + 1;
  t.w = dec_weight_offsets(take, d.C, H, d.L, P, d.Cpad);
  t.table = take((size_t)d.C * 4 * H * 4);
  t.ccount = take(4);
  t.h = take(S * d.L * H * 4);
  t.c = take(S * d.L * H * 4);
  t.p = take(S * P * 4);
  t.pend = take(S * 4);
  t.ids = take(n * 4);
  t.slot_t = take(n * 4); t.slot_sym = take(n * 4); t.slot_tok = take(n * 4); t.slot_ntok = take(n * 4);
  t.need = take(n * 4);
  t.plist = take(R * n * 4); t.pcnt = take(R * 4);
  t.alist = take(R * n * 4); t.acnt = take(R * 4);
  t.hn = take((size_t)d.L * n * H * 4);
  t.part = take(n * d.nfmax * (size_t)(d.Cpad / 64) * 8);
  t.zbuf = take(n * d.nfmax * P * 4);
  t.tokbuf = take(n * d.nfmax * d.m * 4);
  t.frmbuf = take(n * d.nfmax * d.m * 4);
  t.total = take(0);
  return t;
}

thread_local std::string g_dec_error;

}  // namespace

struct cac_dec {
  DecDims d;
  DecLayout lay;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  bool dry = false;
  std::vector<int32_t> stamp;
  int32_t stamp_gen = 0;
  std::string err;
  bool profiling = false;
  Profiler prof;
  std::vector<int32_t> dev_ids;  // contents last uploaded to the ids region
  // recorded decode graphs, one per call shape (streams, frames, token frames wanted)
  struct Graph {
    hipGraph_t g = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<NodeRec> nodes;
    std::vector<std::vector<std::pair<size_t, int>>> offs;  // per node: (offset, caller pointer index)
    const void* ptr[4] = {nullptr, nullptr, nullptr, nullptr};
  };
  bool use_graph = true;
  std::map<uint64_t, Graph> graphs;
  ~cac_dec() {
    for (auto& kv : graphs) {
      if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
      if (kv.second.g) (void)hipGraphDestroy(kv.second.g);
    }
  }
  template <class T> T* P(size_t off) const { return (T*)(ws + off); }
  int fail(int code, const std::string& m) { err = m; return code; }
};

namespace {

int dec_check_ids(cac_dec* c, int32_t n, const int32_t* ids) {
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

void dec_reset_launch(cac_dec* c, Launcher& L, int n) {
  DecResetArgs r{c->P<int32_t>(c->lay.ids), c->P<float>(c->lay.h), c->P<float>(c->lay.c), c->P<float>(c->lay.p),
                 c->P<int32_t>(c->lay.pend), n, c->d.L, c->d.H, c->d.P, c->d.V};
  L.tag("dec_reset", 0.0, 0.0);
  L.launch((const void*)&dec_reset_kernel, dim3(n), dim3(256), 0, &r);
}

// Every kernel of one decode call (see the file comment), in launch order: begin; per round the
// LSTM layers, the projection, the joint and the decision; end.
void dec_enqueue(cac_dec* c, Launcher& L, int n, int nf, const float* d_z, int32_t* d_tokens, int32_t* d_token_frames,
                 int32_t* d_counts) {
  const DecDims& d = c->d;
  const DecLayout& y = c->lay;
  const int rounds = 1 + nf * d.m, ntiles = d.Cpad / 64;
  DecRoundArgs ra{};
  ra.ids = c->P<int32_t>(y.ids);
  ra.slot_t = c->P<int32_t>(y.slot_t); ra.slot_sym = c->P<int32_t>(y.slot_sym); ra.slot_tok = c->P<int32_t>(y.slot_tok);
  ra.slot_ntok = c->P<int32_t>(y.slot_ntok); ra.need = c->P<int32_t>(y.need);
  ra.plist = c->P<int32_t>(y.plist); ra.pcnt = c->P<int32_t>(y.pcnt);
  ra.alist = c->P<int32_t>(y.alist); ra.acnt = c->P<int32_t>(y.acnt);
  ra.part = c->P<float2>(y.part); ra.tokbuf = c->P<int32_t>(y.tokbuf); ra.frmbuf = c->P<int32_t>(y.frmbuf);
  ra.pend = c->P<int32_t>(y.pend);
  ra.n = n; ra.nf = nf; ra.m = d.m; ra.ntiles = ntiles; ra.blank = d.V; ra.rounds = rounds;
  L.tag("dec_begin", 0.0, 0.0);
  L.launch((const void*)&dec_begin_kernel, dim3(1), dim3(256), 0, &ra);
  DecStageArgs sa{(const f32x4_d*)d_z, c->P<f32x4_d>(y.zbuf), (long)n * nf * d.P / 4};
  L.tag("dec_stage", 0.0, 0.0);
  L.launch((const void*)&dec_stage_kernel, dim3((unsigned)std::min<long>((sa.n4 + 255) / 256, 2048)), dim3(256), 0, &sa);
  DecTileArgs ta{};
  ta.ids = ra.ids; ta.slot_tok = ra.slot_tok; ta.embed = c->P<float>(y.w.embed);
  ta.h = c->P<float>(y.h); ta.c = c->P<float>(y.c); ta.hn = c->P<float>(y.hn); ta.p = c->P<float>(y.p);
  ta.need = ra.need; ta.z = c->P<float>(y.zbuf); ta.part = c->P<float2>(y.part); ta.table = c->P<float>(y.table);
  ta.L = d.L; ta.H = d.H; ta.P = d.P; ta.C = d.C; ta.nf = nf; ta.ntiles = ntiles; ta.n = n;
  const dim3 blk(256);
  const unsigned prow = (unsigned)((n + 63) / 64), jrow = (unsigned)((n * nf + 63) / 64);
  for (int j = 0; j < rounds && L.err == hipSuccess; ++j) {
    // predictor step of the slots on P_j
    DecTileArgs t = ta;
    t.list = ra.plist + (size_t)j * n;
    t.count = ra.pcnt + j;
    for (int l = 0; l < d.L; ++l) {
      t.layer = l; t.K = l == 0 ? d.H : 2 * d.H; t.N = 4 * d.H; t.ldw = 2 * d.H;
      // layer 0 contracts h with the W_hh inputs only (its input half is the token table)
      t.W = c->P<float>(y.w.lstm_w) + (size_t)l * 2 * d.H * 4 * d.H + (l == 0 ? (size_t)d.H : 0);
      t.bias = c->P<float>(y.w.lstm_b) + (size_t)l * 4 * d.H;
      L.tag("dec_lstm", 0.0, 0.0);
      L.launch(l == 0 ? (const void*)&dec_tile_kernel<DM_LSTM0> : (const void*)&dec_tile_kernel<DM_LSTM>,
               dim3(4 * d.H / 64, prow), blk, F32T_LDS, &t);
    }
    t.K = d.H; t.N = d.P; t.ldw = d.H; t.W = c->P<float>(y.w.proj_w); t.bias = c->P<float>(y.w.proj_b);
    L.tag("dec_proj", 0.0, 0.0);
    L.launch((const void*)&dec_tile_kernel<DM_PROJ>, dim3(d.P / 64, prow), blk, F32T_LDS, &t);
    // joint of the slots on A_j, all frames
    DecTileArgs jt = ta;
    jt.list = ra.alist + (size_t)j * n;
    jt.count = ra.acnt + j;
    jt.K = d.P; jt.N = d.Cpad; jt.ldw = d.P; jt.W = c->P<float>(y.w.out_w); jt.bias = c->P<float>(y.w.out_b);
    L.tag("dec_joint", 0.0, 0.0);
    L.launch((const void*)&dec_tile_kernel<DM_JOINT>, dim3(ntiles, jrow), blk, F32T_LDS, &jt);
    DecRoundArgs r = ra;
    r.round = j;
    L.tag("dec_decide", 0.0, 0.0);
    L.launch((const void*)&dec_decide_kernel, dim3((n + 255) / 256), blk, 0, &r);
  }
  DecRoundArgs ea = ra;
  ea.tokens = d_tokens; ea.tframes = d_token_frames; ea.counts = d_counts;
  L.tag("dec_end", 0.0, 0.0);
  L.launch((const void*)&dec_end_kernel, dim3((n + 255) / 256), blk, 0, &ea);
}

// Profiled call: once it has run, read back its round counts and give every recorded launch its
// algorithmic flops and weight bytes; launches whose list was empty are named "<kernel>/idle".
hipError_t dec_profile_fix(cac_dec* c, size_t first, int n, int nf) {
  const DecDims& d = c->d;
  const int rounds = 1 + nf * d.m;
  std::vector<int32_t> pc(rounds + 1), ac(rounds + 1);
  hipError_t e = hipMemcpyAsync(pc.data(), c->ws + c->lay.pcnt, pc.size() * 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(ac.data(), c->ws + c->lay.acnt, ac.size() * 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return e;
  std::vector<Profiler::Rec>& rec = c->prof.pending;
  if (rec.size() != first + 3 + (size_t)rounds * (d.L + 3)) return hipSuccess;  // events not taken: nothing to name
  const double H = d.H, P = d.P, C = d.C;
  size_t i = first + 2;  // past begin and stage
  auto set = [&](const char* name, double rows, double flops_per_row, double wbytes) {
    Profiler::Rec& r = rec[i++];
    const std::string nm = std::string(name) + (rows > 0 ? "" : "/idle");
    r.name = c->prof.name_id(nm.c_str());
    r.flops = rows * flops_per_row;
    r.bytes = rows > 0 ? wbytes : 0.0;
  };
  for (int j = 0; j < rounds; ++j) {
    for (int l = 0; l < d.L; ++l) set("dec_lstm", pc[j], 2.0 * (l ? 2 : 1) * H * 4 * H, (l ? 2 : 1) * H * 4 * H * 4);
    set("dec_proj", pc[j], 2.0 * H * P, H * P * 4);
    set("dec_joint", (double)ac[j] * nf, 2.0 * P * C, P * d.Cpad * 4);
    set("dec_decide", ac[j], 0.0, 0.0);
  }
  (void)n;
  return hipSuccess;
}

// Offsets of 8-byte fields of a recorded argument block that hold exactly p.
std::vector<size_t> dec_find_ptr(const std::vector<char>& args, const void* p) {
  std::vector<size_t> offs;
  if (!p) return offs;
  const uint64_t v = (uint64_t)(uintptr_t)p;
  for (size_t o = 0; o + 8 <= args.size(); o += 8) {
    uint64_t w;
    memcpy(&w, args.data() + o, 8);
    if (w == v) offs.push_back(o);
  }
  return offs;
}

// Replay the recorded graph of this call shape (recording it on first use), re-pointing the
// nodes that hold the caller's pointers (z, tokens, token frames, counts).
hipError_t dec_graph(cac_dec* c, int n, int nf, const void* const ptrs[4]) {
  const uint64_t key = ((uint64_t)n << 8) | ((uint64_t)nf << 1) | (ptrs[2] ? 1u : 0u);
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    cac_dec::Graph gr;
    hipError_t e = hipGraphCreate(&gr.g, 0);
    if (e != hipSuccess) return e;
    Launcher L;
    L.stream = c->stream;
    L.graph = gr.g;
    L.rec = &gr.nodes;
    dec_enqueue(c, L, n, nf, (const float*)ptrs[0], (int32_t*)ptrs[1], (int32_t*)ptrs[2], (int32_t*)ptrs[3]);
    if (L.err != hipSuccess) { (void)hipGraphDestroy(gr.g); return L.err; }
    e = hipGraphInstantiate(&gr.exec, gr.g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(gr.g); return e; }
    for (const NodeRec& r : gr.nodes) {
      std::vector<std::pair<size_t, int>> o;
      for (int q = 0; q < 4; ++q)
        for (size_t off : dec_find_ptr(r.args, ptrs[q])) o.push_back({off, q});
      gr.offs.push_back(o);
    }
    for (int q = 0; q < 4; ++q) gr.ptr[q] = ptrs[q];
    it = c->graphs.emplace(key, std::move(gr)).first;
  }
  cac_dec::Graph& gr = it->second;
  bool same = true;
  for (int q = 0; q < 4; ++q) same = same && gr.ptr[q] == ptrs[q];
  if (!same) {
    for (size_t i = 0; i < gr.nodes.size(); ++i) {
      if (gr.offs[i].empty()) continue;
      NodeRec& r = gr.nodes[i];
      for (const auto& oq : gr.offs[i]) memcpy(r.args.data() + oq.first, &ptrs[oq.second], 8);
      hipKernelNodeParams p = r.p;
      void* kp[1] = {r.args.data()};
      p.kernelParams = kp;
      hipError_t e = hipGraphExecKernelNodeSetParams(gr.exec, r.node, &p);
      if (e != hipSuccess) return e;
    }
    for (int q = 0; q < 4; ++q) gr.ptr[q] = ptrs[q];
  }
  return hipGraphLaunch(gr.exec, c->stream);
}

}  // namespace

extern "C" {

size_t cac_dec_param_count(const cac_dec_config* cfg) {
  DecDims d;
  std::string why;
  return dec_dims(cfg, d, why) ? dec_params(d) : 0;
}

size_t cac_dec_workspace_bytes(const cac_dec_config* cfg) {
  DecDims d;
  std::string why;
  return dec_dims(cfg, d, why) ? dec_layout(d).total : 0;
}

const char* cac_dec_last_error(const cac_dec* ctx) { return ctx ? ctx->err.c_str() : g_dec_error.c_str(); }

int32_t cac_dec_create(const cac_dec_config* cfg, const float* h_params, size_t n_params, void* d_workspace,
                       size_t ws_bytes, void* hip_stream, cac_dec** out) {
  g_dec_error.clear();
  if (!out) { g_dec_error = "out is NULL"; return CAC_EINVAL; }
  *out = nullptr;
  DecDims d;
  if (!dec_dims(cfg, d, g_dec_error)) return CAC_EINVAL;
  if (!h_params) { g_dec_error = "parameter array is NULL"; return CAC_EINVAL; }
  if (n_params != dec_params(d)) {
    g_dec_error = "expected " + std::to_string(dec_params(d)) + " parameters, got " + std::to_string(n_params);
    return CAC_EINVAL;
  }
  const bool dry = (d.flags & CAC_FLAG_DRY_RUN) != 0;
  const DecLayout lay = dec_layout(d);
  if (!dry) {
    if (!d_workspace) { g_dec_error = "workspace is NULL"; return CAC_EINVAL; }
    if (((uintptr_t)d_workspace) & 255) { g_dec_error = "workspace must be 256-byte aligned"; return CAC_EINVAL; }
    if (ws_bytes < lay.total) { g_dec_error = "workspace too small: need " + std::to_string(lay.total) + " bytes"; return CAC_ENOMEM; }
  }
  cac_dec* c = new cac_dec();
  c->d = d; c->lay = lay; c->ws = (char*)d_workspace; c->stream = (hipStream_t)hip_stream; c->dry = dry;
  c->stamp.assign(d.S, 0);
  if (dry) { *out = c; return CAC_OK; }
  kernels_init();
  for (const void* f : {(const void*)&dec_tile_kernel<DM_LSTM0>, (const void*)&dec_tile_kernel<DM_LSTM>,
                        (const void*)&dec_tile_kernel<DM_PROJ>, (const void*)&dec_tile_kernel<DM_JOINT>,
                        (const void*)&dec_tile_kernel<DM_TABLE>})
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)F32T_LDS);
  std::vector<uint8_t> buf(lay.w.end, 0);
  dec_repack(h_params, lay.w, d.C, d.H, d.L, d.P, d.Cpad, buf.data());
  hipError_t e = hipMemcpyAsync(c->ws, buf.data(), buf.size(), hipMemcpyHostToDevice, c->stream);
  std::vector<int32_t> all(d.S);
  for (int i = 0; i < d.S; ++i) all[i] = i;
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.ids, all.data(), (size_t)d.S * 4, hipMemcpyHostToDevice, c->stream);
  c->dev_ids = all;
  const int32_t cc = (int32_t)d.C;
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.ccount, &cc, 4, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) {
    Launcher L;
    L.stream = c->stream;
    // first layer's input table: embed[token] W_ih + b_ih + b_hh for every class
    DecTileArgs t{};
    t.K = d.H; t.N = 4 * d.H; t.ldw = 2 * d.H; t.W = c->P<float>(lay.w.lstm_w); t.bias = c->P<float>(lay.w.lstm_b);
    t.count = c->P<int32_t>(lay.ccount); t.embed = c->P<float>(lay.w.embed); t.table = c->P<float>(lay.table);
    t.H = d.H; t.C = d.C;
    L.tag("dec_table", 0.0, 0.0);
    L.launch((const void*)&dec_tile_kernel<DM_TABLE>, dim3(4 * d.H / 64, (d.C + 63) / 64), dim3(256), F32T_LDS, &t);
    dec_reset_launch(c, L, d.S);
    e = L.err;
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    g_dec_error = std::string("HIP error during create: ") + hipGetErrorString(e);
    delete c;
    return CAC_EHIP;
  }
  *out = c;
  return CAC_OK;
}

int32_t cac_dec_greedy(cac_dec* c, int32_t n, const int32_t* ids, int32_t nf, const float* d_z, int32_t* d_tokens,
                       int32_t* d_token_frames, int32_t* d_counts) {
  if (!c) return CAC_EINVAL;
  const DecDims& d = c->d;
  int rc = dec_check_ids(c, n, ids);
  if (rc) return rc;
  if (nf < 1 || nf > d.nfmax) return c->fail(CAC_EINVAL, "n_frames must be in [1, max_frames]");
  if (!d_z || !d_tokens || !d_counts) return c->fail(CAC_EINVAL, "z, tokens or counts pointer is NULL");
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  const hipError_t pe = hipStreamQuery(c->stream);
  if (pe != hipSuccess && pe != hipErrorNotReady)
    return c->fail(CAC_EHIP, std::string("asynchronous device error from earlier work: ") + hipGetErrorString(pe));
  hipError_t e = hipSuccess;
  if ((int)c->dev_ids.size() != n || memcmp(c->dev_ids.data(), ids, (size_t)n * 4) != 0) {
    c->dev_ids.assign(ids, ids + n);
    e = hipMemcpyAsync(c->ws + c->lay.ids, c->dev_ids.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  }
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("id upload failed: ") + hipGetErrorString(e));
  const void* ptrs[4] = {d_z, d_tokens, d_token_frames, d_counts};
  if (c->use_graph && !c->profiling) {
    e = dec_graph(c, n, nf, ptrs);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("graph replay failed: ") + hipGetErrorString(e));
    return CAC_OK;
  }
  Launcher L;
  L.stream = c->stream;
  size_t first = 0;
  if (c->profiling) {
    c->prof.drain();
    L.prof = &c->prof;
    first = c->prof.pending.size();
  }
  dec_enqueue(c, L, n, nf, d_z, d_tokens, d_token_frames, d_counts);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  if (c->profiling) {
    e = dec_profile_fix(c, first, n, nf);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("profiling: ") + hipGetErrorString(e));
  }
  return CAC_OK;
}

int32_t cac_dec_set_graph(cac_dec* c, int32_t enable) {
  if (!c) return CAC_EINVAL;
  c->use_graph = enable != 0;
  return CAC_OK;
}

int32_t cac_dec_profile(cac_dec* c, int32_t enable) {
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

int32_t cac_dec_profile_read(cac_dec* c, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
                             double* total_ms, double* bytes, double* flops) {
  if (!c || max_entries < 0 || name_len < 1) return CAC_EINVAL;
  c->prof.drain();
  if (c->prof.err != hipSuccess) return c->fail(CAC_EHIP, std::string("profiling: ") + hipGetErrorString(c->prof.err));
  const int nn = (int)c->prof.names.size();
  for (int i = 0; i < nn && i < max_entries; ++i) {
    if (names) {
      strncpy(names + (size_t)i * name_len, c->prof.names[i].c_str(), name_len - 1);
      names[(size_t)i * name_len + name_len - 1] = 0;
    }
    if (launches) launches[i] = c->prof.launches[i];
    if (total_ms) total_ms[i] = c->prof.ms[i];
    if (bytes) bytes[i] = c->prof.bytes[i];
    if (flops) flops[i] = c->prof.flops[i];
  }
  return nn;
}

int32_t cac_dec_reset(cac_dec* c, int32_t n, const int32_t* ids) {
  if (!c) return CAC_EINVAL;
  int rc = dec_check_ids(c, n, ids);
  if (rc) return rc;
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  Launcher L;
  L.stream = c->stream;
  c->dev_ids.assign(ids, ids + n);
  L.err = hipMemcpyAsync(c->ws + c->lay.ids, c->dev_ids.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  dec_reset_launch(c, L, n);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  return n;
}

int32_t cac_dec_destroy(cac_dec* c) {
  delete c;
  return CAC_OK;
}

}  // extern "C"

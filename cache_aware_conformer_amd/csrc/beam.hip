// Batched MALSD beam search (include/cac_beam.h): K hypotheses per utterance, float32.
//
// Device state per utterance b: two copies of its K slots (score, frame, labels at the frame,
// transcript length, last label, transcript hash, predictor state entry), the live one by the
// parity of the round, and two copies of their transcripts, tcur[b] naming the live one. Predictor states live in a pool: entry 0 is
// the zero state, entry 1 the state after the start symbol, and utterance b owns 2K entries
// after those. A new label's state goes into an entry that no slot of the old beam refers to,
// so the parents' entries are never overwritten while they are read; blank shares its
// parent's entry.
//
// One iteration ("round") is six kernels:
//   joint   - rows of the joint list (live hypotheses with frames left): ReLU(z[b][t] + p) Wout
//             + bout into a logits row per slot (MFMA tiles, the predictor/joint tile loop);
//   cand    - four waves per hypothesis: log_softmax and its top-K (or forced blank, or a
//             final hypothesis offering itself);
//   select  - one block per utterance: global top-K, new slots and transcripts, recombination,
//             predictor entries for new labels, the next joint list (each entry the frame row,
//             predictor entry and logits row it needs, so the joint reads no beam state);
//             an utterance without work copies its slots to the next parity;
//   lstm x L, proj - the predictor for the new labels (MFMA tiles).
// The host runs rounds in groups (a recorded graph per group) and reads the next joint list's
// length between groups: zero means no hypothesis has frames left. Every kernel loads its list
// length and its list entries together, so each launch waits for one round trip before it
// reads its operands.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/cac.h"
#include "../../include/cac_beam.h"
#include "common.h"
#include "decw.h"
#include "f32tile.h"

void kernels_init();

namespace {

constexpr int BEAM_MAX = 8;
constexpr int BEAM_NV = 32;          // logits held per lane in the select kernel: C <= 64 * 32
constexpr int BEAM_GROUP = 16;       // rounds per recorded graph (even: the parity repeats)
constexpr int POOL_ZERO = 0, POOL_START = 1, POOL_BASE = 2;
constexpr uint64_t HASH_MUL = 0x100000001B3ull;

struct BeamSlot {
  float score;   // -inf: empty slot
  int t;         // frame
  int nsym;      // labels emitted at frame t
  int len;       // transcript length
  int ref;       // predictor state entry
  int last;      // last label, -1 before the first
  uint64_t hash; // of the transcript
};

enum BeamMode { BM_LSTM0 = 0, BM_LSTM = 1, BM_PROJ = 2, BM_JOINT = 3, BM_TABLE = 4 };

struct BeamTileArgs {
  int K, N;                  // contraction length, output columns (multiple of 64)
  const float* W;            // [N][ldw]: output column n's K weights at W + n * ldw
  int ldw;
  const float* bias;         // [N]
  const int32_t* count;      // rows on the list
  const int32_t* psrc;       // predictor list: parent's state entry
  const int32_t* pdst;       // predictor list: new entry
  const int32_t* ptok;       // predictor list: label
  const int4* jlist;         // joint list: (frame row b * T + t, predictor entry, logits row b * beam + k)
  const float* zbuf;         // [n][T][P]
  float* logits;             // [n * beam][Cpad]
  float* ph;                 // pool [E][L][H]
  float* pc;                 // pool [E][L][H]
  float* pp;                 // pool [E][P]
  const float* embed;        // [C][H]
  float* table;              // [C][4H]
  int32_t* clr0;             // joint only: counters to clear for the select kernel that follows
  int32_t* clr1;
  int32_t* rnow;             // joint only: rounds started in this call (advanced by one)
  int32_t* log;              // [rounds][2] rows seen by the joint / the first LSTM layer (profiling)
  int layer, L, H, P, C, T, n, beam, round;
  int gx;                    // column tiles (the grid holds 8 * ceil(gx / 8) per row tile)
};

__device__ __forceinline__ float bsigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// The thread's A row for the shared tile loop: ReLU(s0 + s1) for the joint; s0 for k < H and
// s1 after it for an LSTM layer above the first; s0 otherwise.
template <int MODE>
struct BeamSrc {
  const float* s0;
  const float* s1;
  int split;
  __device__ __forceinline__ f32x4_t operator()(int k) const {
    if constexpr (MODE == BM_JOINT) {
      f32x4_t v = *(const f32x4_t*)(s0 + k) + *(const f32x4_t*)(s1 + k);
      v.x = fmaxf(v.x, 0.0f); v.y = fmaxf(v.y, 0.0f); v.z = fmaxf(v.z, 0.0f); v.w = fmaxf(v.w, 0.0f);
      return v;
    } else if constexpr (MODE == BM_LSTM) {
      return k < split ? *(const f32x4_t*)(s0 + k) : *(const f32x4_t*)(s1 + (k - split));
    } else {
      return *(const f32x4_t*)(s0 + k);
    }
  }
};

// 32 x 32 output tiles (rows of the work list x output columns), each computed by a block's
// BEAM_TW waves splitting the contraction (f32_tile32), then the mode's epilogue. The grid is
// 1-D and bounded; blocks loop over the tiles of the rows the list holds, so a short list costs
// no idle blocks. Tile t runs on XCD t mod 8 (its block's), and each XCD takes a contiguous
// eighth of the column tiles for every row tile, so each weight row is fetched into one XCD's
// L2 only.
constexpr int BEAM_TW = 4;

template <int MODE>
__global__ __launch_bounds__(64 * BEAM_TW) void beam_tile_kernel(BeamTileArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (MODE == BM_JOINT) {
    if (blockIdx.x == 0 && tid == 0) {
      *a.clr0 = 0;
      *a.clr1 = 0;
      *a.rnow += 1;
      if (a.log) a.log[2 * a.round] = *a.count;
    }
  }
  if constexpr (MODE == BM_LSTM0) {
    if (a.log && blockIdx.x == 0 && tid == 0) a.log[2 * a.round + 1] = *a.count;
  }
  const int per = (a.gx + 7) >> 3;
  const int rows = *a.count;
  __shared__ __attribute__((aligned(16))) float red[BEAM_TW * 32 * 33];
  __shared__ int rsrc[32], rdst[32], rtok[32];
  const int L = a.L, H = a.H;
  // tiles t = blockIdx.x, + gridDim.x, ... (gridDim.x a multiple of 8, so all of a block's
  // tiles belong to its XCD's column eighth); the row tile grows with t
  for (int t = blockIdx.x;; t += gridDim.x) {
    const int xcd = t & 7, j = t >> 3;
    const int cx = xcd * per + j % per, ry = j / per;
    const int row0 = ry * 32, col0 = cx * 32;
    if (row0 >= rows) break;
    if (cx >= a.gx) continue;
    // this lane's list entry (rows past the length take the list's first row)
    const int r = row0 + (lane & 31);
    const int rr0 = r < rows ? r : 0;
    int4 je = make_int4(0, 0, 0, 0);
    int ps = 0, pd = 0, pt = 0;
    if constexpr (MODE == BM_JOINT) je = a.jlist[rr0];
    else if constexpr (MODE != BM_TABLE) { ps = a.psrc[rr0]; pd = a.pdst[rr0]; pt = a.ptok[rr0]; }
    __syncthreads();   // the previous tile's epilogue is done with the row info
    if (tid < 32) {
      if constexpr (MODE == BM_JOINT) rdst[tid] = je.z;
      else { rsrc[tid] = ps; rdst[tid] = pd; rtok[tid] = pt; }
    }
    BeamSrc<MODE> src{nullptr, nullptr, 0};
    if constexpr (MODE == BM_JOINT) {
      src.s0 = a.zbuf + (long)je.x * a.P;
      src.s1 = a.pp + (long)je.y * a.P;
    } else if constexpr (MODE == BM_TABLE) {
      src.s0 = a.embed + (long)rr0 * H;
    } else if constexpr (MODE == BM_LSTM0) {
      src.s0 = a.ph + (long)ps * L * H;
    } else if constexpr (MODE == BM_LSTM) {
      src.s0 = a.ph + ((long)pd * L + a.layer - 1) * H;
      src.s1 = a.ph + ((long)ps * L + a.layer) * H;
      src.split = H;
    } else {
      src.s0 = a.ph + ((long)pd * L + L - 1) * H;
    }
    f32_tile32<BEAM_TW>(src, a.W + (long)(col0 + (lane & 31)) * a.ldw, a.K, red);
    float (*Ct)[33] = (float (*)[33])red;

    if constexpr (MODE == BM_LSTM0 || MODE == BM_LSTM) {
      // unit u's gates i, f, g, o are columns 4u .. 4u+3: 32 rows x 8 units, one per thread
      const int er = tid >> 3, u = tid & 7;
      if (tid < 256 && row0 + er < rows) {
        const int col = col0 + 4 * u, U = col >> 2;
        const float* add = MODE == BM_LSTM0 ? a.table + (long)rtok[er] * a.N + col : a.bias + col;
        const float gi = Ct[er][4 * u] + add[0], gf = Ct[er][4 * u + 1] + add[1];
        const float gg = Ct[er][4 * u + 2] + add[2], go = Ct[er][4 * u + 3] + add[3];
        const float cprev = a.pc[((long)rsrc[er] * L + a.layer) * H + U];
        const float cn = bsigm(gf) * cprev + bsigm(gi) * tanhf(gg);
        const long o = ((long)rdst[er] * L + a.layer) * H + U;
        a.pc[o] = cn;
        a.ph[o] = bsigm(go) * tanhf(cn);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 1024 / (64 * BEAM_TW); ++q) {
        const int idx = tid + 64 * BEAM_TW * q, er = idx >> 5, jc = idx & 31;
        if (row0 + er >= rows) continue;
        const float v = Ct[er][jc] + a.bias[col0 + jc];
        if constexpr (MODE == BM_PROJ) a.pp[(long)rdst[er] * a.P + col0 + jc] = v;
        else if constexpr (MODE == BM_TABLE) a.table[(long)(row0 + er) * a.N + col0 + jc] = v;
        else a.logits[(long)rdst[er] * a.N + col0 + jc] = v;
      }
    }
    __syncthreads();   // the output tile's LDS is free for the next tile
  }
}

struct BeamSelArgs {
  const float* logits;   // [n * beam][Cpad]
  float* cand_s;         // [n][64] candidate scores, slot-major (k * beam + rank); -inf: none
  int32_t* cand_c;       // [n][64] candidate classes (-1: a final hypothesis offering itself)
  BeamSlot* slots;       // [2][n][beam]: this round's at parity q, the next round's at q ^ 1
  int32_t* tcur;         // [n] live transcript copy
  int32_t* tr;           // [2][n][beam][U] transcripts
  const int32_t* tlen;   // [n] frames per utterance
  int4* jlist;           // next round's joint list
  int32_t* jcnt;
  int32_t* psrc; int32_t* pdst; int32_t* ptok; int32_t* pcnt;
  int32_t* rounds;       // iterations with work (max over utterances)
  const int32_t* rnow;   // rounds started in this call, this one included
  int n, beam, C, Cpad, U, blank, m, weak_hash, q, T;
};

// (value, index) pairs: higher value first, then lower index
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// The best (value, index) pair over the wave, on every lane: the largest value, then the
// smallest index among the lanes holding it (indices below 2^24, exact in float). Register
// exchanges only (DPP rows and the lane-half swaps).
__device__ __forceinline__ void wave_best(float& v, int& i) {
  const float m = wave_top(v);
  const float fi = (v == m && i != INT_MAX) ? (float)i : 3.0e9f;
  const float mi = -wave_top(-fi);
  v = m;
  i = mi < 2.0e9f ? (int)mi : INT_MAX;
}

// One block of four waves per hypothesis (grid n * beam): its candidates. A live hypothesis
// with frames left takes log_softmax of its logits row; with labels left at its frame its
// candidates are its K best classes (score + log-probability, ranked by logit then class),
// else blank alone with the blank's log-probability; a final hypothesis offers itself; an empty
// slot offers nothing. The classes are dealt to the four waves (class lane + 64 (wave + 4 i)),
// each wave finds its own K best, and the first wave merges the 4 K.
constexpr int CAND_NV = BEAM_NV / 4;   // classes per lane and wave

__global__ __launch_bounds__(256) void beam_cand_kernel(BeamSelArgs a) {
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, K = a.beam;
  const int b = e / K, k = e - b * K;
  const BeamSlot h = a.slots[((long)a.q * a.n + b) * K + k];
  const int T = a.tlen[b];
  // this wave's share of the logits row, loaded with the slot (only used when this round's
  // joint wrote the row)
  const float* row = a.logits + (long)e * a.Cpad;
  float v[CAND_NV];
#pragma unroll
  for (int i = 0; i < CAND_NV; ++i) {
    const int col = lane + 64 * (wave + 4 * i);
    v[i] = col < a.C ? row[col] : -INFINITY;
  }
  __shared__ float red[4];
  __shared__ float pv_s[4 * BEAM_MAX];
  __shared__ int pc_s[4 * BEAM_MAX];
  float* cs = a.cand_s + (long)b * 64 + k * K;
  int32_t* cc = a.cand_c + (long)b * 64 + k * K;
  const bool live = h.score > -INFINITY;
  if (!live || h.t >= T) {   // block-uniform: an empty slot, or a final hypothesis offering itself
    if (tid < K) {
      cs[tid] = (live && tid == 0) ? h.score : -INFINITY;
      cc[tid] = (live && tid == 0) ? -1 : -2;
    }
    return;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < CAND_NV; ++i) mx = fmaxf(mx, v[i]);
  mx = wave_top(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < CAND_NV; ++i) sum += v[i] > -INFINITY ? __expf(v[i] - mx) : 0.0f;
  sum = wave_total(sum);
  __syncthreads();   // every wave has read the maxima
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  const float lse = mx + __logf((red[0] + red[1]) + (red[2] + red[3]));
  if (h.nsym >= a.m) {  // label cap reached: blank only, with its full log-probability
    if (tid < K) {
      cs[tid] = tid == 0 ? h.score + (row[a.blank] - lse) : -INFINITY;
      cc[tid] = tid == 0 ? a.blank : -2;
    }
    return;
  }
  // this wave's K best (logit desc, class asc): each pass takes the best after the previous one
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < K; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < CAND_NV; ++i) {
      const int col = lane + 64 * (wave + 4 * i);
      const bool after = v[i] < pv || (v[i] == pv && col > pi);
      if (after && v[i] > -INFINITY && better(v[i], col, bv, bi)) { bv = v[i]; bi = col; }
    }
    wave_best(bv, bi);
    if (lane == 0) { pv_s[wave * K + r] = bv; pc_s[wave * K + r] = bi; }
    pv = bv;
    pi = bi;
  }
  __syncthreads();
  // the first wave merges the four lists (one candidate per lane, its class as the tie index)
  if (wave == 0) {
    float mine = lane < 4 * K ? pv_s[lane] : -INFINITY;
    const int cls = lane < 4 * K ? pc_s[lane] : INT_MAX;
    float out_s = -INFINITY;
    int out_c = -2;
    for (int r = 0; r < K; ++r) {
      float bv = mine > -INFINITY ? mine : -INFINITY;
      int bi = mine > -INFINITY ? cls : INT_MAX;
      wave_best(bv, bi);
      if (!(bv > -INFINITY)) break;
      if (lane == r) { out_s = h.score + (bv - lse); out_c = bi; }
      if (cls == bi) mine = -INFINITY;
    }
    if (lane < K) { cs[lane] = out_s; cc[lane] = out_c; }
  }
}

// One block of 256 threads per utterance: the global top-K of the candidates, new slots and
// transcripts, recombination, the next round's work lists.
__global__ __launch_bounds__(256) void beam_select_kernel(BeamSelArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.beam, nthr = 256, NWV = 4;
  const int T = a.tlen[b];
  const BeamSlot* old = a.slots + ((long)a.q * a.n + b) * K;
  BeamSlot* nw = a.slots + ((long)(a.q ^ 1) * a.n + b) * K;
  __shared__ BeamSlot so[BEAM_MAX], sn[BEAM_MAX];
  __shared__ int cc[64];
  __shared__ int sel_par[BEAM_MAX], sel_cls[BEAM_MAX], nsel;
  __shared__ float sel_sc[BEAM_MAX], merged[BEAM_MAX];
  __shared__ int eq[BEAM_MAX][BEAM_MAX];
  // candidates (one per lane of wave 0), loaded with the slots
  const float mine = (wave == 0 && lane < K * K) ? a.cand_s[(long)b * 64 + lane] : -INFINITY;
  if (wave == 0) cc[lane] = lane < K * K ? a.cand_c[(long)b * 64 + lane] : -2;
  if (tid < K) so[tid] = old[tid];
  if (tid < BEAM_MAX * BEAM_MAX) eq[tid / BEAM_MAX][tid % BEAM_MAX] = 0;
  __syncthreads();
  bool work = false;
  for (int k = 0; k < K; ++k) work = work || (so[k].score > -INFINITY && so[k].t < T);
  if (!work) {  // every live hypothesis is final: the beam stands, carried to the next parity
    if (tid < K) nw[tid] = so[tid];
    return;
  }
  const int par = a.tcur[b];
  const int32_t* __restrict__ otr = a.tr + ((long)par * a.n + b) * K * a.U;
  int32_t* __restrict__ ntr = a.tr + ((long)(par ^ 1) * a.n + b) * K * a.U;

  // the K best of all candidates (flat index k * K + rank: ties to the lower slot, then class)
  if (wave == 0) {
    bool taken = false;
    int cnt = 0;
    for (int r = 0; r < K; ++r) {
      float bv = taken ? -INFINITY : mine;
      int bi = taken ? INT_MAX : lane;
      wave_best(bv, bi);
      if (!(bv > -INFINITY)) break;
      if (lane == bi) taken = true;
      if (lane == 0) { sel_par[r] = bi / K; sel_cls[r] = cc[bi]; sel_sc[r] = bv; }
      ++cnt;
    }
    if (lane == 0) nsel = cnt;
  }
  __syncthreads();

  // new slots
  if (tid < K) {
    BeamSlot s;
    if (tid >= nsel) {
      s = so[0];
      s.score = -INFINITY;
    } else {
      const int c = sel_cls[tid];
      s = so[sel_par[tid]];
      s.score = sel_sc[tid];
      if (c == a.blank) {
        s.t += 1;
        s.nsym = 0;
      } else if (c >= 0) {
        s.nsym += 1;
        s.len += 1;
        s.last = c;
        s.hash = a.weak_hash ? 0ull : s.hash * HASH_MUL + (uint64_t)(c + 1);
      }
    }
    sn[tid] = s;
  }
  // transcripts: the parent's tokens, then the new label; one pass over every (slot,
  // position) pair, so the loads of all slots are in flight together
  {
    int start[BEAM_MAX + 1];
    start[0] = 0;
    for (int j = 0; j < K; ++j) start[j + 1] = start[j] + (j < nsel ? so[sel_par[j]].len : 0);
    const int tot = start[K];
    for (int e = tid; e < tot; e += nthr) {
      int j = 0;
      while (e >= start[j + 1]) ++j;
      const int i = e - start[j];
      ntr[(long)j * a.U + i] = otr[(long)sel_par[j] * a.U + i];
    }
    if (tid < nsel) {
      const int c = sel_cls[tid];
      if (c >= 0 && c != a.blank) ntr[(long)tid * a.U + so[sel_par[tid]].len] = c;
    }
  }
  __syncthreads();

  // recombination: pairs with equal length, last label and hash compare their tokens (a wave
  // per pair)
  for (int pr = wave; pr < K * K; pr += NWV) {
    const int i = pr / K, j = pr % K;
    if (i >= j || i >= nsel || j >= nsel) continue;
    const BeamSlot& x = sn[i];
    const BeamSlot& y = sn[j];
    if (x.len != y.len || x.last != y.last || x.hash != y.hash) continue;
    const int32_t* ti = ntr + (long)i * a.U;
    const int32_t* tj = ntr + (long)j * a.U;
    bool diff = false;
    for (int q = lane; q < x.len; q += 64) diff = diff || ti[q] != tj[q];
    const bool any = __any(diff);
    if (lane == 0 && !any) { eq[i][j] = 1; eq[j][i] = 1; }
  }
  __syncthreads();
  if (tid < K) {
    float sc = sn[tid].score;
    if (sc > -INFINITY) {
      int best = tid;
      float mx = sc;
      for (int j = 0; j < K; ++j)
        if (eq[tid][j] && better(sn[j].score, j, sn[best].score, best)) best = j;
      for (int j = 0; j < K; ++j) if (eq[tid][j]) mx = fmaxf(mx, sn[j].score);
      if (best != tid) {
        sc = -INFINITY;
      } else {
        float s = 0.0f;
        for (int j = 0; j < K; ++j)
          if (j == tid || eq[tid][j]) s += expf(sn[j].score - mx);
        sc = mx + logf(s);
      }
    }
    merged[tid] = sc;
  }
  __syncthreads();

  if (wave == 0) {
    // Lane j < K finishes new slot j. Predictor entries for the new labels: the utterance's 2K
    // entries minus those the old beam refers to, handed out in slot order; then one
    // reservation on each work list, each slot's place in it from a prefix count of the lanes.
    const int base = POOL_BASE + b * 2 * K;
    uint32_t used = 0;
    for (int k = 0; k < K; ++k) {
      const int r = so[k].ref - base;
      if (r >= 0 && r < 2 * K) used |= 1u << r;
    }
    BeamSlot sj{};
    bool tokj = false, actj = false;
    int cj = -1;
    if (lane < K) {
      sj = sn[lane];
      sj.score = merged[lane];
      const bool live = lane < nsel && sj.score > -INFINITY;
      cj = lane < nsel ? sel_cls[lane] : -1;
      tokj = live && cj >= 0 && cj != a.blank;
      actj = live && sj.t < T;
    }
    const uint64_t tm = __ballot(tokj), am = __ballot(actj);
    const uint64_t below = (1ull << lane) - 1ull;
    int p0 = 0, a0 = 0;
    if (lane == 0) {
      p0 = tm ? atomicAdd(a.pcnt, __popcll(tm)) : 0;
      a0 = am ? atomicAdd(a.jcnt, __popcll(am)) : 0;
    }
    p0 = __shfl(p0, 0, 64);
    a0 = __shfl(a0, 0, 64);
    if (lane < K) {
      if (tokj) {
        // the rank-th entry (slot order) not used by the old beam
        int rank = __popcll(tm & below), e = 0;
        for (; e < 2 * BEAM_MAX - 1; ++e)   // found within the first 2K: the old beam uses at most K
          if (!(used & (1u << e)) && rank-- == 0) break;
        const int at = p0 + __popcll(tm & below);
        a.psrc[at] = so[sel_par[lane]].ref;
        a.pdst[at] = base + e;
        a.ptok[at] = cj;
        sj.ref = base + e;
      }
      if (actj) a.jlist[a0 + __popcll(am & below)] = make_int4(b * a.T + sj.t, sj.ref, b * K + lane, 0);
      nw[lane] = sj;
    }
    if (lane == 0) {
      a.tcur[b] = par ^ 1;
      atomicMax(a.rounds, *a.rnow);
    }
  }
}

struct BeamEdgeArgs {
  BeamSlot* slots;
  int32_t* tcur;
  const int32_t* tlen;
  int4* jlist; int32_t* jcnt;      // [2] counters
  int32_t* pcnt; int32_t* rounds; int32_t* rnow;
  const int32_t* tr;
  int32_t* tokens; int32_t* lens; float* scores; int32_t* frames;   // end: caller's
  const float4* z; float4* zbuf; long n4;                           // stage
  int n, beam, U, Ucall, score_norm, T, q;   // q: parity of the final slots (end)
};

// One block: the start beam of every utterance and the first joint list.
__global__ __launch_bounds__(256) void beam_begin_kernel(BeamEdgeArgs a) {
  __shared__ int cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < a.n; b += 256) {
    a.tcur[b] = 0;
    for (int k = 0; k < a.beam; ++k) {
      BeamSlot s;
      s.score = k == 0 ? 0.0f : -INFINITY;
      s.t = 0; s.nsym = 0; s.len = 0; s.ref = POOL_START; s.last = -1; s.hash = 0;
      a.slots[(long)b * a.beam + k] = s;
    }
    if (a.tlen[b] > 0) a.jlist[atomicAdd(&cnt, 1)] = make_int4(b * a.T, POOL_START, b * a.beam, 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.jcnt[0] = cnt;
    a.jcnt[1] = 0;
    *a.pcnt = 0;
    *a.rounds = 0;
    *a.rnow = 0;
  }
}

__global__ __launch_bounds__(256) void beam_stage_kernel(BeamEdgeArgs a) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.n4; i += (long)gridDim.x * 256) a.zbuf[i] = a.z[i];
}

// One block per utterance: its slots ranked (normalised score, then slot; empty slots last)
// and written out.
__global__ __launch_bounds__(256) void beam_end_kernel(BeamEdgeArgs a) {
  const int b = blockIdx.x, K = a.beam;
  const int par = a.tcur[b];
  const BeamSlot* sl = a.slots + ((long)a.q * a.n + b) * K;
  const int32_t* tr = a.tr + ((long)par * a.n + b) * K * a.U;
  __shared__ int order[BEAM_MAX];
  if (threadIdx.x == 0) {
    float key[BEAM_MAX];
    int o = 0;
    for (int k = 0; k < K; ++k) {
      key[k] = a.score_norm ? sl[k].score / (float)(sl[k].len + 1) : sl[k].score;
      order[k] = k;
    }
    // insertion sort: live before empty, key descending, slot ascending
    for (int i = 1; i < K; ++i) {
      const int x = order[i];
      int j = i - 1;
      auto before = [&](int p, int q) {
        const bool lp = sl[p].score > -INFINITY, lq = sl[q].score > -INFINITY;
        if (lp != lq) return lp;
        if (!lp) return p < q;
        return key[p] > key[q] || (key[p] == key[q] && p < q);
      };
      while (j >= 0 && before(x, order[j])) { order[j + 1] = order[j]; --j; }
      order[j + 1] = x;
    }
    (void)o;
  }
  __syncthreads();
  for (int r = 0; r < K; ++r) {
    const int k = order[r];
    const bool live = sl[k].score > -INFINITY;
    const int len = live ? sl[k].len : 0;
    int32_t* dst = a.tokens + ((long)b * K + r) * a.Ucall;
    for (int i = threadIdx.x; i < a.Ucall; i += 256) dst[i] = i < len ? tr[(long)k * a.U + i] : -1;
    if (threadIdx.x == 0) {
      a.lens[b * K + r] = live ? len : -1;
      a.scores[b * K + r] = sl[k].score;
      if (a.frames) a.frames[b * K + r] = live ? sl[k].t : -1;
    }
  }
}

// ------------------------------------------------------------------------------- host side
struct BeamDims {
  int P, H, L, V, C, Cpad, K, m, S, T, U, norm, flags;
};

bool beam_dims(const cac_beam_config* c, BeamDims& d, std::string& why) {
  if (!c) { why = "config is NULL"; return false; }
  d.P = c->joint_dim; d.H = c->pred_hidden; d.L = c->pred_layers; d.V = c->vocab; d.K = c->beam;
  d.m = c->max_symbols; d.S = c->max_streams; d.T = c->max_frames; d.norm = c->score_norm; d.flags = c->flags;
  auto bad = [&](const char* msg) { why = msg; return false; };
  if (d.P < 64 || d.P > 4096 || d.P % 64) return bad("joint_dim must be a multiple of 64 in [64, 4096]");
  if (d.H < 64 || d.H > 4096 || d.H % 64) return bad("pred_hidden must be a multiple of 64 in [64, 4096]");
  if (d.L < 1 || d.L > 8) return bad("pred_layers must be in [1, 8]");
  if (d.V < 1 || d.V + 2 > 64 * BEAM_NV) return bad("vocab must be in [1, 2046]");
  if (d.K < 1 || d.K > BEAM_MAX) return bad("beam must be in [1, 8]");
  if (d.m < 1 || d.m > 16) return bad("max_symbols must be in [1, 16]");
  if (d.S < 1 || d.S > 4096) return bad("max_streams must be in [1, 4096]");
  if (d.T < 1 || d.T > 4096) return bad("max_frames must be in [1, 4096]");
  if (d.norm != 0 && d.norm != 1) return bad("score_norm must be 0 or 1");
  if (d.flags & ~(CAC_FLAG_DRY_RUN | CAC_BEAM_FLAG_WEAK_HASH)) return bad("unknown flags");
  d.C = d.V + 2;
  d.Cpad = (d.C + 63) / 64 * 64;
  d.U = d.T * d.m;
  return true;
}

struct BeamLayout {
  DecWeights w;
  size_t table, zrow, slots, tcur, tr, tlen, jlist, jcnt, psrc, pdst, ptok, pcnt, rounds, rnow, log, logits, zbuf;
  size_t cand_s, cand_c;
  size_t ph, pc, pp, total;
  size_t entries, rounds_max, lrows;
};

BeamLayout beam_layout(const BeamDims& d) {
  BeamLayout t{};
  size_t off = 0;
  auto take = [&](size_t bytes) { off = (off + 255) & ~(size_t)255; size_t o = off; off += bytes; return o; };
  const size_t H = d.H, P = d.P, S = d.S, K = d.K, L = d.L;
  t.w = dec_weight_offsets(take, d.C, H, L, P, d.Cpad);
  t.table = take((size_t)d.C * 4 * H * 4);
  t.zrow = take(4);
  t.entries = POOL_BASE + S * 2 * K;
  t.rounds_max = (size_t)d.T * (d.m + 1);
  t.slots = take(2 * S * K * sizeof(BeamSlot));
  t.tcur = take(S * 4);
  t.tr = take(2 * S * K * (size_t)d.U * 4);
  t.tlen = take(S * 4);
  // work lists padded to a multiple of 32 rows (a tile block reads its 32 entries whatever
  // the list's length)
  t.lrows = (S * K + 31) / 32 * 32;
  t.jlist = take(2 * t.lrows * 16);
  t.jcnt = take(2 * 4);
  t.psrc = take(t.lrows * 4); t.pdst = take(t.lrows * 4); t.ptok = take(t.lrows * 4);
  t.pcnt = take(4);
  t.rounds = take(4);
  t.rnow = take(4);
  t.log = take((t.rounds_max + 1) * 2 * 4);
  t.logits = take(S * K * (size_t)d.Cpad * 4);
  t.cand_s = take(S * 64 * 4);
  t.cand_c = take(S * 64 * 4);
  t.zbuf = take(S * (size_t)d.T * P * 4);
  t.ph = take(t.entries * L * H * 4);
  t.pc = take(t.entries * L * H * 4);
  t.pp = take(t.entries * P * 4);
  t.total = take(0);
  return t;
}

thread_local std::string g_beam_error;

}  // namespace

struct cac_beam {
  BeamDims d;
  BeamLayout lay;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  bool dry = false;
  std::string err;
  bool profiling = false;
  Profiler prof;
  std::vector<int32_t> tlen_host;
  struct Graph {
    hipGraph_t g = nullptr;
    hipGraphExec_t exec = nullptr;
  };
  bool use_graph = true;
  std::map<uint64_t, Graph> graphs;   // one group of rounds per (utterances, frames)
  ~cac_beam() {
    for (auto& kv : graphs) {
      if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
      if (kv.second.g) (void)hipGraphDestroy(kv.second.g);
    }
  }
  template <class T> T* P(size_t off) const { return (T*)(ws + off); }
  int fail(int code, const std::string& m) { err = m; return code; }
};

namespace {

BeamTileArgs beam_tile_base(cac_beam* c, int n, int T) {
  const BeamDims& d = c->d;
  const BeamLayout& y = c->lay;
  BeamTileArgs t{};
  t.psrc = c->P<int32_t>(y.psrc); t.pdst = c->P<int32_t>(y.pdst); t.ptok = c->P<int32_t>(y.ptok);
  t.zbuf = c->P<float>(y.zbuf);
  t.logits = c->P<float>(y.logits);
  t.ph = c->P<float>(y.ph); t.pc = c->P<float>(y.pc); t.pp = c->P<float>(y.pp);
  t.embed = c->P<float>(y.w.embed); t.table = c->P<float>(y.table);
  t.L = d.L; t.H = d.H; t.P = d.P; t.C = d.C; t.T = T; t.n = n; t.beam = d.K;
  return t;
}

// 1-D grid of a tile launch: one block per tile of the largest list (8 * ceil(gx / 8) per row
// tile), at most BEAM_TILE_BLOCKS; blocks loop over the tiles of the rows the list holds.
constexpr unsigned BEAM_TILE_BLOCKS = 512;
dim3 beam_grid(int gx, unsigned row_tiles) {
  return dim3(std::min<unsigned>((unsigned)((gx + 7) / 8 * 8) * row_tiles, BEAM_TILE_BLOCKS));
}

// The predictor kernels over the list (count) of (parent entry, new entry, label) rows.
void beam_predictor(cac_beam* c, Launcher& L, const BeamTileArgs& base, const int32_t* count, int max_rows, int round) {
  const BeamDims& d = c->d;
  const BeamLayout& y = c->lay;
  BeamTileArgs t = base;
  t.count = count;
  t.round = round;
  const unsigned prow = (unsigned)((max_rows + 31) / 32);
  for (int l = 0; l < d.L; ++l) {
    t.layer = l;
    t.K = l == 0 ? d.H : 2 * d.H;
    t.N = 4 * d.H;
    t.ldw = 2 * d.H;
    // the first layer contracts h with the W_hh inputs only (its input half is the token table)
    t.W = c->P<float>(y.w.lstm_w) + (size_t)l * 2 * d.H * 4 * d.H + (l == 0 ? (size_t)d.H : 0);
    t.bias = c->P<float>(y.w.lstm_b) + (size_t)l * 4 * d.H;
    L.tag("beam_lstm", 0.0, 0.0);
    t.gx = 4 * d.H / 32;
    L.launch(l == 0 ? (const void*)&beam_tile_kernel<BM_LSTM0> : (const void*)&beam_tile_kernel<BM_LSTM>,
             beam_grid(t.gx, prow), dim3(64 * BEAM_TW), 0, &t);
  }
  t.K = d.H; t.N = d.P; t.ldw = d.H; t.W = c->P<float>(y.w.proj_w); t.bias = c->P<float>(y.w.proj_b);
  L.tag("beam_proj", 0.0, 0.0);
  t.gx = d.P / 32;
  L.launch((const void*)&beam_tile_kernel<BM_PROJ>, beam_grid(t.gx, prow), dim3(64 * BEAM_TW), 0, &t);
}

// Rounds r0 .. r0 + count - 1 (parity from the round index).
void beam_rounds(cac_beam* c, Launcher& L, int n, int T, int r0, int count) {
  const BeamDims& d = c->d;
  const BeamLayout& y = c->lay;
  const BeamTileArgs base = beam_tile_base(c, n, T);
  int4* jlist = c->P<int4>(y.jlist);
  int32_t* jcnt = c->P<int32_t>(y.jcnt);
  const int nk = n * d.K;
  for (int i = 0; i < count && L.err == hipSuccess; ++i) {
    const int j = r0 + i, q = j & 1;
    BeamTileArgs jt = base;
    jt.count = jcnt + q;
    jt.jlist = jlist + (size_t)q * y.lrows;
    jt.clr0 = jcnt + (q ^ 1);
    jt.clr1 = c->P<int32_t>(y.pcnt);
    jt.rnow = c->P<int32_t>(y.rnow);
    jt.log = c->profiling ? c->P<int32_t>(y.log) : nullptr;
    jt.round = j;
    jt.K = d.P; jt.N = d.Cpad; jt.ldw = d.P; jt.W = c->P<float>(y.w.out_w); jt.bias = c->P<float>(y.w.out_b);
    L.tag("beam_joint", 0.0, 0.0);
    jt.gx = d.Cpad / 32;
    L.launch((const void*)&beam_tile_kernel<BM_JOINT>, beam_grid(jt.gx, (unsigned)((nk + 31) / 32)), dim3(64 * BEAM_TW),
             0, &jt);
    BeamSelArgs s{};
    s.logits = c->P<float>(y.logits); s.slots = c->P<BeamSlot>(y.slots); s.tcur = c->P<int32_t>(y.tcur);
    s.tr = c->P<int32_t>(y.tr); s.tlen = c->P<int32_t>(y.tlen);
    s.jlist = jlist + (size_t)(q ^ 1) * y.lrows; s.jcnt = jcnt + (q ^ 1);
    s.psrc = c->P<int32_t>(y.psrc); s.pdst = c->P<int32_t>(y.pdst); s.ptok = c->P<int32_t>(y.ptok);
    s.pcnt = c->P<int32_t>(y.pcnt); s.rounds = c->P<int32_t>(y.rounds); s.rnow = c->P<int32_t>(y.rnow);
    s.n = n; s.beam = d.K; s.C = d.C; s.Cpad = d.Cpad; s.U = d.U; s.blank = d.V; s.m = d.m; s.q = q; s.T = T;
    s.weak_hash = (d.flags & CAC_BEAM_FLAG_WEAK_HASH) ? 1 : 0;
    s.cand_s = c->P<float>(y.cand_s); s.cand_c = c->P<int32_t>(y.cand_c);
    L.tag("beam_cand", 0.0, 0.0);
    L.launch((const void*)&beam_cand_kernel, dim3(n * d.K), dim3(256), 0, &s);
    L.tag("beam_select", 0.0, 0.0);
    L.launch((const void*)&beam_select_kernel, dim3(n), dim3(256), 0, &s);
    BeamTileArgs pt = base;
    pt.log = jt.log;
    beam_predictor(c, L, pt, c->P<int32_t>(y.pcnt), nk, j);
  }
}

hipError_t beam_group_graph(cac_beam* c, int n, int T) {
  const uint64_t key = ((uint64_t)n << 20) | (uint64_t)T;
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    cac_beam::Graph gr;
    hipError_t e = hipGraphCreate(&gr.g, 0);
    if (e != hipSuccess) return e;
    Launcher L;
    L.stream = c->stream;
    L.graph = gr.g;
    beam_rounds(c, L, n, T, 0, BEAM_GROUP);
    if (L.err != hipSuccess) { (void)hipGraphDestroy(gr.g); return L.err; }
    e = hipGraphInstantiate(&gr.exec, gr.g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(gr.g); return e; }
    it = c->graphs.emplace(key, gr).first;
  }
  return hipGraphLaunch(it->second.exec, c->stream);
}

// Profiled call: give every recorded launch its algorithmic flops and weight bytes from the
// rows each round saw; launches with no rows are named "<kernel>/idle".
hipError_t beam_profile_fix(cac_beam* c, size_t first, int rounds) {
  const BeamDims& d = c->d;
  std::vector<int32_t> lg((size_t)2 * rounds);
  hipError_t e = hipMemcpyAsync(lg.data(), c->ws + c->lay.log, lg.size() * 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return e;
  std::vector<Profiler::Rec>& rec = c->prof.pending;
  const size_t per = 3 + (size_t)d.L + 1;
  if (rec.size() < first + 2 + (size_t)rounds * per) return hipSuccess;
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
    const double jr = lg[2 * j], pr = lg[2 * j + 1];
    set("beam_joint", jr, 2.0 * P * C, P * d.Cpad * 4);
    set("beam_cand", jr, 0.0, 0.0);
    set("beam_select", jr, 0.0, 0.0);
    for (int l = 0; l < d.L; ++l) set("beam_lstm", pr, 2.0 * (l ? 2 : 1) * H * 4 * H, (l ? 2 : 1) * H * 4 * H * 4);
    set("beam_proj", pr, 2.0 * H * P, H * P * 4);
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t cac_beam_param_count(const cac_beam_config* cfg) {
  BeamDims d;
  std::string why;
  return beam_dims(cfg, d, why) ? dec_param_count(d.C, d.H, d.L, d.P) : 0;
}

size_t cac_beam_workspace_bytes(const cac_beam_config* cfg) {
  BeamDims d;
  std::string why;
  return beam_dims(cfg, d, why) ? beam_layout(d).total : 0;
}

const char* cac_beam_last_error(const cac_beam* ctx) { return ctx ? ctx->err.c_str() : g_beam_error.c_str(); }

int32_t cac_beam_create(const cac_beam_config* cfg, const float* h_params, size_t n_params, void* d_workspace,
                        size_t ws_bytes, void* hip_stream, cac_beam** out) {
  g_beam_error.clear();
  if (!out) { g_beam_error = "out is NULL"; return CAC_EINVAL; }
  *out = nullptr;
  BeamDims d;
  if (!beam_dims(cfg, d, g_beam_error)) return CAC_EINVAL;
  if (!h_params) { g_beam_error = "parameter array is NULL"; return CAC_EINVAL; }
  const size_t np = dec_param_count(d.C, d.H, d.L, d.P);
  if (n_params != np) {
    g_beam_error = "expected " + std::to_string(np) + " parameters, got " + std::to_string(n_params);
    return CAC_EINVAL;
  }
  const bool dry = (d.flags & CAC_FLAG_DRY_RUN) != 0;
  const BeamLayout lay = beam_layout(d);
  if (!dry) {
    if (!d_workspace) { g_beam_error = "workspace is NULL"; return CAC_EINVAL; }
    if (((uintptr_t)d_workspace) & 255) { g_beam_error = "workspace must be 256-byte aligned"; return CAC_EINVAL; }
    if (ws_bytes < lay.total) { g_beam_error = "workspace too small: need " + std::to_string(lay.total) + " bytes"; return CAC_ENOMEM; }
  }
  cac_beam* c = new cac_beam();
  c->d = d; c->lay = lay; c->ws = (char*)d_workspace; c->stream = (hipStream_t)hip_stream; c->dry = dry;
  if (dry) { *out = c; return CAC_OK; }
  kernels_init();
  std::vector<uint8_t> buf(lay.w.end, 0);
  dec_repack(h_params, lay.w, d.C, d.H, d.L, d.P, d.Cpad, buf.data());
  hipError_t e = hipMemcpyAsync(c->ws, buf.data(), buf.size(), hipMemcpyHostToDevice, c->stream);
  // the zero state (entry 0), then the start state (entry 1): the predictor on blank from zero
  const size_t lh = (size_t)d.L * d.H * 4;
  if (e == hipSuccess) e = hipMemsetAsync(c->ws + lay.ph, 0, lh, c->stream);
  if (e == hipSuccess) e = hipMemsetAsync(c->ws + lay.pc, 0, lh, c->stream);
  const int32_t row[4] = {1, POOL_ZERO, POOL_START, d.V};   // count, parent, new entry, token
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.pcnt, &row[0], 4, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.psrc, &row[1], 4, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.pdst, &row[2], 4, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.ptok, &row[3], 4, hipMemcpyHostToDevice, c->stream);
  const int32_t cc = (int32_t)d.C;
  if (e == hipSuccess) e = hipMemcpyAsync(c->ws + lay.zrow, &cc, 4, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) {
    Launcher L;
    L.stream = c->stream;
    BeamTileArgs t = beam_tile_base(c, 1, 1);
    // first layer's input table: embed[token] W_ih + b_ih + b_hh for every class
    t.K = d.H; t.N = 4 * d.H; t.ldw = 2 * d.H; t.W = c->P<float>(lay.w.lstm_w); t.bias = c->P<float>(lay.w.lstm_b);
    t.count = c->P<int32_t>(lay.zrow);
    L.tag("beam_table", 0.0, 0.0);
    t.gx = 4 * d.H / 32;
    L.launch((const void*)&beam_tile_kernel<BM_TABLE>, beam_grid(t.gx, (unsigned)((d.C + 31) / 32)), dim3(64 * BEAM_TW), 0,
             &t);
    beam_predictor(c, L, beam_tile_base(c, 1, 1), c->P<int32_t>(lay.pcnt), 1, 0);
    e = L.err;
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    g_beam_error = std::string("HIP error during create: ") + hipGetErrorString(e);
    delete c;
    return CAC_EHIP;
  }
  *out = c;
  return CAC_OK;
}

int32_t cac_beam_decode(cac_beam* c, int32_t n, const int32_t* h_lengths, int32_t nf, const float* d_z,
                        int32_t max_steps, int32_t* d_tokens, int32_t* d_lengths, float* d_scores, int32_t* d_frames) {
  if (!c) return CAC_EINVAL;
  const BeamDims& d = c->d;
  const BeamLayout& y = c->lay;
  if (n < 1 || n > d.S) return c->fail(CAC_EINVAL, "n_streams must be in [1, max_streams]");
  if (nf < 1 || nf > d.T) return c->fail(CAC_EINVAL, "n_frames must be in [1, max_frames]");
  if (!h_lengths) return c->fail(CAC_EINVAL, "lengths array is NULL");
  for (int i = 0; i < n; ++i)
    if (h_lengths[i] < 0 || h_lengths[i] > nf)
      return c->fail(CAC_EINVAL, "length of utterance " + std::to_string(i) + " out of [0, n_frames]");
  if (max_steps < 0) return c->fail(CAC_EINVAL, "max_steps must be >= 0");
  if (!d_z || !d_tokens || !d_lengths || !d_scores) return c->fail(CAC_EINVAL, "z, tokens, lengths or scores pointer is NULL");
  if ((uintptr_t)d_z & 15) return c->fail(CAC_EINVAL, "z must be 16-byte aligned");
  if (c->dry) return c->fail(CAC_ENODEV, "dry-run context: no device work");
  const hipError_t pe = hipStreamQuery(c->stream);
  if (pe != hipSuccess && pe != hipErrorNotReady)
    return c->fail(CAC_EHIP, std::string("asynchronous device error from earlier work: ") + hipGetErrorString(pe));
  c->tlen_host.assign(h_lengths, h_lengths + n);
  hipError_t e = hipMemcpyAsync(c->ws + y.tlen, c->tlen_host.data(), (size_t)n * 4, hipMemcpyHostToDevice, c->stream);
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("length upload failed: ") + hipGetErrorString(e));
  Launcher L;
  L.stream = c->stream;
  size_t first = 0;
  if (c->profiling) {
    c->prof.drain();
    L.prof = &c->prof;
    first = c->prof.pending.size();
  }
  BeamEdgeArgs ea{};
  ea.slots = c->P<BeamSlot>(y.slots); ea.tcur = c->P<int32_t>(y.tcur); ea.tlen = c->P<int32_t>(y.tlen);
  ea.jlist = c->P<int4>(y.jlist); ea.jcnt = c->P<int32_t>(y.jcnt); ea.pcnt = c->P<int32_t>(y.pcnt);
  ea.rounds = c->P<int32_t>(y.rounds); ea.rnow = c->P<int32_t>(y.rnow); ea.tr = c->P<int32_t>(y.tr);
  ea.tokens = d_tokens; ea.lens = d_lengths; ea.scores = d_scores; ea.frames = d_frames;
  ea.z = (const float4*)d_z; ea.zbuf = c->P<float4>(y.zbuf); ea.n4 = (long)n * nf * d.P / 4;
  ea.n = n; ea.beam = d.K; ea.U = d.U; ea.Ucall = nf * d.m; ea.score_norm = d.norm; ea.T = nf;
  L.tag("beam_begin", 0.0, 0.0);
  L.launch((const void*)&beam_begin_kernel, dim3(1), dim3(256), 0, &ea);
  L.tag("beam_stage", 0.0, 0.0);
  L.launch((const void*)&beam_stage_kernel, dim3((unsigned)std::min<long>((ea.n4 + 255) / 256, 2048)), dim3(256), 0, &ea);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  const int limit = max_steps > 0 ? std::min(max_steps, nf * (d.m + 1)) : nf * (d.m + 1);
  int r = 0;
  while (r < limit) {
    const int g = std::min(BEAM_GROUP, limit - r);
    if (g == BEAM_GROUP && c->use_graph && !c->profiling && (r & 1) == 0) {
      e = beam_group_graph(c, n, nf);
      if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("graph replay failed: ") + hipGetErrorString(e));
    } else {
      beam_rounds(c, L, n, nf, r, g);
      if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
    }
    r += g;
    if (r >= limit) break;
    int32_t left = 0;
    e = hipMemcpyAsync(&left, c->ws + y.jcnt + (size_t)(r & 1) * 4, 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("device error during the search: ") + hipGetErrorString(e));
    if (left == 0) break;
  }
  ea.q = r & 1;   // every round moved every utterance's slots to the next parity
  L.tag("beam_end", 0.0, 0.0);
  L.launch((const void*)&beam_end_kernel, dim3(n), dim3(256), 0, &ea);
  if (L.err != hipSuccess) return c->fail(CAC_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(L.err));
  int32_t rounds = 0;
  e = hipMemcpyAsync(&rounds, c->ws + y.rounds, 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("device error during the search: ") + hipGetErrorString(e));
  if (c->profiling) {
    e = beam_profile_fix(c, first, r);
    if (e != hipSuccess) return c->fail(CAC_EHIP, std::string("profiling: ") + hipGetErrorString(e));
  }
  return rounds;
}

int32_t cac_beam_set_graph(cac_beam* c, int32_t enable) {
  if (!c) return CAC_EINVAL;
  c->use_graph = enable != 0;
  return CAC_OK;
}

int32_t cac_beam_profile(cac_beam* c, int32_t enable) {
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

int32_t cac_beam_profile_read(cac_beam* c, int32_t max_entries, char* names, int32_t name_len, int64_t* launches,
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

int32_t cac_beam_destroy(cac_beam* c) {
  delete c;
  return CAC_OK;
}

}  // extern "C"

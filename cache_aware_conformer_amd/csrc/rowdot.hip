// Dense products of at most two rows: one stream's chunk of two frames (or two streams of one
// frame each), the shape every dense layer of a single-stream chunk step has
// ("True streaming encode — implementation spec", "Per-chunk flow", step 3: FF1, the
// attention projections, the conv module and FF2 of every layer).
//
// At two rows a product is a pass over the weight matrix: each wave owns one or two output
// units (a column, or a GLU value/gate column pair) and reads their weight rows once, 16 bytes
// per lane along K. The two A rows are read straight into registers by every wave (they are a
// few KB and stay in cache), so there is no LDS and no barrier. Every load of the kernel,
// weights, A rows, LayerNorm parameters and epilogue operands, is issued first and without
// conditions (indices are clamped into range and unused values discarded), so a launch pays one
// memory latency. A fused LayerNorm (one or two in a row) is computed by every wave on its own
// copy of the rows. Operand mode, epilogue and K are compile-time, so each instance holds only
// its own code.
//
// The per-lane partial sums of all (unit, column, row) outputs of a wave are reduced together:
// each exchange step halves the number of values a lane carries while pairing lanes, so NV sums
// take NV - 1 + (6 - log2 NV) exchanges instead of 6 NV, and value v ends up on the lanes whose
// bits 5, 4, ... spell v from its lowest bit up. The exchanges are register-to-register (the
// gfx950 lane-half swaps and DPP row patterns), never a round trip through LDS.
#include "common.h"

#include <algorithm>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

enum AMode { AM_PLAIN = 0, AM_LN = 1, AM_LN2 = 2 };
constexpr int RD_ROWS = 2;   // rows per launch
constexpr int RD_TAPS = 16;  // depthwise taps the GLU epilogue takes

// N consecutive elements at p as float (p aligned to the load size).
template <typename T, int N>
__device__ __forceinline__ void load_vals(const T* p, float* f) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 v = ((const f32x4*)p)[i];
      f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
    }
  } else if constexpr (N == 4) {
    const u32x2 v = *(const u32x2*)p;
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const u32x4 v = ((const u32x4*)p)[i];
      const unsigned int u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
        f[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
    }
  }
}

template <typename TW>
__device__ __forceinline__ void unpack_w(const u32x4& r, float* f) {
  if constexpr (sizeof(TW) == 4) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  } else {
    const unsigned int u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[2 * j] = __uint_as_float(u[j] << 16); f[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u); }
  }
}

// 64-lane totals of NV per-lane values; afterwards every lane holds the total of value
// v(lane) = sum_j ((lane >> (5 - j)) & 1) << j. Halving steps pair lanes on bit 5, 4, 3 (a lane
// keeps one of each pair of values and adds its partner's copy of it), then plain sums over the
// remaining bits.
template <int NV>
__device__ __forceinline__ float fold_sums(const float (&s)[NV], int lane) {
  static_assert(NV == 2 || NV == 4 || NV == 8, "two, four or eight values");
  float y[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) y[i] = s[i];
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) y[i] = pair_sum32(y[2 * i], y[2 * i + 1]);
  if constexpr (NV >= 4) {
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) y[i] = pair_sum16(y[2 * i], y[2 * i + 1]);
  }
  if constexpr (NV == 8) {
    const bool hi = (lane & 8) != 0;
    y[0] = (hi ? y[1] : y[0]) + dpp<DPP_MIRROR16>(hi ? y[0] : y[1]);
  }
  float v = y[0];
  if constexpr (NV < 4) v = pair_sum16(v, v);
  if constexpr (NV < 8) v += dpp<DPP_MIRROR16>(v);
  v += dpp<DPP_MIRROR8>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_XOR1>(v);
  return v;
}

// Mean and 1/std (eps 1e-5) of two register rows, one pass: sums of the rows shifted by their
// first element (which keeps the variance free of cancellation for rows far from zero mean).
struct RowStats { float mean[2], rstd[2]; };
__device__ __forceinline__ RowStats stats_from(const float (&t)[4], int lane, float c0, float c1, float inv_n) {
  const float f = fold_sums<4>(t, lane);  // s0 on lane 0, s1 on 32, q0 on 16, q1 on 48
  const float s0 = lane_value(f, 0) * inv_n, s1 = lane_value(f, 32) * inv_n;
  const float q0 = lane_value(f, 16) * inv_n, q1 = lane_value(f, 48) * inv_n;
  RowStats r;
  r.mean[0] = c0 + s0; r.mean[1] = c1 + s1;
  r.rstd[0] = rsqrtf(fmaxf(q0 - s0 * s0, 0.0f) + 1e-5f);
  r.rstd[1] = rsqrtf(fmaxf(q1 - s1 * s1, 0.0f) + 1e-5f);
  return r;
}

// LayerNorm of both register rows.
template <int PER>
__device__ __forceinline__ void ln_two_rows(float (&x)[RD_ROWS][PER], const float (&g)[PER], const float (&b)[PER],
                                            int lane, float inv_k) {
  const float c0 = lane_value(x[0][0], 0), c1 = lane_value(x[1][0], 0);
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const float d0 = x[0][j] - c0, d1 = x[1][j] - c1;
    t[0] += d0; t[1] += d1; t[2] += d0 * d0; t[3] += d1 * d1;
  }
  const RowStats st = stats_from(t, lane, c0, c1, inv_k);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int j = 0; j < PER; ++j) x[r][j] = (x[r][j] - st.mean[r]) * st.rstd[r] * g[j] + b[j];
}

template <typename T>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (sizeof(T) == 2) return bf2f(f2bf(v));
  return v;
}

// Four int8 weights (one 32-bit word, lowest byte first) as floats.
__device__ __forceinline__ void unpack_i8(unsigned int r, float* f) {
  f[0] = (float)((int)(r << 24) >> 24);
  f[1] = (float)((int)(r << 16) >> 24);
  f[2] = (float)((int)(r << 8) >> 24);
  f[3] = (float)((int)r >> 24);
}

// y[m][n] = A[m] . W[n] for m < M <= 2, with the operand transform AM and the epilogue EK.
// K = KCH * 64 * (16 / sizeof(TW)); UPW output units per wave; blocks of 4 waves.
// WQ: the weights are int8 codes [N][K] followed by one float32 scale per row (N of them); TW
// (float) stays the type of activations and caches, each lane reads its VEC codes of a chunk as
// one 32-bit word, and the row's scale multiplies the lane's partial sums.
template <typename TW, typename TA, int KCH, int UPW, int AM, int EK, int WQ = 0>
__global__ __launch_bounds__(256) void rowdot_kernel(GemmArgs a) {
  static_assert(!WQ || sizeof(TW) == 4, "int8 weights with float32 activations");
  constexpr int VEC = 16 / sizeof(TW);
  constexpr int K = KCH * 64 * VEC;
  constexpr int PER = KCH * VEC;  // elements of each row this lane holds
  constexpr bool GLU = EK == EPI_GLU_DW;
  constexpr int COLS = GLU ? 2 : 1;
  constexpr int NV = UPW * RD_ROWS * COLS;
  constexpr int LG = NV == 2 ? 1 : NV == 4 ? 2 : 3;
  static_assert(NV == (1 << LG), "two, four or eight sums per lane");
  static_assert(!GLU || UPW == 1, "the depthwise epilogue puts one tap on each lane of a 16-lane row group");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
  const int units = GLU ? a.N / 2 : a.N;
  const int u0 = wave * UPW;
  if (u0 >= units) return;
  const int M = a.M;
  const EpiArgs& e = a.epi;
  const TW* W = (const TW*)a.W;

  // this lane's output after the fold: value v = ((u * RD_ROWS) + r) * COLS + c
  int v = 0;
#pragma unroll
  for (int j = 0; j < LG; ++j) v |= ((lane >> (5 - j)) & 1) << j;
  const int c_l = v % COLS, r_l = (v / COLS) % RD_ROWS, u_l = v / (COLS * RD_ROWS);
  const int unit = u0 + u_l;
  const bool writer = unit < units && r_l < M && c_l == 0 && (lane & ((64 >> LG) - 1)) == 0;
  const int un = min(unit, units - 1), m = min(r_l, M - 1);
  // the two rows' operand offsets (row 0 is at offset 0): no runtime division
  const long a_off1 = a.amap.group == 1 ? (long)a.amap.group_stride : (long)a.amap.row_stride;

  // stream, frame and absolute position of this lane's row: loaded first, so that the ring
  // loads that depend on them wait for these two loads only, not for the weight stream
  int sid = 0, frame = 0, pos = 0;
  if constexpr (EK == EPI_QKV || GLU) {
    const int s = e.cv.nf == 1 ? m : 0;  // m / nf for m < 2
    frame = m - s * e.cv.nf;
    sid = e.cv.ids[s];
    pos = e.cv.cpos[s] + frame;
  }
  // ---------------------------------------------------------------- every global read
  u32x4 wr[UPW][COLS][WQ ? 1 : KCH];
  unsigned int wq[UPW][COLS][WQ ? KCH : 1];
  float wsc[UPW][COLS];
  const signed char* Wq = (const signed char*)a.W;
  const float* wscale = (const float*)(Wq + (long)a.N * K);
#pragma unroll
  for (int u = 0; u < UPW; ++u)
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      const int uw = min(u0 + u, units - 1);
      const int col = GLU ? glu_a_col(uw) + 32 * c : uw;
      if constexpr (WQ) {
#pragma unroll
        for (int k = 0; k < KCH; ++k)
          wq[u][c][k] = __builtin_nontemporal_load((const unsigned int*)(Wq + (long)col * K + (k * 64 + lane) * VEC));
        wsc[u][c] = wscale[col];
      } else {
#pragma unroll
        for (int k = 0; k < KCH; ++k) wr[u][c][k] = __builtin_nontemporal_load((const u32x4*)(W + (long)col * K + (k * 64 + lane) * VEC));
      }
    }
  float x[RD_ROWS][PER];
#pragma unroll
  for (int r = 0; r < RD_ROWS; ++r) {
    const TA* ar = (const TA*)a.A + (min(r, M - 1) ? a_off1 : 0);
#pragma unroll
    for (int k = 0; k < KCH; ++k) load_vals<TA, VEC>(ar + (k * 64 + lane) * VEC, &x[r][k * VEC]);
  }
  float g1[PER], b1[PER], g0[PER], b0[PER];
  if constexpr (AM != AM_PLAIN) {
#pragma unroll
    for (int k = 0; k < KCH; ++k) {
      load_vals<float, VEC>(a.ln_g + (k * 64 + lane) * VEC, &g1[k * VEC]);
      load_vals<float, VEC>(a.ln_b + (k * 64 + lane) * VEC, &b1[k * VEC]);
      if constexpr (AM == AM_LN2) {
        load_vals<float, VEC>(a.pre_g + (k * 64 + lane) * VEC, &g0[k * VEC]);
        load_vals<float, VEC>(a.pre_b + (k * 64 + lane) * VEC, &b0[k * VEC]);
      }
    }
  }

  float bias0 = 0.0f, bias1 = 0.0f;
  if (e.bias) {
    bias0 = e.bias[un];
    if constexpr (GLU) bias1 = e.bias[e.D + un];
  }
  // residual base, and the residual rows for their LayerNorm statistics
  float base = 0.0f;
  f32x4 rx[RD_ROWS][4];
  int rch = 0;  // float4 chunks per lane of a residual row
  if constexpr (EK == EPI_RESID) {
    const float* src = a.res_src ? a.res_src : (const float*)e.out;
    base = src[(long)m * e.ldo + un];
    if (a.res_g) {
      rch = e.ldo / 256;
#pragma unroll
      for (int r = 0; r < RD_ROWS; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rx[r][j] = *(const f32x4*)(a.res_src + (long)min(r, M - 1) * e.ldo + (min(j, rch - 1) * 64 + lane) * 4);
    }
  }
  // depthwise operands. After the fold a GLU wave (one unit) holds each (row, value/gate) total
  // on a 16-lane group, so lane o of a row's group takes tap o: the tap weight and, for taps
  // behind the rows of this call, the ring row o positions back (loaded after the stream info)
  float dw_tap = 0.0f, dw_old = 0.0f, dwb = 0.0f;
  const int tap = lane & 15;
  if constexpr (GLU) {
    const int T = a.dw_taps, Rc = e.Rc;
    const int oa = tap < T ? tap : T - 1;  // T - 1 < Rc: one wrap below
    const float tw = a.dw_w[(long)(T - 1 - oa) * e.D + un];
    dw_tap = tap < T ? tw : 0.0f;
    int sl = pos % Rc - oa;
    sl += sl < 0 ? Rc : 0;
    const float rv = ld<TW>((const TW*)e.cring + cring_idx(sid, sl, un, e.D, Rc));
    dw_old = (tap >= 1 && tap < T && tap > frame && pos - tap >= 0) ? rv : 0.0f;
    dwb = a.dw_b[un];
  }
  int orow = m;
  if constexpr (EK == EPI_F32) {
    if (e.omap) {  // m / ogroup and m % ogroup for m < 2
      const int q = e.ogroup == 1 ? m : 0;
      orow = e.omap[q] * e.ostride + (m - q * e.ogroup);
    }
  }

  // ---------------------------------------------------------------- operand transforms
  if constexpr (AM == AM_LN2) ln_two_rows<PER>(x, g0, b0, lane, 1.0f / (float)K);
  if constexpr (AM != AM_PLAIN) ln_two_rows<PER>(x, g1, b1, lane, 1.0f / (float)K);
  if constexpr (sizeof(TW) == 2 && (AM != AM_PLAIN || sizeof(TA) == 4)) {
#pragma unroll
    for (int r = 0; r < RD_ROWS; ++r)
#pragma unroll
      for (int j = 0; j < PER; ++j) x[r][j] = round_to<TW>(x[r][j]);
  }
  float rmean = 0.0f, rrstd = 1.0f;
  if constexpr (EK == EPI_RESID) {
    if (a.res_g) {
      const float c0 = lane_value(rx[0][0].x, 0), c1 = lane_value(rx[1][0].x, 0);
      float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < rch) {
          const f32x4 d0 = rx[0][j] - c0, d1 = rx[1][j] - c1;
          t[0] += d0.x + d0.y + d0.z + d0.w;
          t[1] += d1.x + d1.y + d1.z + d1.w;
          t[2] += d0.x * d0.x + d0.y * d0.y + d0.z * d0.z + d0.w * d0.w;
          t[3] += d1.x * d1.x + d1.y * d1.y + d1.z * d1.z + d1.w * d1.w;
        }
      const RowStats st = stats_from(t, lane, c0, c1, 1.0f / (float)e.ldo);
      rmean = r_l == 0 ? st.mean[0] : st.mean[1];
      rrstd = r_l == 0 ? st.rstd[0] : st.rstd[1];
    }
  }

  // ---------------------------------------------------------------- products and fold
  float p[NV];
#pragma unroll
  for (int u = 0; u < UPW; ++u)
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      float acc[RD_ROWS] = {0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        float w[VEC];
        if constexpr (WQ) unpack_i8(wq[u][c][k], w);
        else unpack_w<TW>(wr[u][c][k], w);
#pragma unroll
        for (int r = 0; r < RD_ROWS; ++r)
#pragma unroll
          for (int j = 0; j < VEC; ++j) acc[r] += w[j] * x[r][k * VEC + j];
      }
#pragma unroll
      for (int r = 0; r < RD_ROWS; ++r) p[(u * RD_ROWS + r) * COLS + c] = WQ ? acc[r] * wsc[u][c] : acc[r];
    }
  const float val = fold_sums<NV>(p, lane);

  // ---------------------------------------------------------------- epilogue
  if constexpr (GLU) {
    // value lanes (bit 5 clear) take the gate from lane + 32; the row before in the same call
    // (frame - 1) sits on lane - 16 (bit 4 is the row bit)
    const float gate = xor32(val, lane);
    const float g = round_to<TW>((val + bias0) * sigmoid_f(gate + bias1));
    const float prev = xor16(g, lane);
    const float xin = tap == 0 ? g : (tap == 1 && frame >= 1 ? prev : dw_old);
    float conv = dw_tap * xin;  // this lane's tap; summed over the 16 lanes of the row's group
    conv += dpp<DPP_MIRROR16>(conv);
    conv += dpp<DPP_MIRROR8>(conv);
    conv += dpp<DPP_XOR2>(conv);
    conv += dpp<DPP_XOR1>(conv);
    if (writer) {
      st<TW>((TW*)e.cring + cring_idx(sid, pos % e.Rc, unit, e.D, e.Rc), g);
      st<TW>((TW*)e.out + (long)m * e.ldo + unit, silu_f(dwb + conv));
    }
  } else if (writer) {
    const float y = val + bias0;
    if constexpr (EK == EPI_SILU) {
      st<TW>((TW*)e.out + (long)m * e.ldo + unit, silu_f(y));
    } else if constexpr (EK == EPI_RESID) {
      float b = base;
      if (a.res_g) b = (b - rmean) * rrstd * a.res_g[unit] + a.res_b[unit];
      ((float*)e.out)[(long)m * e.ldo + unit] = b + e.alpha * y;
    } else if constexpr (EK == EPI_F32) {
      ((float*)e.out)[(long)orow * e.ldo + unit] = y;
    } else if constexpr (EK == EPI_QKV) {
      const int which = (unit >= e.D) + (unit >= 2 * e.D), c = unit - which * e.D;
      if (which == 0) {
        e.qbuf[(long)m * e.D + c] = y;
      } else {
        const int slot = pos % e.R;
        const int lg = 31 - __clz(e.hd);  // head sizes are powers of two
        TW* ring = (TW*)(which == 1 ? e.kring : e.vring);
        st<TW>(ring + (((long)sid * e.H + (c >> lg)) * e.R + slot) * e.hd + (c & (e.hd - 1)), y);
      }
    }
  }
}

// ------------------------------------------------------------------------------ dispatch
template <typename TW, typename TA, int AM, int EK, int UPW, int WQ>
const void* pick_kch(int kch) {
  constexpr int KMAX = AM == AM_PLAIN ? (sizeof(TW) == 4 ? 8 : 4) : (sizeof(TW) == 4 ? 4 : 2);
  if (kch == 1) return (const void*)&rowdot_kernel<TW, TA, 1, UPW, AM, EK, WQ>;
  if (kch == 2) return (const void*)&rowdot_kernel<TW, TA, 2, UPW, AM, EK, WQ>;
  if constexpr (KMAX >= 4)
    if (kch == 4) return (const void*)&rowdot_kernel<TW, TA, 4, UPW, AM, EK, WQ>;
  if constexpr (KMAX >= 8)
    if (kch == 8) return (const void*)&rowdot_kernel<TW, TA, 8, UPW, AM, EK, WQ>;
  return nullptr;
}

template <typename TW, typename TA, int AM, int EK, int WQ>
const void* pick_upw(int upw, int kch) {
  if constexpr (AM == AM_PLAIN || EK == EPI_GLU_DW) return upw == 1 ? pick_kch<TW, TA, AM, EK, 1, WQ>(kch) : nullptr;
  else return upw == 2 ? pick_kch<TW, TA, AM, EK, 2, WQ>(kch) : pick_kch<TW, TA, AM, EK, 1, WQ>(kch);
}

// The instantiated mixes: LayerNorm'ed float rows into SiLU (also after a second LayerNorm),
// QKV, GLU + depthwise and float32 (joint) epilogues; plain compute-dtype rows into the
// residual epilogue.
template <typename TW, typename TA, int WQ = 0>
const void* pick_mode(int am, int ek, int upw, int kch) {
  if constexpr (sizeof(TA) == 4) {
    if (am == AM_LN2) return ek == EPI_SILU ? pick_upw<TW, TA, AM_LN2, EPI_SILU, WQ>(upw, kch) : nullptr;
    if (am == AM_LN) {
      switch (ek) {
        case EPI_SILU: return pick_upw<TW, TA, AM_LN, EPI_SILU, WQ>(upw, kch);
        case EPI_QKV: return pick_upw<TW, TA, AM_LN, EPI_QKV, WQ>(upw, kch);
        case EPI_GLU_DW: return pick_upw<TW, TA, AM_LN, EPI_GLU_DW, WQ>(upw, kch);
        case EPI_F32: return pick_upw<TW, TA, AM_LN, EPI_F32, WQ>(upw, kch);
        default: return nullptr;
      }
    }
  }
  if constexpr (sizeof(TA) == sizeof(TW)) {
    if (am == AM_PLAIN && ek == EPI_RESID) return pick_upw<TW, TA, AM_PLAIN, EPI_RESID, WQ>(upw, kch);
  }
  return nullptr;
}

struct Plan {
  const void* fn = nullptr;
  dim3 grid;
  int wpb = 4;  // waves per block
};

Plan plan(const GemmArgs& a, int dtype) {
  Plan p;
  if (a.M < 1 || a.M > RD_ROWS || a.a_dw) return p;
  const int wsz = dtype == DT_BF16 ? 2 : 4, vec = 16 / wsz;  // int8 weights keep the float32 lane layout
  if (a.K % (64 * vec)) return p;
  const int kch = a.K / (64 * vec);
  const int ek = a.epi.kind;
  int am = AM_PLAIN;
  if (a.ln_g) am = a.pre_g ? AM_LN2 : AM_LN;
  else if (a.pre_g) return p;
  if (am != AM_PLAIN && !a.ln_b) return p;
  if (am == AM_LN2 && !a.pre_b) return p;
  if (ek == EPI_RESID && a.res_g && (a.epi.ldo % 256 || a.epi.ldo > 1024 || !a.res_src || !a.res_b)) return p;
  if (ek == EPI_GLU_DW && (a.dw_taps < 1 || a.dw_taps > RD_TAPS || !a.dw_w || !a.dw_b || a.N % 64)) return p;
  const bool a_float = dtype != DT_BF16 || a.a_f32;
  const int units = ek == EPI_GLU_DW ? a.N / 2 : a.N;
  // two units per wave only where that still leaves a wave per SIMD; 4-wave blocks only where
  // they still cover every CU
  // (the GLU + depthwise epilogue needs one unit per wave: 16-lane groups, a lane per tap)
  const int upw = (am != AM_PLAIN && units >= 2048 && ek != EPI_GLU_DW) ? 2 : 1;
  const int waves = (units + upw - 1) / upw;
  p.wpb = waves >= 1024 ? 4 : 1;
  if (dtype == DT_F32) p.fn = pick_mode<float, float>(am, ek, upw, kch);
  else if (dtype == DT_I8W) p.fn = pick_mode<float, float, 1>(am, ek, upw, kch);
  else if (a_float) p.fn = pick_mode<bf16_t, float>(am, ek, upw, kch);
  else p.fn = pick_mode<bf16_t, bf16_t>(am, ek, upw, kch);
  p.grid = dim3((waves + p.wpb - 1) / p.wpb);
  return p;
}

}  // namespace

bool rowdot_supported(const GemmArgs& a, int dtype) { return plan(a, dtype).fn != nullptr; }

bool rowdot_launch(Launcher& L, const GemmArgs& a, int dtype) {
  const Plan p = plan(a, dtype);
  if (!p.fn) return false;
  L.tag(dtype == DT_F32 ? "gemm_tworow_f32" : dtype == DT_I8W ? "gemm_tworow_i8w" : "gemm_tworow_bf16",
        gemm_bytes(a, dtype == DT_F32 ? 4 : dtype == DT_I8W ? 1 : 2), 2.0 * a.M * a.N * a.K);
  GemmArgs args = a;
  L.launch(p.fn, p.grid, dim3(64 * p.wpb), 0, &args);
  return true;
}

// Shared device/host definitions of the chunk-step library: element types, kernel argument
// structs (every kernel takes exactly one POD struct, so a launch sequence can be recorded as
// HIP graph kernel nodes and re-pointed later), and the launch wrappers kernels.hip exports.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>
#include <vector>

typedef uint16_t bf16_t;  // bfloat16 storage

// DT_I8W: float32 activations and caches, int8 weights with a float32 scale per output row
enum DType { DT_F32 = 0, DT_BF16 = 1, DT_I8W = 2 };

// ------------------------------------------------------------------------ element helpers
__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
// float -> bf16, round to nearest even, NaN kept a (quiet) NaN: the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32), checked bit for bit against the software rounding over
// random bit patterns, ties, subnormals, infinities and NaNs
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_hw{(__bf16)lo, (__bf16)hi});
}
template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

// The logistic function through the hardware reciprocal (v_rcp_f32, 1 ulp): 1 + e^-x is at
// least 1, so no denormal input reaches it, and the 5-instruction form replaces the 14 of an
// IEEE division in every activation epilogue.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ------------------------------------------------------------------------ register exchanges
// Cross-lane exchanges that never go through LDS: v_readlane, the gfx950 lane-half swaps
// (v_permlane32_swap / v_permlane16_swap) and DPP row patterns.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
// pair_sum32(a, b): lanes 0..31 get a[L] + a[L + 32], lanes 32..63 get b[L - 32] + b[L]
// (pair_sum16 likewise across the two 16-lane halves of each 32).
__device__ __forceinline__ float pair_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// value of lane L ^ 32 / L ^ 16
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor16(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
// value of lane L ^ 15 (row mirror), L ^ 7 (half-row mirror), L ^ 2, L ^ 1
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_MIRROR16 = 0x140, DPP_MIRROR8 = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1;

// sum / max over all 64 lanes, the result on every lane
__device__ __forceinline__ float wave_total(float v) {
  v += dpp<DPP_MIRROR16>(v);
  v += dpp<DPP_MIRROR8>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_XOR1>(v);
  v = pair_sum16(v, v);
  return pair_sum32(v, v);
}
__device__ __forceinline__ float wave_top(float v) {
  v = fmaxf(v, dpp<DPP_MIRROR16>(v));
  v = fmaxf(v, dpp<DPP_MIRROR8>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ------------------------------------------------------------------------ row addressing
// Row m of a logical [M][K] operand lives at base + (m / group) * group_stride +
// (m % group) * row_stride elements. Plain row-major: group = M (or any value > M),
// row_stride = lda. Used for strided im2col views and for picking emitted rows.
struct RowMap {
  int group, group_stride, row_stride;
  __host__ __device__ __forceinline__ long off(int m) const {
    return (long)(m / group) * group_stride + (long)(m % group) * row_stride;
  }
};

// ------------------------------------------------------------------------ per-call view
// What a kernel needs to know about the streams of the current call: row m of the call's
// activations belongs to call slot s = m / nf (stream id ids[s]) and is that stream's frame
// m % nf, at absolute position pos[ids[s]] + m % nf.
struct CallView {
  const int32_t* ids;  // [n_streams] stream ids of this call (device)
  const int32_t* pos;  // [max_streams] stream positions (device)
  int nf;              // frames per stream in this call
  int n_streams;
  int32_t* cpos;       // [n_streams] pos[ids[s]] of this call, written by the call's first kernel
};

// ------------------------------------------------------------------------ epilogues
enum EpiKind {
  EPI_STORE = 0,   // out_t[m][n] = acc + b                       (compute dtype)
  EPI_SILU = 1,    // out_t[m][n] = silu(acc + b)                 (compute dtype)
  EPI_RELU_FE = 2, // out_t[m][n] = relu(acc + b), 0 for rows before the stream start
  EPI_RESID = 3,   // x[m][n] += alpha * (acc + b)                (float32 residual)
  EPI_F32 = 4,     // out_f[row_out(m)][n] = acc + b              (float32)
  EPI_QKV = 5,     // q -> qbuf (f32); k, v -> ring slots of the row's position
  EPI_GLU = 6,     // a*sigmoid(b) of GLU-packed column pairs -> conv ring slot
  EPI_GLU_DW = 7,  // EPI_GLU, then the causal depthwise conv + SiLU of the call's rows over the
                   // ring -> out_t[m][c] (compute dtype; GemmArgs dw_*): two-row kernel, and the
                   // MFMA kernel (kernel size <= 9; the streams whose rows cross a multiple of
                   // 64 rows are left to launch_dwconv_straddle)
  EPI_PART = 8,    // part[z][m][n] = acc over k-range z (float32, no bias): split-K partial of
                   // the MFMA kernel, summed by resid_ln (GemmArgs ksplit, EpiArgs pstride)
  EPI_SILU_KEEP = 9,  // EPI_SILU with write-back stores that leave the rows in L2 (MFMA kernel;
                      // the other kernels take it as EPI_SILU)
  EPI_RESID_KEEP = 10,  // EPI_RESID likewise
  EPI_RESID_LNS = 11,   // EPI_RESID_KEEP that also writes what the next LayerNorm needs (MFMA
                        // kernel, 64-column tiles): the rows centred on a per-row shift in the
                        // compute dtype (xc) and each row's (mean, M2) over every 64-column tile
  EPI_LNC = 0x100,      // flag on EPI_SILU(_KEEP) / EPI_QKV / EPI_GLU (MFMA kernel): A holds the
                        // centred rows, W the gain-scaled weights, and the epilogue finishes the
                        // LayerNorm from the tile statistics before the kind's own work
};

// GLU packing of the pointwise-1 weight rows: packed row (c / 32) * 64 + c % 32 holds value
// channel c, 32 rows further its gate (so a 32-wide tile holds matching value/gate halves).
__host__ __device__ __forceinline__ int glu_a_col(int c) { return (c >> 5) * 64 + (c & 31); }

// Depthwise conv input ring of one layer: [S][D / 32][Rc][32] in the compute dtype (D a multiple
// of 32). A stream's rows of one 32-channel block lie together, so a reader of a few positions
// of a block (the GLU tile's conv) takes whole cache lines. Element (slot, channel c) of ring
// row group g (a stream of one layer, or layer l x S + stream across the layers):
__host__ __device__ __forceinline__ long cring_idx(long g, int slot, int c, int D, int Rc) {
  return g * Rc * D + ((long)(c >> 5) * Rc + slot) * 32 + (c & 31);
}

struct EpiArgs {
  int kind;
  const float* bias;  // [N] (may be null)
  void* out;          // EPI_STORE/SILU/RELU_FE: compute dtype; EPI_RESID/F32: float
  int ldo;
  float alpha;
  long pstride;       // EPI_PART: elements between the partials of consecutive k-ranges
  // EPI_F32 output row remap (lookahead emits a subset of rows): row_out = omap[m / ogroup] *
  // ostride + m % ogroup when omap != null
  const int32_t* omap;
  int ogroup, ostride;
  // EPI_RELU_FE: rows (s, j) with j < fe_neg_rows are zeroed for streams at position 0
  int fe_rows_per_stream, fe_neg_rows;
  // EPI_QKV / EPI_GLU
  CallView cv;
  float* qbuf;          // [M][D] float32
  void* kring;          // [S][H][R][hd] of this layer (compute dtype)
  void* vring;
  void* cring;          // conv ring of this layer (cring_idx layout, compute dtype)
  int D, H, hd, R, Rc;
  // LayerNorm carried through the products (EPI_RESID_LNS writes, EPI_LNC reads):
  //   lns[t * lns_ld + m] = (mean, sum of squared deviations) of row m's columns 64 t .. 64 t + 63
  //   lns_shift[m] = the shift s_m the centred rows xc[m] = x[m] - s_m were taken around (the
  //     row's mean before the residual update)
  // and the consumer's output column n is rstd (acc - (mean - s) c1[n]) + c2[n] with
  // c1[n] = sum_k w'[n][k] of its gain-scaled weights w'[n][k] = g[k] w[n][k] and
  // c2[n] = sum_k b[k] w[n][k] + bias[n] (for GLU in the bias order: values, then gates); its
  // blocks of the first column tile also write each row's mean to lns_mean (the next shift)
  float2* lns;
  const float* lns_shift;
  float* lns_mean;
  int lns_ld, lns_ntl;
  void* xc;               // EPI_RESID_LNS: [M][ldo] centred rows (compute dtype)
  const float* lnc_c1;
  const float* lnc_c2;
};

// ------------------------------------------------------------------------ kernel args
struct GemmArgs {
  int M, N, K;           // C[M][N] = A[M][K] . W[N][K]^T ; for EPI_GLU N counts packed columns
  const void* A;         // compute dtype, or float32 when a_f32
  RowMap amap;
  const void* W;         // [N][K] compute dtype
  int a_f32;             // A is float32: LayerNorm'ed (ln_g != null) and/or rounded to the
  const float* ln_g;     // compute dtype before the product; the MFMA path first writes that
  const float* ln_b;     // operand to a_scratch ([M][K], compute dtype)
  void* a_scratch;
  // small-M kernel only:
  const float* pre_g;    // LayerNorm the A rows with (pre_g, pre_b) before (ln_g, ln_b)
  const float* pre_b;
  int a_dw;              // A rows are SiLU(depthwise conv over the ring) (see DwArgs fields)
  const void* dw_ring;   // conv ring of the layer (cring_idx layout, width K)
  const float* dw_w;     // [taps][K] (also EPI_GLU_DW's taps, K = the GLU channels)
  const float* dw_b;     // [K]
  int dw_taps, dw_Rc;
  const float* res_src;  // EPI_RESID: out = LN(res_src rows; res_g, res_b) + alpha (acc + b)
  const float* res_g;    // (res_g null: out = res_src + alpha (acc + b)); out != res_src
  const float* res_b;
  int upb;               // small-M kernel: output units (columns, or GLU channels) per block
  int ksplit;            // MFMA kernel with EPI_PART: K in ksplit equal ranges (0 or 1: one)
  int xrg;               // MFMA kernel, set by its dispatch: XCD tile rectangles (see there)
  EpiArgs epi;
};

struct LnArgs {
  const float* x;  // [M][D]
  void* y;         // [M][D] (compute dtype, or float32 when in place)
  const float* g;
  const float* b;
  int M, D;
  int out_f32;     // 1: y is float32
};

// Residual update and LayerNorm(s) of whole rows, one wave per row (D a multiple of 256, at
// most 1024):  v = sum_z part[z][m] (z in order) + bias;  x[m] += alpha * v  (nparts > 0);
// x[m] = LN(x[m]; go, bo) when go;  y[m] = LN(x[m]; gn, bn) (gn) or x[m] (gn null) when y.
struct ResLnArgs {
  const float* part;  // [nparts][M][D] split-K partials (nparts 0: no residual update)
  long pstride;       // elements between consecutive partials
  int nparts;
  const float* bias;  // [D] or null
  float alpha;
  float* x;           // [M][D] float32 residual stream, updated in place
  const float* go;    // LayerNorm applied to x in place (null: none)
  const float* bo;
  const float* gn;    // LayerNorm of the y rows (null: y = x)
  const float* bn;
  void* y;            // [M][D] compute dtype (null: not written)
  int M, D;
  int keep;           // rows in XCD-contiguous eighths and y by write-back stores (see the kernel)
  float* mean;        // mean[m] = mean of the final x row (null: not written): the shift the
                      // next residual product centres its rows around
};

struct AttnArgs {
  CallView cv;
  const float* q;       // [M][D] float32 (q rows of the call)
  const void* kring;    // layer base [S][H][R][hd]
  const void* vring;
  const float* posproj; // layer base [H][nrel][hd]
  const float* pos_u;   // [H][hd]
  const float* pos_v;
  void* o;              // [M][D] compute dtype
  int D, H, R, Lc, chunk, right, lookahead, rel_lo, nrel;
  float scale;
  const void* posproj_bf;  // bf16 copy of posproj (MFMA attention kernel), or null
};

struct DwArgs {
  CallView cv;
  const void* cring;   // conv ring of the layer (cring_idx layout)
  const float* w;      // [K][D] taps
  const float* b;      // [D]
  void* e;             // [M][D] compute dtype
  int D, K, Rc;
};

struct InputArgs {      // x[m][c] = in[m][c] (float32 residual from compute dtype input)
  CallView cv;          // also fills cv.cpos, then advances the streams' positions by adv
  const void* in;
  float* x;
  int M, D;
  int32_t* pos;         // [max_streams] positions, advanced by adv (the same array as cv.pos)
  int adv;
};

struct FeWindowArgs {   // win[s] = [tail(14) || mel_new(16)]; tail = last 14 of win
  CallView cv;
  const void* mel;      // [n][mel_per_chunk][bins]
  void* tail;           // [S][mel_tail][bins]
  void* win;            // [n][mel_tail + mel_per_chunk][bins]
  int bins, mel_tail, mel_new;
};

// 2-D front end, one 3 x 3 stride-2 stage over channels-last maps [n][Tin][Fin][C] (bf16),
// frequency padded by one column on each side, time valid (output row r reads input rows
// 2r .. 2r+2): stage 1 (cin1: a single input channel, the mel window [n][Tin][Fin], + ReLU,
// rows r < neg of streams at position 0 zeroed) or depthwise (C channels, no activation).
struct Fe2dArgs {
  CallView cv;
  const void* in;
  void* out;
  const float* w;      // [9][C] taps
  const float* b;      // [C]
  int Tin, Fin, Tout, Fout, C, cin1, neg;
};

// 2-D front end stage 1 and the depthwise stage after it in one launch (fe2d_s1dw_kernel): the
// stage-1 map [T1][F1][C] of each stream stays on chip; the depthwise output [n][T2][F2][C]
// (bf16) is written. Stage 1 as Fe2dArgs with cin1 (ReLU, rows r < neg1 zero for streams at
// position 0), the depthwise stage as Fe2dArgs without (no activation).
struct Fe2dS1DwArgs {
  CallView cv;
  const void* in;      // [n][Tin][Fin] the mel window (bf16)
  void* out;           // [n][T2][F2][C]
  const float* w1;     // [9][C] stage-1 taps
  const float* b1;     // [C]
  const float* w2;     // [9][C] depthwise taps
  const float* b2;     // [C]
  int Tin, Fin, T1, F1, T2, F2, C, neg1;
};

struct CopyRowsArgs {    // out[row_out(m)][c] = x[amap(m) + c], row_out as in EPI_F32
  const float* x;
  RowMap amap;
  float* out;
  const int32_t* omap;
  int ogroup, ostride, M, D;
};

struct CvtArgs {         // y[m][k] = bf16(x[amap(m) + k])
  const float* x;
  RowMap amap;
  void* y;
  int M, K;
};

struct FillArgs {       // p[0 .. n) = v
  float* p;
  long n;
  float v;
};

struct AdvanceArgs {    // pos[ids[s]] += adv, pend[ids[s]] += dpend
  const int32_t* ids;
  int32_t* pos;
  int32_t* pend;
  int n, adv, dpend;
};

struct PosProjArgs {    // table[l][h][r][d] = sum_e PE(rel_lo + r, e) Wpos_l[e][h*hd + d]
  const float* wpos;    // [L][D][D]
  float* table;         // [L][H][nrel][hd]
  int L, D, H, hd, rel_lo, nrel;
};

// Every stream's state blob starts with STATE_HDR 32-bit words: STATE_MAGIC, STATE_VERSION and
// a 64-bit hash of the config it was made with (written on export, checked on import).
constexpr int STATE_HDR = 4;
constexpr uint32_t STATE_MAGIC = 0x53434143u;  // "CACS"
constexpr uint32_t STATE_VERSION = 1u;

struct StateArgs {      // reset / import / export of whole streams
  const int32_t* ids;   // [n]
  const int32_t* hpos;  // [n] positions (import) ; out for export via pos array
  const int32_t* hpend; // [n]
  int32_t* pos;         // [S]
  int32_t* pend;        // [S]
  void* kring; void* vring; void* cring; void* tail; void* x0;  // whole state regions
  float* blob;          // [n][state_floats]
  int n, S, L, D, H, hd, R, Rc, Lc, Kc, tail_rows, bins, nla, Rx;
  long state_floats;     // per stream, header included
  int dtype, poison;
  uint32_t hdr[STATE_HDR];  // header export writes
};

struct LaStoreArgs {    // lookahead: append new frames to each stream's pending ring
  CallView cv;          // call streams; nf = frames per push
  const int32_t* pend;
  const void* in;       // [n][nf][D]
  void* x0;             // [S][Rx][D]
  int D, Rx;
};
struct LaGatherArgs {   // lookahead: x rows of a pass from the pending ring
  CallView cv;          // compute streams; nf = frames per pass
  const void* x0;
  float* x;
  int D, Rx;
};

// ------------------------------------------------------------------------ launcher
// Kernels are launched through a Launcher: either straight onto a stream, or appended to a
// HIP graph as a chain of kernel nodes (node handles are kept so pointer arguments can be
// re-pointed before each replay).
// Optional per-kernel timing (direct launches): each kernel is launched with a start and a stop
// HIP event bound to its own dispatch (hipExtLaunchKernel), so the elapsed time is the kernel's
// execution on the launch stream, without the host's submission gaps; aggregated by kernel name
// together with the launch's algorithmic bytes and flops.
struct Profiler {
  struct Rec { int name; double bytes, flops; hipEvent_t a, b; };
  std::vector<hipEvent_t> free_ev;
  std::vector<Rec> pending;
  std::vector<std::string> names;
  std::vector<long> launches;
  std::vector<double> ms, bytes, flops;
  hipError_t err = hipSuccess;
  int name_id(const char* n);
  hipEvent_t get();
  void drain();   // synchronise pending events, accumulate, recycle
  void clear();
  ~Profiler();
};

// A kernel node recorded into a graph, with a copy of its argument bytes so pointer arguments
// can be re-pointed before a replay.
struct NodeRec {
  hipGraphNode_t node;
  hipKernelNodeParams p;
  std::vector<char> args;
  std::string name;     // kernel tag ("family/role")
  double bytes, flops;  // algorithmic bytes and flops of the launch
  // attention: the part of bytes and flops that grows with the K/V rows the call reads (per row),
  // and those rows as of the push that last used the node, so that a replay at another cache
  // fill can restate them
  double kv_bytes = 0.0, kv_flops = 0.0, kv_rows = 0.0;
};

struct Launcher {
  hipStream_t stream = nullptr;
  std::vector<NodeRec>* rec = nullptr;  // record mode: nodes appended here
  hipGraph_t graph = nullptr;        // non-null: record instead of launch
  hipGraphNode_t last = nullptr;
  hipGraphNode_t last_node = nullptr;  // node of the most recent launch (record mode)
  hipError_t err = hipSuccess;
  Profiler* prof = nullptr;          // direct launches only
  const char* tag_name = "kernel";   // set by the wrappers before each launch
  const char* role = nullptr;        // optional role of the next dense product ("qkv", ...)
  char name_buf[64];
  double tag_bytes = 0.0, tag_flops = 0.0;
  double tag_kv_rows = 0.0, tag_kv_bytes = 0.0, tag_kv_flops = 0.0;
  // after tag(): how much of its bytes and flops is per K/V row read, and the call's rows
  void tag_kv(double rows, double bytes_per_row, double flops_per_row) {
    tag_kv_rows = rows;
    tag_kv_bytes = bytes_per_row;
    tag_kv_flops = flops_per_row;
  }
  void tag(const char* n, double bytes, double flops) {
    tag_name = n;
    if (role) {
      snprintf(name_buf, sizeof(name_buf), "%s/%s", n, role);
      tag_name = name_buf;
      role = nullptr;
    }
    tag_bytes = bytes;
    tag_flops = flops;
  }
  void launch_raw(const void* fn, dim3 grid, dim3 block, size_t shmem, void* args, size_t args_size);
  template <class A> void launch(const void* fn, dim3 grid, dim3 block, size_t shmem, A* args) {
    launch_raw(fn, grid, block, shmem, (void*)args, sizeof(A));
  }
};

// ------------------------------------------------------------------------ wrappers
void launch_gemm(Launcher& L, const GemmArgs& a, int dtype, int path);
// Two-row kernel: true when it takes this product (M <= 2 and a supported operand/epilogue mix);
// rowdot_launch returns false, launching nothing, otherwise.
bool rowdot_supported(const GemmArgs& a, int dtype);
bool rowdot_launch(Launcher& L, const GemmArgs& a, int dtype);
double gemm_bytes(const GemmArgs& a, int wsz);
void launch_ln(Launcher& L, const LnArgs& a, int dtype);
void launch_cvt(Launcher& L, const CvtArgs& a);  // y = bf16(x rows)
// false (nothing launched) when D is not a multiple of 256 up to 1024 or nparts is not 0, 2 or 4
bool launch_resid_ln(Launcher& L, const ResLnArgs& a, int dtype);
void launch_attention(Launcher& L, const AttnArgs& a, int dtype, int hd);
void launch_dwconv(Launcher& L, const DwArgs& a, int dtype);
// the conv of the streams whose rows cross a multiple of 64 rows (bf16), after a product with
// EPI_GLU_DW; false (nothing launched) when no stream crosses one
bool launch_dwconv_straddle(Launcher& L, const DwArgs& a);
void launch_input(Launcher& L, const InputArgs& a, int dtype);
void launch_copy_rows(Launcher& L, const CopyRowsArgs& a);
void kernels_init();
void launch_fe_window(Launcher& L, const FeWindowArgs& a, int dtype);
void launch_fe2d(Launcher& L, const Fe2dArgs& a);
// false (nothing launched) where the stage-1 map does not fit the kernel's LDS (F1 > 64) or C is
// not a multiple of 32
bool launch_fe2d_s1dw(Launcher& L, const Fe2dS1DwArgs& a);
void launch_advance(Launcher& L, const AdvanceArgs& a);
void launch_fill(Launcher& L, const FillArgs& a);
void launch_posproj(Launcher& L, const PosProjArgs& a);
void launch_state(Launcher& L, const StateArgs& a, int op);  // 0 reset, 1 import, 2 export
void launch_la_store(Launcher& L, const LaStoreArgs& a, int dtype);
void launch_la_gather(Launcher& L, const LaGatherArgs& a, int dtype);
size_t attention_shmem(int nf, int R, int nrel, int hd, int esz);

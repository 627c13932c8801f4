// HIP kernels (gfx950) of the cache-aware streaming Conformer chunk step.
//
// Dense products: a small-M kernel that streams each weight row once per launch with all rows
// of the call held in LDS (LayerNorm of those rows fused into its prologue), and a bf16 MFMA
// tile kernel (v_mfma_f32_32x32x16_bf16, LDS-staged A and W tiles) for many rows. Both end in
// the same fused epilogues: bias, SiLU, ReLU, scaled residual add, QKV scatter into the K/V
// rings, GLU into the depthwise ring.
//
// Caches are rings indexed by absolute position: K/V of position q sits in slot q mod R with
// R = att_left + frames per call, the depthwise input (GLU output) of position q in slot
// q mod Rc with Rc = (dw_kernel - 1) + frames per call. New rows are written by the producing
// GEMM's epilogue before any reader of the same call runs, and the extra slots guarantee the
// rows a call still reads are never the ones it overwrites.
#include "common.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <climits>

// =============================================================================== launcher
int Profiler::name_id(const char* n) {
  for (size_t i = 0; i < names.size(); ++i)
    if (names[i] == n) return (int)i;
  names.emplace_back(n);
  launches.push_back(0);
  ms.push_back(0.0);
  bytes.push_back(0.0);
  flops.push_back(0.0);
  return (int)names.size() - 1;
}
hipEvent_t Profiler::get() {
  if (free_ev.empty() && pending.size() >= 2048) drain();
  if (!free_ev.empty()) { hipEvent_t e = free_ev.back(); free_ev.pop_back(); return e; }
  hipEvent_t e = nullptr;
  hipError_t r = hipEventCreate(&e);
  if (r != hipSuccess && err == hipSuccess) err = r;
  return e;
}
void Profiler::drain() {
  for (Rec& r : pending) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && err == hipSuccess) err = e;
    launches[r.name] += 1;
    ms[r.name] += t;
    bytes[r.name] += r.bytes;
    flops[r.name] += r.flops;
    free_ev.push_back(r.a);
    free_ev.push_back(r.b);
  }
  pending.clear();
}
void Profiler::clear() {
  drain();
  names.clear(); launches.clear(); ms.clear(); bytes.clear(); flops.clear();
  err = hipSuccess;
}
Profiler::~Profiler() {
  drain();
  for (hipEvent_t e : free_ev) (void)hipEventDestroy(e);
}

void Launcher::launch_raw(const void* fn, dim3 grid, dim3 block, size_t shmem, void* args, size_t args_size) {
  if (err != hipSuccess) return;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return;
  void* kp[1] = {args};
  if (!graph) {
    if (prof) {
      hipEvent_t a = prof->get(), b = prof->get();
      if (a && b) {
        err = hipExtLaunchKernel(fn, grid, block, kp, shmem, stream, a, b, 0);
        if (err == hipSuccess) prof->pending.push_back({prof->name_id(tag_name), tag_bytes, tag_flops, a, b});
      } else {
        err = hipLaunchKernel(fn, grid, block, kp, shmem, stream);
      }
      tag_bytes = tag_flops = 0.0;
      tag_kv_rows = tag_kv_bytes = tag_kv_flops = 0.0;
      return;
    }
    err = hipLaunchKernel(fn, grid, block, kp, shmem, stream);
    tag_bytes = tag_flops = 0.0;
    tag_kv_rows = tag_kv_bytes = tag_kv_flops = 0.0;
    return;
  }
  hipKernelNodeParams p = {};
  p.func = const_cast<void*>(fn);
  p.gridDim = grid;
  p.blockDim = block;
  p.sharedMemBytes = (unsigned)shmem;
  p.kernelParams = kp;
  p.extra = nullptr;
  hipGraphNode_t node;
  err = hipGraphAddKernelNode(&node, graph, last ? &last : nullptr, last ? 1 : 0, &p);
  if (err == hipSuccess) {
    last = last_node = node;
    if (rec) {
      NodeRec r;
      r.node = node;
      r.p = p;
      r.p.kernelParams = nullptr;
      r.args.assign((const char*)args, (const char*)args + args_size);
      r.name = tag_name;
      r.bytes = tag_bytes;
      r.flops = tag_flops;
      r.kv_rows = tag_kv_rows;
      r.kv_bytes = tag_kv_bytes;
      r.kv_flops = tag_kv_flops;
      rec->push_back(std::move(r));
    }
  }
  tag_bytes = tag_flops = 0.0;
  tag_kv_rows = tag_kv_bytes = tag_kv_flops = 0.0;
}

// =============================================================================== epilogue
// One output element (row m, packed column n) of a dense product, value v = accumulator.
template <typename T>
__device__ __forceinline__ void epi_one(const EpiArgs& e, int m, int n, float v) {
  switch (e.kind) {
    case EPI_STORE: {
      if (e.bias) v += e.bias[n];
      st<T>((T*)e.out + (long)m * e.ldo + n, v);
    } break;
    case EPI_SILU: {
      if (e.bias) v += e.bias[n];
      st<T>((T*)e.out + (long)m * e.ldo + n, silu_f(v));
    } break;
    case EPI_RELU_FE: {
      if (e.bias) v += e.bias[n];
      int s = m / e.fe_rows_per_stream, j = m % e.fe_rows_per_stream;
      bool before_start = e.cv.cpos[s] == 0 && j < e.fe_neg_rows;
      st<T>((T*)e.out + (long)m * e.ldo + n, before_start ? 0.0f : fmaxf(v, 0.0f));
    } break;
    case EPI_RESID: {
      if (e.bias) v += e.bias[n];
      float* x = (float*)e.out + (long)m * e.ldo + n;
      *x += e.alpha * v;
    } break;
    case EPI_F32: {
      if (e.bias) v += e.bias[n];
      long row = e.omap ? (long)e.omap[m / e.ogroup] * e.ostride + m % e.ogroup : m;
      ((float*)e.out)[row * e.ldo + n] = v;
    } break;
    case EPI_QKV: {
      if (e.bias) v += e.bias[n];
      int which = n / e.D, c = n % e.D;
      if (which == 0) {
        e.qbuf[(long)m * e.D + c] = v;
      } else {
        int s = m / e.cv.nf, i = m % e.cv.nf;
        int id = e.cv.ids[s];
        int slot = (e.cv.cpos[s] + i) % e.R;
        int h = c / e.hd, d = c % e.hd;
        T* ring = (T*)(which == 1 ? e.kring : e.vring);
        st<T>(ring + (((long)id * e.H + h) * e.R + slot) * e.hd + d, v);
      }
    } break;
    default: break;
  }
}

// GLU pair: a (value column) and b (gate column) of channel c.
template <typename T>
__device__ __forceinline__ void epi_glu(const EpiArgs& e, int m, int c, float va, float vb) {
  va += e.bias[c];
  vb += e.bias[e.D + c];
  float g = va * sigmoid_f(vb);
  int s = m / e.cv.nf, i = m % e.cv.nf;
  int id = e.cv.ids[s];
  int slot = (e.cv.cpos[s] + i) % e.Rc;
  st<T>((T*)e.cring + cring_idx(id, slot, c, e.D, e.Rc), g);
}


// =============================================================================== small-M GEMM
// C[M][N] = A[M][K] W[N][K]^T for few rows (MR per block). Each wave owns whole output units
// (a column, or a GLU value/gate column pair) and issues the 16-byte loads of all their weight
// rows before anything else, so HBM latency overlaps the A prologue: the block's rows of A are
// staged in LDS as float, optionally formed from the depthwise ring (A = SiLU(dwconv)), then
// LayerNorm'ed (an optional earlier LayerNorm first) and rounded to bf16 for bf16 weights.
// KCH > 0: K == KCH * 64 * (16 / sizeof(TW)) and weights sit in registers; KCH == 0: generic K.
template <typename TW> __device__ __forceinline__ void wunpack(const uint4& r, float* f);
template <> __device__ __forceinline__ void wunpack<float>(const uint4& r, float* f) {
  f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}
template <> __device__ __forceinline__ void wunpack<bf16_t>(const uint4& r, float* f) {
  const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = __uint_as_float(u[i] << 16); f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u); }
}

template <int KCH, bool GLU> struct GemvShape {
  static constexpr int COLS = GLU ? 2 : 1;
  static constexpr int UMAX = KCH > 0 ? (8 / (COLS * KCH) > 0 ? 8 / (COLS * KCH) : 1) : 1;
  static constexpr int NR = KCH > 0 ? UMAX * COLS * KCH : 1;
};

constexpr int GEMV_LPL = 16;  // LayerNorm parameters held per lane: K <= 1024

// LayerNorm of one LDS row with this lane's gains/shifts in registers (k = lane + 64 j).
__device__ __forceinline__ void row_ln_regs(float* row, int K, const float* g, const float* b, int lane) {
  const int per = K / 64;
  float v[GEMV_LPL];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < GEMV_LPL; ++j) { v[j] = j < per ? row[lane + 64 * j] : 0.0f; s += v[j]; }
  const float mean = wave_sum(s) / (float)K;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < GEMV_LPL; ++j) if (j < per) { const float d = v[j] - mean; q += d * d; }
  const float rstd = rsqrtf(wave_sum(q) / (float)K + 1e-5f);
#pragma unroll
  for (int j = 0; j < GEMV_LPL; ++j) if (j < per) row[lane + 64 * j] = (v[j] - mean) * rstd * g[j] + b[j];
}

// Small-M dense product. Every global read the block will need is issued in one phase at the
// start (weights, A rows, LayerNorm parameters, epilogue biases and residual bases, the rows'
// stream slots), so one memory latency is paid per launch instead of one per dependent step.
template <typename TW, typename TA, int MR, int KCH, bool GLU>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs a) {
  extern __shared__ float sm[];
  using Sh = GemvShape<KCH, GLU>;
  constexpr int VEC = 16 / sizeof(TW);
  constexpr int COLS = Sh::COLS, UMAX = Sh::UMAX, NR = Sh::NR;
  constexpr int UE = KCH > 0 ? UMAX : 1;  // units whose epilogue operands are prefetched
  const int K = a.K;
  float* sA = sm;              // [MR][K]
  float* stats = sm + MR * K;  // [MR][2] mean, rstd of the residual base rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * MR;
  const int mr = min(MR, a.M - m0);
  const int units = GLU ? a.N / 2 : a.N;
  const int upw = a.upb;
  const int u0 = (blockIdx.x * 4 + wave) * upw;
  const TW* W = (const TW*)a.W;
  const EpiArgs& e = a.epi;
  const int D = e.ldo;  // residual row length for EPI_RESID

  // ================= phase 0: issue every global load
  // (a) weight rows of this wave's units
  uint4 wr[NR];
  if constexpr (KCH > 0) {
#pragma unroll
    for (int u = 0; u < UMAX; ++u)
#pragma unroll
      for (int c = 0; c < COLS; ++c)
#pragma unroll
        for (int k = 0; k < KCH; ++k) {
          const int unit = u0 + u;
          const bool ok = u < upw && unit < units;
          const int col = GLU ? glu_a_col(unit) + 32 * c : unit;
          wr[(u * COLS + c) * KCH + k] = ok ? *(const uint4*)(W + (long)col * K + (k * 64 + lane) * VEC) : make_uint4(0u, 0u, 0u, 0u);
        }
  }
  // (b) LayerNorm parameters of this lane's columns
  float lg[GEMV_LPL], lb[GEMV_LPL], pg[GEMV_LPL], pb[GEMV_LPL];
  const int per = K / 64;
#pragma unroll
  for (int j = 0; j < GEMV_LPL; ++j) {
    const bool ok = j < per;
    lg[j] = (ok && a.ln_g) ? a.ln_g[lane + 64 * j] : 0.0f;
    lb[j] = (ok && a.ln_g) ? a.ln_b[lane + 64 * j] : 0.0f;
    pg[j] = (ok && a.pre_g) ? a.pre_g[lane + 64 * j] : 0.0f;
    pb[j] = (ok && a.pre_g) ? a.pre_b[lane + 64 * j] : 0.0f;
  }
  // (c) epilogue operands of this lane's row (lane < mr) for each prefetched unit
  const int m_lane = m0 + (lane < mr ? lane : 0);
  int row_slot_pos = 0, row_id = 0;  // stream id and position of this lane's row
  if (lane < mr && (e.kind == EPI_QKV || GLU || e.kind == EPI_RELU_FE)) {
    const int sidx = (e.kind == EPI_RELU_FE ? m_lane / e.fe_rows_per_stream : m_lane / e.cv.nf);
    row_id = e.cv.ids[sidx];
    row_slot_pos = e.cv.cpos[sidx];
  }
  float eb[UE][COLS], er[UE];
  int omap_row = m_lane;
#pragma unroll
  for (int u = 0; u < UE; ++u) {
    const int unit = u0 + u;
    const bool ok = lane < mr && u < upw && unit < units && KCH > 0;
#pragma unroll
    for (int c = 0; c < COLS; ++c)
      eb[u][c] = (ok && e.bias) ? e.bias[GLU ? unit + c * e.D : unit] : 0.0f;
    er[u] = 0.0f;
    if (ok && e.kind == EPI_RESID) er[u] = a.res_src ? a.res_src[(long)m_lane * D + unit] : ((const float*)e.out)[(long)m_lane * D + unit];
  }
  if (e.kind == EPI_F32 && e.omap && lane < mr) omap_row = e.omap[m_lane / e.ogroup] * e.ostride + m_lane % e.ogroup;
  // (d) residual-base rows for the LayerNorm statistics (rows wave and wave + 4)
  constexpr int RPW = MR > 4 ? 2 : 1;
  float xv[RPW][GEMV_LPL];
  const bool res_stats = a.res_src && a.res_g;
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int r = wave + 4 * t;
    const float* x = a.res_src + (long)(m0 + (r < mr ? r : 0)) * D;
#pragma unroll
    for (int j = 0; j < GEMV_LPL; ++j) xv[t][j] = (res_stats && r < mr && j < D / 64) ? x[lane + 64 * j] : 0.0f;
  }
  // (e) A rows into LDS
  if (a.a_dw) {
    const int items = MR * (K / 4);
    for (int it = tid; it < items; it += 256) {
      const int r = it / (K / 4), ch = (it - r * (K / 4)) * 4;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (r < mr) {
        const int m = m0 + r, sidx = m / e.cv.nf, i = m % e.cv.nf;
        const int id = e.cv.ids[sidx];
        const int p = e.cv.cpos[sidx] + i;
        const TA* ring = (const TA*)a.dw_ring;  // 4 channels of one 32-channel block per read
        float g[16][4];
        float4 w[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int q = p - (a.dw_taps - 1) + t;
          const bool ok = t < a.dw_taps && q >= 0;
          w[t] = t < a.dw_taps ? *(const float4*)(a.dw_w + t * K + ch) : make_float4(0.f, 0.f, 0.f, 0.f);
          if constexpr (sizeof(TA) == 4) {
            const float4 v = ok ? *(const float4*)(ring + cring_idx(id, q % a.dw_Rc, ch, K, a.dw_Rc)) : make_float4(0.f, 0.f, 0.f, 0.f);
            g[t][0] = v.x; g[t][1] = v.y; g[t][2] = v.z; g[t][3] = v.w;
          } else {
            const uint2 v = ok ? *(const uint2*)(ring + cring_idx(id, q % a.dw_Rc, ch, K, a.dw_Rc)) : make_uint2(0u, 0u);
            g[t][0] = __uint_as_float(v.x << 16); g[t][1] = __uint_as_float(v.x & 0xffff0000u);
            g[t][2] = __uint_as_float(v.y << 16); g[t][3] = __uint_as_float(v.y & 0xffff0000u);
          }
        }
        const float4 b4 = *(const float4*)(a.dw_b + ch);
        acc[0] = b4.x; acc[1] = b4.y; acc[2] = b4.z; acc[3] = b4.w;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          acc[0] += w[t].x * g[t][0]; acc[1] += w[t].y * g[t][1]; acc[2] += w[t].z * g[t][2]; acc[3] += w[t].w * g[t][3];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = silu_f(acc[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sA[r * K + ch + q] = acc[q];
    }
  } else if (K % (16 / sizeof(TA)) == 0) {
    constexpr int VA = 16 / sizeof(TA);
    const int cpr = K / VA, chunks = MR * cpr;
    for (int c0 = 0; c0 < chunks; c0 += 256 * 8) {
      uint4 rr[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * 256 + tid, r = c / cpr, kc = c - r * cpr;
        rr[u] = (c < chunks && r < mr) ? *(const uint4*)((const TA*)a.A + a.amap.off(m0 + r) + kc * VA) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * 256 + tid;
        if (c >= chunks) continue;
        float f[VA];
        wunpack<TA>(rr[u], f);
        float* dst = sA + c * VA;  // rows are contiguous: c * VA == r * K + kc * VA
#pragma unroll
        for (int q = 0; q < VA; ++q) dst[q] = f[q];
      }
    }
  } else {
    for (int idx = tid; idx < MR * K; idx += 256) {
      const int r = idx / K, k = idx - r * K;
      sA[idx] = r < mr ? ld<TA>((const TA*)a.A + a.amap.off(m0 + r) + k) : 0.0f;
    }
  }
  __syncthreads();

  // ================= phase 1: row transforms (a wave per row), residual statistics
  constexpr bool round_bf16 = sizeof(TW) == 2;
  for (int r = wave; r < mr; r += 4) {
    float* row = sA + r * K;
    if (a.pre_g) row_ln_regs(row, K, pg, pb, lane);
    if (a.ln_g) row_ln_regs(row, K, lg, lb, lane);
    if (round_bf16 && (sizeof(TA) == 4 || a.a_dw))
      for (int k = lane; k < K; k += 64) row[k] = bf2f(f2bf(row[k]));
  }
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const int r = wave + 4 * t;
    if (!res_stats || r >= mr) continue;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < GEMV_LPL; ++j) s += xv[t][j];
    const float mean = wave_sum(s) / (float)D;
    float q = 0.0f;
#pragma unroll
    for (int j = 0; j < GEMV_LPL; ++j) if (j < D / 64) { const float d = xv[t][j] - mean; q += d * d; }
    const float rstd = rsqrtf(wave_sum(q) / (float)D + 1e-5f);
    if (lane == 0) { stats[2 * r] = mean; stats[2 * r + 1] = rstd; }
  }
  __syncthreads();

  // ================= phase 2: products, reductions, epilogue
  if constexpr (KCH > 0) {
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const int unit = u0 + u;
      if (u < upw && unit < units) {
        float acc[COLS][MR];
#pragma unroll
        for (int c = 0; c < COLS; ++c)
#pragma unroll
          for (int r = 0; r < MR; ++r) acc[c][r] = 0.0f;
#pragma unroll
        for (int c = 0; c < COLS; ++c)
#pragma unroll
          for (int k = 0; k < KCH; ++k) {
            float w[VEC];
            wunpack<TW>(wr[(u * COLS + c) * KCH + k], w);
            const float* ap = sA + (k * 64 + lane) * VEC;
#pragma unroll
            for (int r = 0; r < MR; ++r) {
              float sacc = 0.0f;
#pragma unroll
              for (int v = 0; v < VEC; ++v) sacc += w[v] * ap[r * K + v];
              acc[c][r] += sacc;
            }
          }
#pragma unroll
        for (int c = 0; c < COLS; ++c)
#pragma unroll
          for (int r = 0; r < MR; ++r) acc[c][r] = wave_sum(acc[c][r]);
        float va = 0.0f, vb = 0.0f;
#pragma unroll
        for (int r = 0; r < MR; ++r)
          if (r == lane) { va = acc[0][r]; vb = acc[COLS - 1][r]; }
        if (lane < mr) {
          const int m = m_lane;
          if constexpr (GLU) {
            const float g = (va + eb[u][0]) * sigmoid_f(vb + eb[u][COLS - 1]);
            const int slot = (row_slot_pos + m % e.cv.nf) % e.Rc;
            st<TW>((TW*)e.cring + cring_idx(row_id, slot, unit, e.D, e.Rc), g);
          } else {
            const float v = va + eb[u][0];
            switch (e.kind) {
              case EPI_STORE: st<TW>((TW*)e.out + (long)m * e.ldo + unit, v); break;
              case EPI_SILU: st<TW>((TW*)e.out + (long)m * e.ldo + unit, silu_f(v)); break;
              case EPI_RELU_FE: {
                const bool before_start = row_slot_pos == 0 && m % e.fe_rows_per_stream < e.fe_neg_rows;
                st<TW>((TW*)e.out + (long)m * e.ldo + unit, before_start ? 0.0f : fmaxf(v, 0.0f));
              } break;
              case EPI_RESID: {
                float base = er[u];
                if (res_stats) base = (base - stats[2 * lane]) * stats[2 * lane + 1] * a.res_g[unit] + a.res_b[unit];
                ((float*)e.out)[(long)m * D + unit] = base + e.alpha * v;
              } break;
              case EPI_F32: ((float*)e.out)[(long)omap_row * e.ldo + unit] = v; break;
              case EPI_QKV: {
                const int which = unit / e.D, c = unit % e.D;
                if (which == 0) {
                  e.qbuf[(long)m * e.D + c] = v;
                } else {
                  const int slot = (row_slot_pos + m % e.cv.nf) % e.R;
                  TW* ring = (TW*)(which == 1 ? e.kring : e.vring);
                  st<TW>(ring + (((long)row_id * e.H + c / e.hd) * e.R + slot) * e.hd + c % e.hd, v);
                }
              } break;
              default: break;
            }
          }
        }
      }
    }
  } else {
    // generic K: weights read here, epilogue operands read at the end
    for (int u = 0; u < upw; ++u) {
      const int unit = u0 + u;
      if (unit >= units) break;
      float acc[COLS][MR];
#pragma unroll
      for (int c = 0; c < COLS; ++c)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[c][r] = 0.0f;
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        const int col = GLU ? glu_a_col(unit) + 32 * c : unit;
        const TW* wrow = W + (long)col * K;
        for (int k = lane; k < K; k += 64) {
          const float w = ld<TW>(wrow + k);
#pragma unroll
          for (int r = 0; r < MR; ++r) acc[c][r] += w * sA[r * K + k];
        }
      }
#pragma unroll
      for (int c = 0; c < COLS; ++c)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[c][r] = wave_sum(acc[c][r]);
      float va = 0.0f, vb = 0.0f;
#pragma unroll
      for (int r = 0; r < MR; ++r)
        if (r == lane) { va = acc[0][r]; vb = acc[COLS - 1][r]; }
      if (lane < mr) {
        const int m = m_lane;
        if constexpr (GLU) {
          epi_glu<TW>(e, m, unit, va, vb);
        } else if (e.kind == EPI_RESID && a.res_src) {
          float base = a.res_src[(long)m * D + unit];
          if (a.res_g) base = (base - stats[2 * lane]) * stats[2 * lane + 1] * a.res_g[unit] + a.res_b[unit];
          if (e.bias) va += e.bias[unit];
          ((float*)e.out)[(long)m * D + unit] = base + e.alpha * va;
        } else {
          epi_one<TW>(e, m, unit, va);
        }
      }
    }
  }
}

// =============================================================================== MFMA GEMM (bf16)
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int CPOL_NT = 2;  // cache-policy bits of a vector memory load: non-temporal
// Raw buffer resource over [p, p + bytes) (stride 0; word 3 = 32-bit data format): loads at byte
// offsets at or past `bytes` return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_v;  // 16-byte staging register
typedef __attribute__((ext_vector_type(4))) float f32x4_v;

// Block tile BM x BN, k-step 64, KS groups of 4 waves; in a group the waves form WM x WN, each
// (BM/WM) x (BN/WN) of 32x32 MFMA fragments (v_mfma_f32_32x32x16_bf16, 4 per k-step). Group g
// takes k-steps [g KT/KS, (g+1) KT/KS) through its own ring of S stages in LDS. A stage holds
// the A tile [BM][64] and then the W tile [BN][64], 128 bytes per row, with the 16-byte chunk c
// of row r at chunk position c ^ ((r >> 1) & 7): the 16 rows that one quarter of an operand
// read spans then fall on distinct banks. The stages are filled by direct buffer-to-LDS copies
// (one wave instruction moves 8 rows, 1 KB), so operands never pass through registers: right
// after the barrier of k-step kt the waves issue the copies of k-step kt + S - 1 into the stage
// that k-step kt - 1 used, and S - 1 k-steps of operands are in flight while the MFMAs run. A
// wave waits for its own copies of a stage (vmcnt), then the block barrier publishes them all.
// More groups give a CU more waves when the tile grid alone has about one block per CU; their
// partial tiles are summed in group order in the epilogue, so the result does not depend on
// timing. The epilogue kind is a template parameter; the accumulator tiles go through LDS and
// every thread finishes 8 consecutive columns of a row with 16-byte accesses.

// Epilogue stores are non-temporal: the product's output is read by the next kernel, after the
// kernel boundary has written the L2 back anyway, so streaming it past the L2 saves that
// write-back at the end of the kernel (measured: ~3 us of a 13 us 2048x2048x512 product).
// The exception (EPI_SILU_KEEP) is an output whose consumer runs its rows on the same XCD and
// is bound by reading them: there the write-back pays for itself.
__device__ __forceinline__ void st_bf8(bf16_t* p, const float* y) {
  __builtin_nontemporal_store(u32x4_v{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]), pack_bf2(y[4], y[5]), pack_bf2(y[6], y[7])},
                              (u32x4_v*)p);
}
__device__ __forceinline__ void st_bf8_keep(bf16_t* p, const float* y) {
  *(u32x4_v*)p = u32x4_v{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]), pack_bf2(y[4], y[5]), pack_bf2(y[6], y[7])};
}
__device__ __forceinline__ void ld_f8(const float* p, float* v) {
  const f32x4_v a = ((const f32x4_v*)p)[0], b = ((const f32x4_v*)p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st_f8(float* p, const float* v) {
  __builtin_nontemporal_store(f32x4_v{v[0], v[1], v[2], v[3]}, (f32x4_v*)p);
  __builtin_nontemporal_store(f32x4_v{v[4], v[5], v[6], v[7]}, (f32x4_v*)p + 1);
}

// Epilogue of 8 consecutive output columns col..col+7 of row `row` (v = accumulators). The
// residual kinds take the row's x values and the biases loaded earlier (xp, bp).
template <int EK>
__device__ __forceinline__ void mfma_epi8(const GemmArgs& a, int row, int col, float* v, const float* xp = nullptr,
                                          const float* bp = nullptr, const int* meta = nullptr) {
  // meta (loaded earlier): the row's stream position and id (EPI_QKV), or position (EPI_RELU_FE)
  const EpiArgs& e = a.epi;
  if (bp) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += bp[q];
  } else if (e.bias) {
    float b[8];
    ld_f8(e.bias + col, b);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += b[q];
  }
  if constexpr (EK == EPI_STORE) {
    st_bf8((bf16_t*)e.out + (long)row * e.ldo + col, v);
  } else if constexpr (EK == EPI_SILU || EK == EPI_SILU_KEEP) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = silu_f(v[q]);
    if constexpr (EK == EPI_SILU_KEEP) st_bf8_keep((bf16_t*)e.out + (long)row * e.ldo + col, v);
    else st_bf8((bf16_t*)e.out + (long)row * e.ldo + col, v);
  } else if constexpr (EK == EPI_RELU_FE) {
    const int s = row / e.fe_rows_per_stream, j = row - s * e.fe_rows_per_stream;
    const bool before_start = (meta ? meta[0] : e.cv.cpos[s]) == 0 && j < e.fe_neg_rows;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = before_start ? 0.0f : fmaxf(v[q], 0.0f);
    st_bf8((bf16_t*)e.out + (long)row * e.ldo + col, v);
  } else if constexpr (EK == EPI_RESID || EK == EPI_RESID_KEEP) {
    float* x = (float*)e.out + (long)row * e.ldo + col;
    float r[8];
    if (xp) {
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q] = xp[q];
    } else {
      ld_f8(x, r);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] += e.alpha * v[q];
    if constexpr (EK == EPI_RESID_KEEP) {
      ((f32x4_v*)x)[0] = f32x4_v{r[0], r[1], r[2], r[3]};
      ((f32x4_v*)x)[1] = f32x4_v{r[4], r[5], r[6], r[7]};
    } else {
      st_f8(x, r);
    }
  } else if constexpr (EK == EPI_F32) {
    const long ro = e.omap ? (long)e.omap[row / e.ogroup] * e.ostride + row % e.ogroup : row;
    st_f8((float*)e.out + ro * e.ldo + col, v);
  } else if constexpr (EK == EPI_QKV) {
    const int which = (col >= e.D) + (col >= 2 * e.D), c = col - which * e.D;
    if (which == 0) {
      st_f8(e.qbuf + (long)row * e.D + c, v);
    } else {
      const int s = row / e.cv.nf, i = row - s * e.cv.nf;
      const int slot = ((meta ? meta[0] : e.cv.cpos[s]) + i) % e.R;
      const int id = meta ? meta[1] : e.cv.ids[s];
      const int lg = 31 - __clz(e.hd);  // head sizes are powers of two; 8 columns stay in one head
      bf16_t* ring = (bf16_t*)(which == 1 ? e.kring : e.vring);
      st_bf8(ring + (((long)id * e.H + (c >> lg)) * e.R + slot) * e.hd + (c & (e.hd - 1)), v);
    }
  }
}

// s_waitcnt vmcnt(N): this wave's vector memory operations, direct LDS copies included, down
// to the N most recent
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int KS>
__device__ __forceinline__ void mfma_ct8(const float* ct, int idx, float* v) {
  // 8 accumulator-tile values at idx of every group's tile, summed in group order
  ld_f8(ct + idx, v);
#pragma unroll
  for (int g = 1; g < KS; ++g) {
    float w[8];
    ld_f8(ct + g * BM * (BN + 4) + idx, w);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += w[q];
  }
}

template <int BM, int BN, int S, int KS>
constexpr size_t mfma_lds() {
  // KS rings of S stages, reused afterwards for KS float accumulator tiles and the LayerNorm
  // row and column terms of EPI_LNC
  return std::max((size_t)KS * S * (BM + BN) * 128, (size_t)KS * BM * (BN + 4) * sizeof(float) + (BM + BN) * 8);
}
// EPI_GLU_DW also keeps the tile's GLU outputs and 16 rows of conv taps there: only the tiles
// whose rings cover that take it
template <int BM, int BN, int S, int KS>
constexpr bool mfma_dw_fits() {
  return (size_t)KS * BM * (BN + 4) * sizeof(float) + (BM + BN) * 8 + (size_t)(BM + 16) * (BN / 2) * sizeof(float) <=
         mfma_lds<BM, BN, S, KS>();
}

template <int BM, int BN, int WM, int WN, int S, int KS, int EK>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(KS, 2 * KS))) void gemm_mfma_kernel(GemmArgs a) {
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int SB = (BM + BN) * 128;        // bytes of one stage
  constexpr int NA = BM / 32, NB = BN / 32;  // 1 KB copies of A and of W per wave and stage
  static_assert(WM * WN == 4 && BM % 32 == 0 && BN % 32 == 0 && S >= 2, "tile shape");
  constexpr int EB = EK & 0xff;  // the kind without the EPI_LNC flag
  constexpr bool LNC = (EK & EPI_LNC) != 0, LNS = EB == EPI_RESID_LNS;
  static_assert(!LNS || BN == 64, "tile statistics cover one 64-column tile per block");
  // EPI_GLU_DW: the GLU epilogue, then the depthwise conv + SiLU over the tile's channels of its
  // rows, for the streams whose rows of the call lie in one 64-row block
  constexpr bool DW = EB == EPI_GLU_DW, GLU = EB == EPI_GLU || DW;
  static_assert(!DW || mfma_dw_fits<BM, BN, S, KS>(), "conv taps and GLU rows past the tile's LDS");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds8[];
  // wave and group indices are wave-uniform: in scalar registers, so the copies' LDS bases and
  // k offsets need no per-lane handling
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3), grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wm = wave / WN, wn = wave % WN;
  // XCD-aware tile order: workgroup L runs on XCD L mod 8, each with its own L2. With a.xrg
  // row groups (one k-range, tile grid divisible into 8 = a.xrg x (8 / a.xrg) rectangles) XCD x
  // takes rectangle (x / (8 / a.xrg), x mod (8 / a.xrg)), row-major inside: it fetches only its
  // rows of A and its columns of W. Otherwise every XCD gets a contiguous run of tiles (column
  // tiles fastest, then row tiles, then k-ranges), so the blocks that share A rows, and most of
  // those sharing W rows, meet in one L2 instead of fetching them once per XCD.
  const int gx = gridDim.x, ntiles = gridDim.x * gridDim.y, nall = ntiles * gridDim.z;
  const int L = (blockIdx.z * gridDim.y + blockIdx.y) * gx + blockIdx.x, xcd = L % 8;
  int kz, bm0, bn0;
  if (a.xrg > 0) {
    const int cg = 8 / a.xrg, hr = (int)gridDim.y / a.xrg, wc = gx / cg, j = L / 8;
    const int tr = j / wc, tc = j - tr * wc;
    kz = 0;
    bm0 = ((xcd / cg) * hr + tr) * BM;
    bn0 = ((xcd % cg) * wc + tc) * BN;
  } else {
    const int xq = nall / 8, xr = nall % 8;
    const int f = xcd * xq + min(xcd, xr) + L / 8;
    kz = f / ntiles;
    const int t = f - kz * ntiles;
    bm0 = (t / gx) * BM;
    bn0 = (t - (t / gx) * gx) * BN;
  }
  // split-K over blocks (gridDim.z ranges, EPI_PART): this block's k-range starts at column k0;
  // within it, group grp takes k-steps kb .. kb + KT - 1
  const int M = a.M, N = a.N, K = a.K, Ks = K / (int)gridDim.z, k0 = kz * Ks;
  const int KT = Ks / 64 / KS, kb = grp * KT;
  // byte offsets from A + k0 and W + k0 (the dispatch checks that they fit 31 bits); rows past
  // the matrix read its last row, whose products land in rows or columns the epilogue skips
  const __amdgpu_buffer_rsrc_t ar = raw_rsrc((const bf16_t*)a.A + k0, 0x7fffffff);
  const __amdgpu_buffer_rsrc_t wr = raw_rsrc((const bf16_t*)a.W + k0, 0x7fffffff);
  // copy i of wave w moves stage rows (4 i + w) * 8 .. + 7 of A (i < NA) or W (i < NB); its
  // lane l takes row 8 (4 i + w) + l / 8 and the chunk stored at position l % 8
  const int wv = wave;
  unsigned char* ring = lds8 + grp * S * SB;
  int voa[NA], vob[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int rr = (4 * i + wave) * 8 + (lane >> 3), c = (lane & 7) ^ ((rr >> 1) & 7);
    voa[i] = (int)(a.amap.off(min(bm0 + rr, M - 1)) * 2) + c * 16;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int rr = (4 * i + wave) * 8 + (lane >> 3), c = (lane & 7) ^ ((rr >> 1) & 7);
    vob[i] = min(bn0 + rr, N - 1) * K * 2 + c * 16;
  }
  // (the offsets are copied to locals at the call: the builtin does not take an array element)
#define MFMA_ISSUE(stage, kt)                                                                     \
  {                                                                                               \
    const int so_ = (kt) * 128;                                                                   \
    _Pragma("unroll") for (int i = 0; i < NA; ++i) {                                              \
      const int vo_ = voa[i];                                                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_t*)(ring + (stage) * SB + (4 * i + wv) * 1024), 16, vo_, so_, 0, 0); \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < NB; ++i) {                                              \
      const int vo_ = vob[i];                                                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)(ring + (stage) * SB + BM * 128 + (4 * i + wv) * 1024), 16, vo_, so_, 0, 0); \
    }                                                                                             \
  }
  f32x16_v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // Operands of the epilogue are loaded before the k-loop, so their memory latency hides behind
  // it instead of following it: residual products load the x values (and biases, and with
  // EPI_RESID_LNS the row shifts) their items update; EPI_LNC products load their rows' tile
  // statistics and shifts (thread t < BM: row t) and their columns' c1, c2 (thread t < BN).
  // The other kinds load their items' biases, and the QKV and front-end kinds their rows'
  // stream positions and ids, the same way (GLU: per 8-channel item, both halves' biases).
  constexpr bool RES = EB == EPI_RESID || EB == EPI_RESID_KEEP || LNS;
  constexpr bool PB = !LNC && EB != EPI_PART && !GLU, PM = EB == EPI_QKV || EB == EPI_RELU_FE;
  constexpr int NT = 256 * KS, C8 = BN / 8, NIT8 = (BM * C8 + NT - 1) / NT;
  constexpr int G8 = BN / 16, NITG = (BM * G8 + NT - 1) / NT;  // GLU: 8-channel items
  constexpr int RI = RES ? NIT8 : 1, BI = PB ? NIT8 : 1, MI = PM ? NIT8 : GLU ? NITG : 1;
  constexpr int GI = GLU && !LNC ? NITG : 1, LT = LNC ? 16 : 1;
  float xpre[RI][8], bpre[BI][8], spre[RI], gpre[GI][16];
  int mpre[MI][2];
  if constexpr (RES || PB || PM) {
#pragma unroll
    for (int k = 0; k < NIT8; ++k) {
      const int it = tid + NT * k, rr = it / C8, cc = (it - rr * C8) * 8;
      const int row = min(bm0 + rr, M - 1), col = min(bn0 + cc, N - 8);
      if (it < BM * C8) {
        if constexpr (RES) ld_f8((const float*)a.epi.out + (long)row * a.epi.ldo + col, xpre[k]);
        if constexpr (LNS) spre[k] = a.epi.lns_shift[row];
        if constexpr (PB) {
          if (a.epi.bias) ld_f8(a.epi.bias + col, bpre[k]);
          else
#pragma unroll
            for (int q = 0; q < 8; ++q) bpre[k][q] = 0.0f;
        }
        if constexpr (EB == EPI_QKV) {
          const int st = row / a.epi.cv.nf;
          mpre[k][0] = a.epi.cv.cpos[st];
          mpre[k][1] = a.epi.cv.ids[st];
        } else if constexpr (EB == EPI_RELU_FE) {
          mpre[k][0] = a.epi.cv.cpos[row / a.epi.fe_rows_per_stream];
        }
      }
    }
  }
  if constexpr (GLU) {
#pragma unroll
    for (int k = 0; k < NITG; ++k) {
      const int it = tid + NT * k, rr = it / G8, ch = (it - rr * G8) * 8;
      const int row = min(bm0 + rr, M - 1), c = min(bn0 / 2 + ch, a.epi.D - 8);
      mpre[k][0] = 0;
      mpre[k][1] = 0;
      if (it < BM * G8) {
        const int st = row / a.epi.cv.nf;
        mpre[k][0] = a.epi.cv.cpos[st];
        mpre[k][1] = a.epi.cv.ids[st];
        if constexpr (!LNC) {
          ld_f8(a.epi.bias + c, gpre[k]);
          ld_f8(a.epi.bias + a.epi.D + c, gpre[k] + 8);
        }
      }
    }
  }
  // EPI_GLU_DW: the block's channels of the conv taps (16 rows, zero past the kernel size),
  // staged to LDS after the k-loop, and each item's channels of the conv bias
  constexpr int CH = BN / 2, TPI = DW ? (16 * CH + NT - 1) / NT : 1, DI = DW ? NITG : 1;
  float tpre[TPI], dbpre[DI][8];
  if constexpr (DW) {
    const int D = a.epi.D, ntap = a.dw_taps;
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int e = tid + NT * u, t = e / CH, c = bn0 / 2 + (e - t * CH);
      tpre[u] = (e < 16 * CH && t < ntap && c < D) ? a.dw_w[t * D + c] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < DI; ++k) {
      const int it = tid + NT * k, rr = it / G8, ch = (it - rr * G8) * 8;
      ld_f8(a.dw_b + min(bn0 / 2 + ch, D - 8), dbpre[k]);
    }
  }
  float2 lst[LT];
  float lsh = 0.0f, lc1 = 0.0f, lc2 = 0.0f;
  if constexpr (LNC) {
    const EpiArgs& e = a.epi;
    if (tid < BM) {
      const int row = min(bm0 + tid, M - 1);
#pragma unroll
      for (int t = 0; t < LT; ++t) lst[t] = t < e.lns_ntl ? e.lns[t * e.lns_ld + row] : make_float2(0.0f, 0.0f);
      lsh = e.lns_shift[row];
    }
    if (tid < BN) {
      int idx = min(bn0 + tid, N - 1);
      if constexpr (GLU) {  // packed column -> value channel c, or its gate at D + c
        const int ch = (idx >> 6) * 32 + (idx & 31);
        idx = (idx & 63) >= 32 ? e.D + ch : ch;
      }
      lc1 = e.lnc_c1[idx];
      lc2 = e.lnc_c2[idx];
    }
  }
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) MFMA_ISSUE(s, kb + s);
  // EPI_GLU_DW: each item's conv input rows at positions p0 - 8 .. p0 - 1 of its stream (p0:
  // the call's first position), 8 channels each, issued after the prologue's copies since their
  // addresses wait for the stream ids: NDW loads per wave, every wave issuing all of them
  // (offsets past the resource read zero: rows before the stream start or outside the kernel's
  // reach, and items past the tile), so the k-loop's first S - 1 waits can count them. Read
  // once per call: non-temporal (measured at 1024 streams: 2.20 -> 2.15 ms per step against
  // the default policy, within 10 us of the same loads all hitting one cached stream's rows)
  constexpr int NDW = DW ? 8 * DI : 0;
  u32x4_v dwo[DI][DW ? 8 : 1];
  if constexpr (DW) {
    asm volatile("" ::: "memory");
    const EpiArgs& e = a.epi;
    const __amdgpu_buffer_rsrc_t cr = raw_rsrc(e.cring, 0x7fffffff);
#pragma unroll
    for (int k = 0; k < DI; ++k) {
      const int it = tid + NT * k, rr = it / G8, ch = (it - rr * G8) * 8;
      const int c = min(bn0 / 2 + ch, e.D - 8), p0 = mpre[k][0], lo = max(0, p0 - (a.dw_taps - 1));
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int q = p0 - 8 + r;
        const int off = (it < BM * G8 && q >= lo) ? (int)(cring_idx(mpre[k][1], q % e.Rc, c, e.D, e.Rc) * 2) : INT_MIN;
        dwo[k][r] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(cr, off, 0, CPOL_NT));
      }
    }
  }
  // operand read offsets in a stage (bytes): lane l reads row l % 32 of a fragment, logical
  // chunk 2 kk + l / 32 for the kk-th 16-k MFMA of the k-step
  int aoffs[FM][4], boffs[FN][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * TM + i * 32 + (lane & 31);
      aoffs[i][kk] = r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * TN + j * 32 + (lane & 31);
      boffs[j][kk] = BM * 128 + r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    }
  }
  int buf = 0;
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's copies of k-step kt have landed (later stages may still be in flight) ...
    if (kt + S - 2 < KT) {
      if (DW && kt < S - 1) wait_vmcnt<(S - 2) * (NA + NB) + NDW>();  // the conv rows came after
      else wait_vmcnt<(S - 2) * (NA + NB)>();
    } else {
      wait_vmcnt<0>();
    }
    // ... and every wave's, once all have passed the barrier; every wave has also finished
    // reading the stage of k-step kt - 1, which the copies of k-step kt + S - 1 overwrite
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + S - 1 < KT) {
      int nb = buf + S - 1;
      nb -= nb >= S ? S : 0;
      MFMA_ISSUE(nb, kb + kt + S - 1);
    }
    // the k-step's MFMA block at raised wave priority, so that the SIMD's other wave (the second
    // block on the CU) issues its copies and LDS reads between them rather than in a burst
    // (1024 streams 2.128 -> 2.123 ms, lookahead workload 3.480 -> 3.454 ms per step, one box)
    const unsigned char* st = ring + buf * SB;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_v af[FM], bfv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8_v*)(st + aoffs[i][kk]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfv[j] = *(const bf16x8_v*)(st + boffs[j][kk]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    asm volatile("" ::: "memory");
    buf = buf + 1 == S ? 0 : buf + 1;
  }
#undef MFMA_ISSUE
  __syncthreads();  // every copy has landed and every wave is done reading the stages

  // Each group's accumulator tile goes to its own LDS tile (fragment element r of a lane is row
  // 8*(r/4) + 4*(lane/32) + r%4, column lane%32; all indices compile-time, so acc stays in
  // registers), then each thread takes 8 consecutive columns of a row at a time.
  constexpr int CS = BN + 4;
  // EPI_LNC: per row (rstd, -rstd (mean - shift)) and per column (c1, c2) after the tiles
  float2* lnrow = (float2*)((float*)lds8 + KS * BM * CS);
  float2* lncol = lnrow + BM;
  // EPI_GLU_DW: the tile's GLU outputs [BM][CH] and the conv taps [16][CH] after those
  float* fresh = (float*)(lncol + BN);
  float* taps = fresh + BM * CH;
  if constexpr (DW) {
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int e = tid + NT * u;
      if (e < 16 * CH) taps[e] = tpre[u];
    }
  }
  if constexpr (LNC) {
    if (tid < BM) {  // combine the row's 64-column tiles (Chan et al.'s pairwise update)
      const int ntl = a.epi.lns_ntl;
      float mean = 0.0f;
#pragma unroll
      for (int t = 0; t < LT; ++t) mean += t < ntl ? lst[t].x : 0.0f;
      mean /= (float)ntl;
      float m2 = 0.0f;
#pragma unroll
      for (int t = 0; t < LT; ++t)
        if (t < ntl) {
          const float d = lst[t].x - mean;
          m2 += lst[t].y + 64.0f * d * d;
        }
      const float rstd = rsqrtf(m2 / (float)(64 * ntl) + 1e-5f);
      lnrow[tid] = make_float2(rstd, -rstd * (mean - lsh));
      if (bn0 == 0 && bm0 + tid < M) a.epi.lns_mean[bm0 + tid] = mean;
    }
    if (tid < BN) lncol[tid] = make_float2(lc1, lc2);
  }
  {
    float* ctg = (float*)lds8 + grp * BM * CS;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ctg[(wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * CS + wn * TN + j * 32 + (lane & 31)] = acc[i][j][r];
  }
  __syncthreads();
  const float* ct = (const float*)lds8;
  if constexpr (GLU) {
    // packed columns: each 64-column block holds 32 value columns then their 32 gates; a thread
    // takes 8 channels (8 values, 8 gates) and writes them to the conv ring with one store
    const EpiArgs& e = a.epi;
#pragma unroll
    for (int k = 0; k < NITG; ++k) {
      const int it = tid + NT * k;
      if (it >= BM * G8) break;
      const int rr = it / G8, ch = (it - rr * G8) * 8;
      const int pc = (ch >> 5) * 64 + (ch & 31);
      const int row = bm0 + rr, c = bn0 / 2 + ch;
      if (row >= M || bn0 + pc >= N) continue;
      float va[8], vb[8], ba[8], bb[8];
      mfma_ct8<BM, BN, KS>(ct, rr * CS + pc, va);
      mfma_ct8<BM, BN, KS>(ct, rr * CS + pc + 32, vb);
      if constexpr (LNC) {  // LayerNorm finished; c2 holds the biases
        const float2 lr = lnrow[rr];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float2 ca = lncol[pc + q], cb = lncol[pc + 32 + q];
          va[q] = lr.x * va[q] + lr.y * ca.x;
          vb[q] = lr.x * vb[q] + lr.y * cb.x;
          ba[q] = ca.y;
          bb[q] = cb.y;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ba[q] = gpre[k][q];
          bb[q] = gpre[k][8 + q];
        }
      }
      float g[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = (va[q] + ba[q]) * sigmoid_f(vb[q] + bb[q]);
      const int s = row / e.cv.nf, i = row - s * e.cv.nf;
      const int slot = (mpre[k][0] + i) % e.Rc;
      st_bf8((bf16_t*)e.cring + cring_idx(mpre[k][1], slot, c, e.D, e.Rc), g);
      if constexpr (DW) {
        *(f32x4_v*)(fresh + rr * CH + ch) = f32x4_v{g[0], g[1], g[2], g[3]};
        *(f32x4_v*)(fresh + rr * CH + ch + 4) = f32x4_v{g[4], g[5], g[6], g[7]};
      }
    }
    if constexpr (DW) {
      // row (stream s, frame i) at position p = p0 + i: out = SiLU(b + sum_t w[t] u[p - (K - 1) + t])
      // over the conv inputs u, the older ones from dwo (tap t = r + K - 9 - i for the row at
      // p0 - 8 + r), the call's own from the tile (tap t = j - i + K - 1 for frame j <= i)
      __syncthreads();
      const int ntap = a.dw_taps;
#pragma unroll
      for (int k = 0; k < NITG; ++k) {
        const int it = tid + NT * k;
        if (it >= BM * G8) break;
        const int rr = it / G8, ch = (it - rr * G8) * 8;
        const int pc = (ch >> 5) * 64 + (ch & 31);
        const int row = bm0 + rr, c = bn0 / 2 + ch;
        if (row >= M || bn0 + pc >= N) continue;
        const int i = row - (row / e.cv.nf) * e.cv.nf;
        if (((row - i) >> 6) != ((row - i + e.cv.nf - 1) >> 6)) continue;  // across 64 rows: dw_straddle_kernel
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = dbpre[k][q];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = r + ntap - 9 - i;
          const float* w = taps + max(t, 0) * CH + ch;
          const u32x4_v u = t >= 0 ? dwo[k][r] : u32x4_v{0u, 0u, 0u, 0u};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc[2 * h] += w[2 * h] * __uint_as_float(u[h] << 16);
            acc[2 * h + 1] += w[2 * h + 1] * __uint_as_float(u[h] & 0xffff0000u);
          }
        }
        for (int j = max(0, i - ntap + 1); j <= i; ++j) {
          const float* w = taps + (j - i + ntap - 1) * CH + ch;
          const float* f = fresh + (rr - i + j) * CH + ch;
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += w[q] * f[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = silu_f(acc[q]);
        st_bf8_keep((bf16_t*)e.out + (long)row * e.ldo + c, acc);  // pw2 reads it next (-6 us per step)
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < NIT8; ++k) {
      const int it = tid + NT * k;
      if (it >= BM * C8) break;
      const int rr = it / C8, cc = (it - rr * C8) * 8;
      const int row = bm0 + rr, col = bn0 + cc;
      if (row >= M || col >= N) continue;
      float v[8];
      mfma_ct8<BM, BN, KS>(ct, rr * CS + cc, v);
      if constexpr (LNC) {  // LayerNorm finished (c2 holds the bias; the kind adds none)
        const float2 lr = lnrow[rr];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float2 cl = lncol[cc + q];
          v[q] = lr.x * v[q] + lr.y * cl.x + cl.y;
        }
      }
      if constexpr (EB == EPI_PART) {
        st_f8((float*)a.epi.out + kz * a.epi.pstride + (long)row * a.epi.ldo + col, v);
      } else if constexpr (LNS) {
        // x += alpha (acc + b), streamed (its next reader is the next residual product); this
        // row's 64 columns of the tile sit on 8 neighbouring lanes (items it .. it + 7), which
        // form the tile's (mean, M2) and write the row centred on its shift, kept in the L2 of
        // the XCD whose blocks of the consumer read the same rows
        const EpiArgs& e = a.epi;
        float r[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) r[q] = xpre[k][q] + e.alpha * (v[q] + bpre[k][q]);
        st_f8((float*)e.out + (long)row * e.ldo + col, r);
        float sum = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        const float mt = sum * (1.0f / 64.0f);
        float m2 = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m2 += (r[q] - mt) * (r[q] - mt);
        m2 += __shfl_xor(m2, 1);
        m2 += __shfl_xor(m2, 2);
        m2 += __shfl_xor(m2, 4);
        if ((tid & 7) == 0) e.lns[(col >> 6) * e.lns_ld + row] = make_float2(mt, m2);
        float c8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) c8[q] = r[q] - spre[k];
        st_bf8_keep((bf16_t*)e.xc + (long)row * e.ldo + col, c8);
      } else if constexpr (RES) {
        mfma_epi8<EB>(a, row, col, v, xpre[k], bpre[k]);
      } else if constexpr (PB && PM) {
        mfma_epi8<EB>(a, row, col, v, nullptr, bpre[k], mpre[k]);
      } else if constexpr (PB) {
        mfma_epi8<EB>(a, row, col, v, nullptr, bpre[k]);
      } else if constexpr (PM) {
        mfma_epi8<EB>(a, row, col, v, nullptr, nullptr, mpre[k]);
      } else {
        mfma_epi8<EB>(a, row, col, v);
      }
    }
  }
}


// =============================================================================== LayerNorm
// One wave per row. D a multiple of 256 up to 1024: the row, gains and shifts are loaded
// together as 16-byte chunks, the statistics come from one pass over the row shifted by its
// first element (register-exchange reductions), and the output is written 4 elements at a
// time. Other D: scalar two-pass fallback.
template <typename TO>
__device__ __forceinline__ void st4(TO* p, float a, float b, float c, float d) {
  if constexpr (sizeof(TO) == 4) {
    __builtin_nontemporal_store(f32x4_v{a, b, c, d}, (f32x4_v*)p);
  } else {
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_v;
    __builtin_nontemporal_store(u32x2_v{pack_bf2(a, b), pack_bf2(c, d)}, (u32x2_v*)p);
  }
}

template <typename TO>
__global__ __launch_bounds__(256) void ln_kernel(LnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.M) return;
  const float* x = a.x + (long)row * a.D;
  TO* y = (TO*)a.y + (long)row * a.D;
  if (a.D % 256 == 0 && a.D <= 1024) {
    const int nv = a.D / 256;
    f32x4_v xv[4], gv[4], bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = (min(j, nv - 1) * 64 + lane) * 4;  // clamped: every load unconditional
      xv[j] = *(const f32x4_v*)(x + k);
      gv[j] = *(const f32x4_v*)(a.g + k);
      bv[j] = *(const f32x4_v*)(a.b + k);
    }
    const float c0 = lane_value(xv[0].x, 0);
    float s = 0.0f, q = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nv) {
        const f32x4_v d = xv[j] - c0;
        s += d.x + d.y + d.z + d.w;
        q += d.x * d.x + d.y * d.y + d.z * d.z + d.w * d.w;
      }
    const float inv = 1.0f / (float)a.D;
    s = wave_total(s) * inv;
    q = wave_total(q) * inv;
    const float mean = c0 + s, rstd = rsqrtf(fmaxf(q - s * s, 0.0f) + 1e-5f);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nv) {
        const f32x4_v o = (xv[j] - mean) * rstd * gv[j] + bv[j];
        st4<TO>(y + (j * 64 + lane) * 4, o.x, o.y, o.z, o.w);
      }
    return;
  }
  float s = 0.0f;
  for (int k = lane; k < a.D; k += 64) s += x[k];
  const float mean = wave_total(s) / (float)a.D;
  float q = 0.0f;
  for (int k = lane; k < a.D; k += 64) { float d = x[k] - mean; q += d * d; }
  const float rstd = rsqrtf(wave_total(q) / (float)a.D + 1e-5f);
  for (int k = lane; k < a.D; k += 64) st<TO>(y + k, (x[k] - mean) * rstd * a.g[k] + a.b[k]);
}

// =============================================================================== residual + LayerNorm rows
// One wave per row of D = 256 * NV: chunk j of the row is elements (j * 64 + lane) * 4 .. +3.
// Every operand of the row (x, the NP split-K partials, bias, both LayerNorms' gains and
// shifts) is loaded up front, null operands from a stand-in address and ignored, so the row
// costs one memory round trip. The partials are added in k-range order, so the result does
// not depend on which block of the product finished first.
template <int NV>
__device__ __forceinline__ void row_layernorm(f32x4_v* v, const f32x4_v* g, const f32x4_v* b, float inv_d) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_total(s) * inv_d;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const f32x4_v d = v[j] - mean;
    q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
  }
  const float rstd = rsqrtf(wave_total(q) * inv_d + 1e-5f);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = (v[j] - mean) * rstd * g[j] + b[j];
}

// KEEP: block L takes rows of the XCD-contiguous eighth L mod 8 (the dense products give each
// XCD such an eighth of their rows), and y goes out by write-back stores, so the x rows the
// residual product just wrote and the y rows the next product reads stay in one XCD's L2.
template <typename TO, int NP, int NV, bool KEEP>
__global__ __launch_bounds__(256) void resid_ln_kernel(ResLnArgs a) {
  const int blk = KEEP ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int row = blk * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.M) return;
  const long ro = (long)row * a.D;
  float* x = a.x + ro;
  const float* any = a.x;  // stand-in for null operands
  const float* bias = a.bias ? a.bias : any;
  const float* go = a.go ? a.go : any;
  const float* bo = a.bo ? a.bo : any;
  const float* gn = a.gn ? a.gn : any;
  const float* bn = a.bn ? a.bn : any;
  f32x4_v xv[NV], bv[NV], gov[NV], bov[NV], gnv[NV], bnv[NV];
  f32x4_v pv[NP > 0 ? NP : 1][NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k = (j * 64 + lane) * 4;
    xv[j] = *(const f32x4_v*)(x + k);
#pragma unroll
    for (int z = 0; z < NP; ++z) pv[z][j] = *(const f32x4_v*)(a.part + z * a.pstride + ro + k);
    bv[j] = *(const f32x4_v*)(bias + k);
    gov[j] = *(const f32x4_v*)(go + k);
    bov[j] = *(const f32x4_v*)(bo + k);
    gnv[j] = *(const f32x4_v*)(gn + k);
    bnv[j] = *(const f32x4_v*)(bn + k);
  }
  const float inv_d = 1.0f / (float)a.D;
  if constexpr (NP > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      f32x4_v v = pv[0][j];
#pragma unroll
      for (int z = 1; z < NP; ++z) v += pv[z][j];
      if (a.bias) v += bv[j];
      xv[j] += a.alpha * v;
    }
  }
  if (a.go) row_layernorm<NV>(xv, gov, bov, inv_d);
  if (NP > 0 || a.go) {
#pragma unroll
    for (int j = 0; j < NV; ++j) *(f32x4_v*)(x + (j * 64 + lane) * 4) = xv[j];
  }
  if (a.mean) {  // the row's mean: the shift the next residual product centres around
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) sum += (xv[j].x + xv[j].y) + (xv[j].z + xv[j].w);
    sum = wave_total(sum);
    if (lane == 0) a.mean[row] = sum * inv_d;
  }
  if (a.y) {
    if (a.gn) row_layernorm<NV>(xv, gnv, bnv, inv_d);
    TO* y = (TO*)a.y + ro;
    if constexpr (KEEP && sizeof(TO) == 2) {
      typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_v;
#pragma unroll
      for (int j = 0; j < NV; ++j)
        *(u32x2_v*)(y + (j * 64 + lane) * 4) = u32x2_v{pack_bf2(xv[j].x, xv[j].y), pack_bf2(xv[j].z, xv[j].w)};
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) st4<TO>(y + (j * 64 + lane) * 4, xv[j].x, xv[j].y, xv[j].z, xv[j].w);
    }
  }
}

template <typename TO, int NP, bool KEEP>
static const void* resid_ln_pick_nv(int nv) {
  switch (nv) {
    case 1: return (const void*)&resid_ln_kernel<TO, NP, 1, KEEP>;
    case 2: return (const void*)&resid_ln_kernel<TO, NP, 2, KEEP>;
    case 3: return (const void*)&resid_ln_kernel<TO, NP, 3, KEEP>;
    case 4: return (const void*)&resid_ln_kernel<TO, NP, 4, KEEP>;
    default: return nullptr;
  }
}
template <typename TO, bool KEEP>
static const void* resid_ln_pick(int np, int nv) {
  switch (np) {
    case 0: return resid_ln_pick_nv<TO, 0, KEEP>(nv);
    case 2: return resid_ln_pick_nv<TO, 2, KEEP>(nv);
    case 4: return resid_ln_pick_nv<TO, 4, KEEP>(nv);
    default: return nullptr;
  }
}

bool launch_resid_ln(Launcher& L, const ResLnArgs& a, int dtype) {
  if (a.D % 256 || a.D > 1024 || a.M < 1) return false;
  // the XCD eighths need a whole number of blocks per XCD
  const bool keep = a.keep && ((a.M + 3) / 4) % 8 == 0;
  const void* fn = dtype == DT_F32 ? (keep ? resid_ln_pick<float, true>(a.nparts, a.D / 256) : resid_ln_pick<float, false>(a.nparts, a.D / 256))
                                   : (keep ? resid_ln_pick<bf16_t, true>(a.nparts, a.D / 256) : resid_ln_pick<bf16_t, false>(a.nparts, a.D / 256));
  if (!fn) return false;
  ResLnArgs args = a;
  // algorithmic bytes: none (activations and partials stay in the last-level cache)
  L.tag("resid_ln", 0.0, 0.0);
  L.launch(fn, dim3((a.M + 3) / 4), dim3(256), 0, &args);
  return true;
}

// =============================================================================== dense dispatch
// Algorithmic HBM bytes of one dense product: the weights once, plus the depthwise ring rows
// it reads and what its epilogue writes to per-stream state (K/V rows, depthwise input rows)
// or to the caller's output. Activations that stay on chip or in cache are not counted.
double gemm_bytes(const GemmArgs& a, int wsz) {
  // int8 weights (wsz 1): the codes, one float32 scale per row, float32 caches
  double b = (double)a.N * a.K * wsz + (wsz == 1 ? 4.0 * a.N : 0.0);
  const double esz = wsz == 1 ? 4.0 : (double)wsz;
  if (a.a_dw) b += (double)a.epi.cv.n_streams * (a.dw_taps - 1 + a.epi.cv.nf) * a.K * esz;
  switch (a.epi.kind & 0xff) {
    case EPI_QKV: b += (double)a.M * 2.0 * a.epi.D * esz; break;
    case EPI_GLU: b += (double)a.M * (a.N / 2) * esz; break;
    case EPI_GLU_DW:  // ring rows written and the older ring rows the conv reads
      b += (double)a.M * (a.N / 2) * esz + (double)a.epi.cv.n_streams * (a.dw_taps - 1) * (a.N / 2) * esz;
      break;
    case EPI_F32: if (a.epi.ldo != a.epi.D || a.epi.omap) b += (double)a.M * a.N * 4.0; break;
    default: break;
  }
  return b;
}

template <typename TW, typename TA, int MR, int KCH>
static const void* gemv_pick_glu(bool glu) {
  return glu ? (const void*)&gemv_kernel<TW, TA, MR, KCH, true> : (const void*)&gemv_kernel<TW, TA, MR, KCH, false>;
}
template <typename TW, typename TA, int MR>
static const void* gemv_pick_kch(int kch, bool glu) {
  constexpr bool f32w = sizeof(TW) == 4;
  switch (kch) {
    case 1: return gemv_pick_glu<TW, TA, MR, 1>(glu);
    case 2: return f32w ? gemv_pick_glu<TW, TA, MR, 2>(glu) : nullptr;
    case 3: return f32w ? nullptr : gemv_pick_glu<TW, TA, MR, 3>(glu);
    case 4: return f32w ? nullptr : gemv_pick_glu<TW, TA, MR, 4>(glu);
    case 6: return f32w ? gemv_pick_glu<TW, TA, MR, 6>(glu) : nullptr;
    case 8: return f32w ? gemv_pick_glu<TW, TA, MR, 8>(glu) : nullptr;
    default: return gemv_pick_glu<TW, TA, MR, 0>(glu);
  }
}
static int gemv_umax(int kch, bool glu) {
  const int cols = glu ? 2 : 1;
  return kch > 0 ? std::max(1, 8 / (cols * kch)) : 1 << 30;
}

template <typename TW, typename TA>
static void gemv_dispatch(Launcher& L, const GemmArgs& a) {
  const bool glu = a.epi.kind == EPI_GLU;
  const int units = glu ? a.N / 2 : a.N;
  constexpr int VEC = 16 / sizeof(TW);
  int kch = a.K % (64 * VEC) == 0 ? a.K / (64 * VEC) : 0;
  if (kch && !gemv_pick_kch<TW, TA, 2>(kch, glu)) kch = 0;
  if (kch != 1 && kch != 2 && kch != 3 && kch != 4 && kch != 6 && kch != 8) kch = 0;
  // units per wave: enough waves for the chip, within the register budget
  int upw = std::max(1, (units + 4 * 256 - 1) / (4 * 256));
  upw = std::min(upw, gemv_umax(kch, glu));
  GemmArgs args = a;
  args.upb = upw;
  const int MR = a.M <= 2 ? 2 : 8;
  const void* fn = MR == 2 ? gemv_pick_kch<TW, TA, 2>(kch, glu) : gemv_pick_kch<TW, TA, 8>(kch, glu);
  const size_t shm = ((size_t)MR * a.K + 2 * MR) * sizeof(float);
  L.tag(sizeof(TW) == 4 ? "gemm_small_m_f32" : "gemm_small_m_bf16", gemm_bytes(a, (int)sizeof(TW)), 2.0 * a.M * a.N * a.K);
  L.launch(fn, dim3((units + 4 * upw - 1) / (4 * upw), (a.M + MR - 1) / MR), dim3(256), shm, &args);
}

template <int BM, int BN, int WM, int WN, int S, int KS>
static const void* mfma_pick_epi(int ek) {
  switch (ek) {
    case EPI_STORE: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_STORE>;
    case EPI_SILU: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_SILU>;
    case EPI_SILU_KEEP: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_SILU_KEEP>;
    case EPI_RELU_FE: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_RELU_FE>;
    case EPI_RESID: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_RESID>;
    case EPI_RESID_KEEP: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_RESID_KEEP>;
    case EPI_F32: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_F32>;
    case EPI_QKV: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_QKV>;
    case EPI_GLU: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_GLU>;
    case EPI_PART: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_PART>;
    case EPI_SILU | EPI_LNC: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_SILU | EPI_LNC>;
    case EPI_SILU_KEEP | EPI_LNC: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_SILU_KEEP | EPI_LNC>;
    case EPI_QKV | EPI_LNC: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_QKV | EPI_LNC>;
    case EPI_GLU | EPI_LNC: return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_GLU | EPI_LNC>;
    case EPI_GLU_DW:
      if constexpr (BN % 64 == 0 && mfma_dw_fits<BM, BN, S, KS>()) return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_GLU_DW>;
      return nullptr;
    case EPI_GLU_DW | EPI_LNC:
      if constexpr (BN % 64 == 0 && mfma_dw_fits<BM, BN, S, KS>())
        return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_GLU_DW | EPI_LNC>;
      return nullptr;
    case EPI_RESID_LNS:
      if constexpr (BN == 64) return (const void*)&gemm_mfma_kernel<BM, BN, WM, WN, S, KS, EPI_RESID_LNS>;
      return nullptr;
    default: return nullptr;
  }
}

// The block tiles: shape, waves, stages and k-groups (stage counts measured at 2048 rows, K 512
// and 2048, with operands that come from HBM rather than the caches)
struct MfmaTile {
  int bm, bn, groups;
  const void* (*pick)(int);
  size_t lds;
};
static const MfmaTile kMfmaTiles[9] = {
    {0, 0, 0, nullptr, 0},
    {128, 128, 1, &mfma_pick_epi<128, 128, 2, 2, 2, 1>, mfma_lds<128, 128, 2, 1>()},
    {128, 64, 1, &mfma_pick_epi<128, 64, 4, 1, 3, 1>, mfma_lds<128, 64, 3, 1>()},
    {64, 128, 1, &mfma_pick_epi<64, 128, 2, 2, 3, 1>, mfma_lds<64, 128, 3, 1>()},
    {64, 64, 1, &mfma_pick_epi<64, 64, 2, 2, 3, 1>, mfma_lds<64, 64, 3, 1>()},
    {64, 64, 2, &mfma_pick_epi<64, 64, 2, 2, 3, 2>, mfma_lds<64, 64, 3, 2>()},
    {64, 64, 4, &mfma_pick_epi<64, 64, 2, 2, 2, 4>, mfma_lds<64, 64, 2, 4>()},
    {128, 128, 2, &mfma_pick_epi<128, 128, 2, 2, 2, 2>, mfma_lds<128, 128, 2, 2>()},
    {128, 96, 2, &mfma_pick_epi<128, 96, 4, 1, 2, 2>, mfma_lds<128, 96, 2, 2>()},
};

// tile: 0 = chosen here; 1 = 128x128, 2 = 128x64, 3 = 64x128, 4 = 64x64, 5 / 6 = 64x64 with its
// k-steps split over 2 / 4 groups of waves, 7 / 8 = 128x128 / 128x96 over 2 groups (test
// entry point)
static void mfma_dispatch(Launcher& L, const GemmArgs& a, int tile) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  GemmArgs args = a;
  // the product with the depthwise conv in its epilogue is a family of its own
  const bool dw = (a.epi.kind & 0xff) == EPI_GLU_DW;
  if (dw) L.tag("gemm_mfma_bf16_dwconv", gemm_bytes(a, 2), 2.0 * a.M * a.N * a.K + 2.0 * a.dw_taps * (a.N / 2) * a.M);
  else L.tag("gemm_mfma_bf16", gemm_bytes(a, 2), 2.0 * a.M * a.N * a.K);
  const int ks = std::max(a.ksplit, 1);
  auto fail = [&]() {
    if (L.err == hipSuccess) L.err = hipErrorInvalidValue;
  };
  if (ks > 1 && (a.epi.kind != EPI_PART || a.K % (64 * ks))) return fail();  // split-K writes partials only
  // byte offsets of the operand copies are 32-bit: the A rows the row map reaches and all of W
  const long amax = (long)((a.M - 1) / std::max(a.amap.group, 1)) * a.amap.group_stride +
                    (long)(std::min(a.amap.group, a.M) - 1) * a.amap.row_stride + a.K;
  if (a.M < 1 || a.N < 8 || a.N % 8 || a.K < 64 || amax * 2 >= (1L << 31) || (long)a.N * a.K * 2 >= (1L << 31)) return fail();
  const bool lns = a.epi.kind == EPI_RESID_LNS, lnc = (a.epi.kind & EPI_LNC) != 0;
  if ((lns || lnc) && (ks > 1 || !a.epi.lns || !a.epi.lns_shift || a.epi.lns_ntl < 1 || a.epi.lns_ntl > 16)) return fail();
  if (lns && (a.N % 64 || a.N / 64 != a.epi.lns_ntl || !a.epi.xc)) return fail();
  if (lnc && (!a.epi.lnc_c1 || !a.epi.lnc_c2 || !a.epi.lns_mean || a.K != 64 * a.epi.lns_ntl)) return fail();
  // EPI_GLU_DW: the conv reads 8 older ring rows (kernel size at most 9); the epilogue convolves
  // the streams whose rows of the call lie in one 64-row block (at most 64 frames per call: the
  // others cross one boundary each and are left to dw_straddle_kernel), and the ring offsets are
  // 32-bit (the caller checks the layer's ring size)
  if (dw && (a.dw_taps < 1 || a.dw_taps > 9 || !a.dw_w || !a.dw_b || !a.epi.out || !a.epi.cring || a.epi.D % 32 ||
             a.epi.cv.nf < 1 || a.epi.cv.nf > 64))
    return fail();
  const int kt = a.K / 64 / ks;  // k-steps per block
  if (tile == 0) {
    // measured at 512 - 5120 rows (K 512 / 2048, N 512 - 2048): a larger tile pays from about
    // 1.25 workgroups per CU (320 tiles), two stages of 128x128 then leaving room for two
    // blocks per CU; below that 64x64 (always with split-K, whose k-ranges add the blocks),
    // whose k-steps go to 2 groups of waves when there is about one tile per CU or fewer
    // (2048 rows, operands from HBM, residual epilogue: 2048x512x512 8.7 -> 6.6 us,
    // 2048x512x2048 16.7 -> 13.0 us against the register-staged kernel)
    // A column count that 128x64 tiles cover in 1.5 rounds of the CUs and 128x96 tiles in one
    // takes the latter over two groups of waves (2048x1536x512, qkv at 2048 rows: 11.6 -> 10.7 us
    // in the step). 128x128 over two groups (tile 7) measured no better than 128x64 for
    // 2048x2048x512 in the step, though 9.1 -> 8.6 us in a lab loop.
    if (ks == 1 && tiles(128, 128) >= 320) tile = 1;
    else if (ks == 1 && (a.epi.kind & 0xff) != EPI_GLU && !dw && a.N % 96 == 0 && tiles(128, 96) >= 192 && tiles(128, 96) <= 256 &&
             kt % 2 == 0)
      tile = 8;
    else if (ks == 1 && tiles(128, 64) >= 320) tile = 2;
    else if (ks == 1 && tiles(64, 64) <= 256 && kt % 2 == 0) tile = 5;
    else tile = 4;
  }
  if (tile < 1 || tile > 8) return fail();
  if (lns && kMfmaTiles[tile].bn != 64) tile = tiles(128, 64) >= 320 ? 2 : 4;  // one 64-column tile per block
  if (dw && tile == 1) tile = 2;  // 128x128 has no LDS room for the conv's rows
  if (((a.epi.kind & 0xff) == EPI_GLU || dw) && kMfmaTiles[tile].bn % 64) return fail();  // whole value/gate blocks
  const MfmaTile& T = kMfmaTiles[tile];
  if (kt % T.groups) return fail();  // every group takes the same number of k-steps
  const void* fn = T.pick(a.epi.kind);
  if (!fn) return fail();
  dim3 grid((a.N + T.bn - 1) / T.bn, (a.M + T.bm - 1) / T.bm, ks);
  // XCD rectangles (one k-range, tile grid divisible): the row-group count whose rectangles
  // fetch the fewest A rows and W columns into the 8 L2s, taken when that is at most 60% of what
  // the contiguous runs fetch (each XCD: its rows of A, all of W). Measured: products whose
  // weights outweigh their 512 A rows gain (256 streams: 1.594 -> 1.542 ms per step); at 2048
  // rows, savings of 20-33% made the 1024-stream step 0.5% slower. 0 keeps the contiguous runs.
  args.xrg = 0;
  if (ks == 1) {
    const long runs = (long)grid.y * T.bm + 8L * grid.x * T.bn;
    long best = runs;
    for (int rg = 1; rg <= 8; rg *= 2) {
      const int cg = 8 / rg;
      if (grid.y % rg || grid.x % cg) continue;
      const long cost = 8L * ((long)(grid.y / rg) * T.bm + (long)(grid.x / cg) * T.bn);
      if (cost < best && 10 * cost <= 6 * runs) { best = cost; args.xrg = rg; }
    }
  }
  L.launch(fn, grid, dim3(256 * T.groups), T.lds, &args);
}

__global__ __launch_bounds__(256) void cvt_kernel(CvtArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.M * a.K) return;
  const int m = (int)(idx / a.K), k = (int)(idx % a.K);
  ((bf16_t*)a.y)[idx] = f2bf(a.x[a.amap.off(m) + k]);
}

void launch_gemm(Launcher& L, const GemmArgs& a0, int dtype, int path) {
  GemmArgs a = a0;
  // only the MFMA kernel keeps its SiLU / residual rows in L2; the others store as usual
  const bool mfma = dtype != DT_F32 && path != 1 && !(path == 0 && (a.M <= 8 || a.N % 8 != 0)) && a.K % 64 == 0;
  if (a.epi.kind == EPI_SILU_KEEP && !mfma) a.epi.kind = EPI_SILU;
  if (a.epi.kind == EPI_RESID_KEEP && !mfma) a.epi.kind = EPI_RESID;
  if ((a.epi.kind == EPI_RESID_LNS || (a.epi.kind & EPI_LNC)) && !mfma) {  // the MFMA kernel's kinds only
    if (L.err == hipSuccess) L.err = hipErrorInvalidValue;
    return;
  }
  if (path == 0 && rowdot_launch(L, a, dtype)) return;
  // int8 weights: the two-row kernel only; the depthwise conv in the GLU epilogue: the two-row
  // and MFMA kernels
  if (dtype == DT_I8W || ((a.epi.kind & 0xff) == EPI_GLU_DW && !mfma)) {
    if (L.err == hipSuccess) L.err = hipErrorInvalidValue;
    return;
  }
  if (dtype == DT_F32) {
    gemv_dispatch<float, float>(L, a);
    return;
  }
  const bool small = path == 1 || (path == 0 && (a.M <= 8 || a.N % 8 != 0)) || a.K % 64 != 0;
  if (small) {
    if (a.a_f32 && !a.a_dw) gemv_dispatch<bf16_t, float>(L, a);
    else gemv_dispatch<bf16_t, bf16_t>(L, a);
    return;
  }
  GemmArgs g = a;
  if (a.a_f32) {
    // materialise the bf16 operand first: LayerNorm rows, or a rounded (gathered) copy
    const char* role = L.role;
    L.role = nullptr;
    if (a.ln_g) {
      LnArgs la{(const float*)a.A, a.a_scratch, a.ln_g, a.ln_b, a.M, a.K, 0};
      L.tag("layernorm", 0.0, 0.0);
      L.launch((const void*)&ln_kernel<bf16_t>, dim3((a.M + 3) / 4), dim3(256), 0, &la);
    } else {
      CvtArgs cv{(const float*)a.A, a.amap, a.a_scratch, a.M, a.K};
      const long total = (long)a.M * a.K;
      L.tag("convert_rows", 0.0, 0.0);
      L.launch((const void*)&cvt_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &cv);
    }
    L.role = role;
    g.A = a.a_scratch;
    g.amap = RowMap{INT_MAX, 0, a.K};
    g.a_f32 = 0;
    g.ln_g = g.ln_b = nullptr;
  }
  // paths 3..6: tiles 1..4; 9..12: tiles 5..8 (64x64 over 2 / 4 groups of waves, 128x128 and
  // 128x96 over 2)
  mfma_dispatch(L, g, path >= 9 ? path - 4 : path >= 3 ? path - 2 : 0);
}

void launch_cvt(Launcher& L, const CvtArgs& a) {
  CvtArgs args = a;
  const long total = (long)a.M * a.K;
  L.tag("convert_rows", 0.0, 0.0);
  L.launch((const void*)&cvt_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

void launch_ln(Launcher& L, const LnArgs& a, int dtype) {
  LnArgs args = a;
  const void* fn = (a.out_f32 || dtype == DT_F32) ? (const void*)&ln_kernel<float> : (const void*)&ln_kernel<bf16_t>;
  L.tag("layernorm", 0.0, 0.0);
  L.launch(fn, dim3((a.M + 3) / 4), dim3(256), 0, &args);
}

// =============================================================================== attention
// One block of 4 waves per (call stream, head). Every global read is issued before the block's
// single barrier: all R slots of the head's K and V rings (their addresses depend on the stream
// id only, not on its position), the head's projected-position rows, the call's q rows and u, v.
// K and V stay in their storage type in LDS. Then a wave per query row i, lanes over ring slots
// j (slot j holds position q_j, the one position of the ring window congruent to j mod R):
//   s[i][j] = ((q_i + u) . k_j + (q_i + v) . P[p_i - q_j]) * scale on visible keys, else -inf;
// max and sum of the row by register exchanges, and o_i = sum_j softmax(s)_ij v_j with lanes
// over head dims taking each p_ij from the lane that holds it.
// 16-byte chunks per thread per staging pass: K/V rings (a 72-80 slot ring is 576-640 chunks in
// bf16, 1152-1280 in float32) and position rows (73-74 rows of 16 chunks). Larger rings take
// more passes. Slots past an array's end reload its last chunk: skipping them by a branch
// serialises the loads (measured 5x slower).
template <typename T> constexpr int att_um_kv() { return sizeof(T) == 2 ? 3 : 5; }
constexpr int ATT_UM_P = 5;

size_t attention_shmem(int nf, int R, int nrel, int hd, int esz) {
  const size_t kv_row = ((size_t)hd * esz / 16 + 1) * 16;  // rows padded by one chunk
  const size_t f_row = ((size_t)hd / 4 + 1) * 16;
  return 2 * (size_t)R * kv_row + (size_t)nrel * f_row + ((size_t)nf + 2) * hd * 4 + 4 * 256 * 4;
}

__device__ __forceinline__ bool att_visible(const AttnArgs& a, int p, int q) {
  if (q < 0) return false;
  if (a.lookahead) return q >= p - a.Lc && q <= p + a.right;
  const int cs = p - p % a.chunk;
  return q >= cs - a.Lc && q <= cs + a.chunk - 1;
}


// four consecutive elements (index 4c..4c+3) of an LDS row of T as float
template <typename T>
__device__ __forceinline__ f32x4_v lds4(const unsigned char* row, int c) {
  if constexpr (sizeof(T) == 4) {
    return ((const f32x4_v*)row)[c];
  } else {
    const uint2 u = ((const uint2*)row)[c];
    return f32x4_v{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
  }
}

template <typename T, int HD, int JT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smb[];
  constexpr int KC = HD * (int)sizeof(T) / 16;  // 16-byte chunks per K/V row
  constexpr int KS = (KC + 1) * 16;             // LDS bytes per K/V row
  constexpr int FC = HD / 4;                    // chunks per float row
  constexpr int FS = (FC + 1) * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nf = a.cv.nf, R = a.R, nrel = a.nrel;
  const int s = blockIdx.x / a.H, h = blockIdx.x - s * a.H;
  const int id = a.cv.ids[s];
  const int pos0 = a.cv.cpos[s];
  unsigned char* Ks = smb;
  unsigned char* Vs = Ks + R * KS;
  unsigned char* Ps = Vs + R * KS;
  float* Qs = (float*)(Ps + nrel * FS);  // [nf][HD], then u [HD], v [HD]
  float* Pw = Qs + (nf + 2) * HD + wave * 256;  // this wave's softmax weights, by ring slot
  const u32x4_v* kg = (const u32x4_v*)((const T*)a.kring + ((long)id * a.H + h) * R * HD);
  const u32x4_v* vg = (const u32x4_v*)((const T*)a.vring + ((long)id * a.H + h) * R * HD);
  const u32x4_v* pg = (const u32x4_v*)(a.posproj + (long)h * nrel * HD);
  const int nkv = R * KC, np = nrel * FC, nq = (nf + 2) * FC;

  // ---- staging: K, V, P in passes of UKV / UP chunks per thread (one pass at the usual sizes),
  // indices clamped so that every load is unconditional; q, u, v with the first pass
  constexpr int UKV = att_um_kv<T>(), UP = ATT_UM_P;
  for (int pass = 0; pass * 256 * UKV < nkv || pass * 256 * UP < np; ++pass) {
    const int bkv = pass * 256 * UKV, bp = pass * 256 * UP;
    u32x4_v rk[UKV], rv[UKV], rp[UP], rq[2];
    // position rows and q/u/v first: they do not wait for the stream id, K and V do
#pragma unroll
    for (int u = 0; u < UP; ++u) rp[u] = pg[min(bp + u * 256 + tid, np - 1)];
    if (pass == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = min(u * 256 + tid, nq - 1), row = c / FC, col = c - row * FC;
        const float* src = row < nf ? a.q + (long)(s * nf + row) * a.D + h * HD : (row == nf ? a.pos_u : a.pos_v) + h * HD;
        rq[u] = *((const u32x4_v*)src + col);
      }
    }
    // the rings are read once per call: non-temporal loads (streaming them past the caches
    // measured 2.2x the bandwidth of default-policy reads of the same rows in isolation)
#pragma unroll
    for (int u = 0; u < UKV; ++u) {
      const int ck = min(bkv + u * 256 + tid, nkv - 1);
      rk[u] = __builtin_nontemporal_load(kg + ck);
      rv[u] = __builtin_nontemporal_load(vg + ck);
    }
    // stored in arrival order
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int c = bp + u * 256 + tid;
      if (c < np) {
        const int row = c / FC, col = c - row * FC;
        *(u32x4_v*)(Ps + row * FS + col * 16) = rp[u];
      }
    }
    if (pass == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = u * 256 + tid;
        if (c < nq) ((u32x4_v*)Qs)[c] = rq[u];
      }
    }
#pragma unroll
    for (int u = 0; u < UKV; ++u) {
      const int c = bkv + u * 256 + tid;
      if (c < nkv) {
        const int row = c / KC, col = c - row * KC;
        *(u32x4_v*)(Ks + row * KS + col * 16) = rk[u];
        *(u32x4_v*)(Vs + row * KS + col * 16) = rv[u];
      }
    }
  }
  __syncthreads();

  // ---- ring slots of this lane: slot j holds position pe - ((pe - j) mod R)
  const int pe = pos0 + nf - 1, pm = pe % R, q_lo = max(0, pos0 - a.Lc);
  int qj[JT];
#pragma unroll
  for (int t = 0; t < JT; ++t) {
    const int j = lane + 64 * t;
    int dd = pm - j;
    dd += dd < 0 ? R : 0;
    qj[t] = (j < R && pe - dd >= q_lo) ? pe - dd : -1;  // -1: no key in this slot
  }
  const float* Us = Qs + nf * HD;
  const float* Ws = Us + HD;
  constexpr int NCH = HD / 4, NPH = 64 / NCH;  // PV lanes as (4-dim chunk, key phase)
  const int c4 = lane % NCH, ph = lane / NCH;

  if (JT == 2 && nf <= 2) {
    // ---- two query rows or fewer: all 4 waves busy as (query row i, half kh of the ring
    // slots); each half keeps its own max, sum and unnormalised PV, combined after a barrier
    const int i = wave & 1, kh = wave >> 1;
    const int ii = i < nf ? i : 0;  // a wave without a row computes row 0 and stores nothing
    const int p = pos0 + ii, j = lane + 64 * kh, q = qj[kh];
    const bool vis = q >= 0 && att_visible(a, p, q);
    const int rel = vis ? p - q - a.rel_lo : 0;
    const unsigned char* krow = Ks + min(j, R - 1) * KS;
    const unsigned char* prow = Ps + rel * FS;
    const f32x4_v* qi = (const f32x4_v*)(Qs + ii * HD);
    // (q + u) and (q + v) of this wave's row in registers: the loop then reads only the lane's
    // own K and position rows from LDS
    f32x4_v qu[FC], qv[FC];
#pragma unroll
    for (int c = 0; c < FC; ++c) {
      const f32x4_v q4 = qi[c];
      qu[c] = q4 + ((const f32x4_v*)Us)[c];
      qv[c] = q4 + ((const f32x4_v*)Ws)[c];
    }
    float ac = 0.0f, bd = 0.0f;
#pragma unroll
    for (int c = 0; c < FC; ++c) {
      const f32x4_v k4 = lds4<T>(krow, c), p4 = ((const f32x4_v*)prow)[c];
      ac += qu[c].x * k4.x + qu[c].y * k4.y + qu[c].z * k4.z + qu[c].w * k4.w;
      bd += qv[c].x * p4.x + qv[c].y * p4.y + qv[c].z * p4.z + qv[c].w * p4.w;
    }
    const float sc = vis ? (ac + bd) * a.scale : -INFINITY;
    const float mw = wave_top(sc);  // -inf when this half holds no visible key
    const float ew = vis ? __expf(sc - mw) : 0.0f;
    const float lw = wave_total(ew);
    f32x4_v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (64 * kh < R) {
      // weights to the strip; slots of this half holding no key get a zero V row first
      Pw[lane] = ew;
      if (j < R && q < 0) {
#pragma unroll
        for (int c = 0; c < KC; ++c) *(u32x4_v*)(Vs + j * KS + c * 16) = u32x4_v{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int m = 0; m < 64 / NPH; ++m) {
        const int jj = ph + NPH * m;  // rows past R - 1 clamp to R - 1, inside this half
        acc += Pw[jj] * lds4<T>(Vs + min(64 * kh + jj, R - 1) * KS, c4);
      }
#pragma unroll
      for (int b = NCH; b < 64; b <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[e];
          if (b == 32) v = pair_sum32(v, v);
          else if (b == 16) v = pair_sum16(v, v);
          else v += __shfl_xor(v, b, 64);
          acc[e] = v;
        }
      }
    }
    float* cmb = Pw + 64;  // [max, sum, o[HD]] of this wave's half
    if (lane < NCH) *(f32x4_v*)(cmb + 4 + 4 * lane) = acc;
    if (lane == 0) { cmb[0] = mw; cmb[1] = lw; }
    __syncthreads();
    if (kh == 0 && i < nf) {
      const float* c1 = cmb + 2 * 256;  // the same row's other half (wave + 2)
      const float m0 = cmb[0], m1 = c1[0], mx = fmaxf(m0, m1);  // finite: a row sees itself
      const float f0 = m0 == -INFINITY ? 0.0f : __expf(m0 - mx), f1 = m1 == -INFINITY ? 0.0f : __expf(m1 - mx);
      const float inv = 1.0f / (cmb[1] * f0 + c1[1] * f1);
      if (lane < HD)
        st<T>((T*)a.o + (long)(s * nf + i) * a.D + h * HD + lane, (cmb[4 + lane] * f0 + c1[4 + lane] * f1) * inv);
    }
    return;
  }

  for (int i = wave; i < nf; i += 4) {
    const int p = pos0 + i;
    bool vis[JT];
    int rel[JT];
    const unsigned char* krow[JT];
#pragma unroll
    for (int t = 0; t < JT; ++t) {
      vis[t] = qj[t] >= 0 && att_visible(a, p, qj[t]);
      rel[t] = vis[t] ? p - qj[t] - a.rel_lo : 0;
      krow[t] = Ks + min(lane + 64 * t, R - 1) * KS;
    }
    float ac[JT], bd[JT];
#pragma unroll
    for (int t = 0; t < JT; ++t) { ac[t] = 0.0f; bd[t] = 0.0f; }
    const f32x4_v* qi = (const f32x4_v*)(Qs + i * HD);
#pragma unroll 4
    for (int c = 0; c < FC; ++c) {
      const f32x4_v q4 = qi[c];
      const f32x4_v qu = q4 + ((const f32x4_v*)Us)[c], qv = q4 + ((const f32x4_v*)Ws)[c];
#pragma unroll
      for (int t = 0; t < JT; ++t) {
        const f32x4_v k4 = lds4<T>(krow[t], c);
        const f32x4_v p4 = ((const f32x4_v*)(Ps + rel[t] * FS))[c];
        ac[t] += qu.x * k4.x + qu.y * k4.y + qu.z * k4.z + qu.w * k4.w;
        bd[t] += qv.x * p4.x + qv.y * p4.y + qv.z * p4.z + qv.w * p4.w;
      }
    }
    float sc[JT], mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < JT; ++t) {
      sc[t] = vis[t] ? (ac[t] + bd[t]) * a.scale : -INFINITY;
      mx = fmaxf(mx, sc[t]);
    }
    mx = wave_top(mx);  // finite: a query always sees its own position
    float pr[JT], sum = 0.0f;
#pragma unroll
    for (int t = 0; t < JT; ++t) {
      pr[t] = vis[t] ? __expf(sc[t] - mx) : 0.0f;
      sum += pr[t];
    }
    const float inv = 1.0f / wave_total(sum);
    // o_i = sum_j p_ij v_j: the weights go to this wave's LDS strip; slots holding no key get a
    // zero V row first (their weight is 0 but their contents are arbitrary, and 0 * NaN is NaN;
    // every wave zeroes the same rows before reading them, so no wave depends on another)
#pragma unroll
    for (int t = 0; t < JT; ++t) {
      const int j = lane + 64 * t;
      Pw[j] = pr[t];
      if (j < R && qj[t] < 0) {
#pragma unroll
        for (int c = 0; c < KC; ++c) *(u32x4_v*)(Vs + j * KS + c * 16) = u32x4_v{0u, 0u, 0u, 0u};
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lanes as (4-dim chunk c4, key phase ph): lane sums slots ph, ph + NPH, ... of its chunk
    f32x4_v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < JT * 64 / NPH; ++m) {
      const int j = ph + NPH * m;
      const float pj = Pw[j];  // 0 for slots past R
      acc += pj * lds4<T>(Vs + min(j, R - 1) * KS, c4);
    }
    // sum over the phases (lane bits log2(NCH) .. 5)
#pragma unroll
    for (int b = NCH; b < 64; b <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = acc[e];
        if (b == 32) v = pair_sum32(v, v);
        else if (b == 16) v = pair_sum16(v, v);
        else v += __shfl_xor(v, b, 64);
        acc[e] = v;
      }
    }
    if (lane < NCH) {
      T* dst = (T*)a.o + (long)(s * nf + i) * a.D + h * HD + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; ++e) st<T>(dst + e, acc[e] * inv);
    }
    __builtin_amdgcn_wave_barrier();  // the strip is rewritten by this wave's next query row
  }
}

// ------------------------------------------------------------------ bf16, head size 64, MFMA
// One wave per (call stream, head); the score and position-term products on
// v_mfma_f32_16x16x32_bf16 with the query rows as the 16-row A operand (rows past nf zero):
//   S[i][j] = (q_i + u) . K_j over 16-slot tiles, B operand = the slot's K row read straight
//     from the ring (non-temporal: read once per call);
//   T[i][r] = (q_i + v) . P[r] over 16-distance tiles of the head's position table (bf16 copy);
//   score[i][j] = (S[i][j] + T[i][p_i - q_j - rel_lo]) * scale on visible slots, else -inf
//     (T goes through LDS for the lookup by distance);
//   softmax per query row over the 16 lanes that hold it (MFMA output layout: lane l holds
//     slot 16 t + l % 16 of rows 4 (l / 16) .. + 3);
//   PV on VALU from the V rows staged in LDS by non-temporal direct copies, lanes as (4-dim
//   chunk, slot phase mod 4), every query row at once.
// q + u and q + v are rounded to bf16 for the products (K and V are bf16 already); everything
// after the products is float32. Slots holding no key (and padding slots past R) get weight 0
// and a zeroed V row.
// LDS written by some lanes of a wave and read by others: order the accesses (a wave's LDS
// operations execute in issue order, so a compiler fence suffices)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// LDS of the MFMA attention kernel: V rows of NT 16-slot tiles, then the position terms of NR
// query rows, each
// row overwritten by its softmax weights once its scores are formed (the 16 lanes that read a
// row's terms are the ones that write its weights)
__host__ __device__ constexpr int attn_mfma_vrows(int nt) { return nt * 16; }
static size_t attn_mfma_lds(int nt, int nr) { return (size_t)attn_mfma_vrows(nt) * 128 + (size_t)nr * nt * 16 * 4; }

typedef __attribute__((ext_vector_type(4))) short s16x4_v;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_w;
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4_t;

__device__ __forceinline__ float row16_max(float v) {  // over the 16 lanes of v's DPP row
  v = fmaxf(v, dpp<DPP_MIRROR16>(v));
  v = fmaxf(v, dpp<DPP_MIRROR8>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  return fmaxf(v, dpp<DPP_XOR1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<DPP_MIRROR16>(v);
  v += dpp<DPP_MIRROR8>(v);
  v += dpp<DPP_XOR2>(v);
  return v + dpp<DPP_XOR1>(v);
}

// At least 4 waves per SIMD (128 registers) up to 5 tiles and 4 query rows. Wider rings hold
// 24 registers of operands and products per tile, and 8 rows or more hold a float4 accumulator
// per row and lane in PV; their LDS already keeps them to 2-3 waves per SIMD, so they get up to
// 256 registers rather than spilling (measured 0.3% per step on the lookahead workload).
template <int NT, int NR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NR >= 8 || NT >= 6 ? 2 : 4, 8))) void attn_mfma_kernel(AttnArgs a) {
  constexpr int HD = 64, NS = NT * 16;
  static_assert(attn_mfma_vrows(NT) == NS, "LDS layout");
  extern __shared__ __attribute__((aligned(16))) unsigned char mf_lds[];
  unsigned char* Vs = mf_lds;                // [NS][128 B] V rows
  float* Ts = (float*)(mf_lds + NS * 128);   // [NR][NS] position terms by distance, then weights
  float* Ws = Ts;
  const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
  const int s = blockIdx.x / a.H, h = blockIdx.x - s * a.H;
  const int id = a.cv.ids[s];
  const int pos0 = a.cv.cpos[s];
  const int nf = a.cv.nf, R = a.R, nrel = a.nrel;
  const long head = ((long)id * a.H + h) * R * HD;
  // The head's K and V rows and its position rows are read through buffer resources sized to
  // them: the hardware range check turns reads past the last row into zeros, so the 16-row tiles
  // need no clamped addresses (the slots past R are masked, and their V rows zeroed, below).
  const __amdgpu_buffer_rsrc_t kr = raw_rsrc((const bf16_t*)a.kring + head, R * HD * 2);
  const __amdgpu_buffer_rsrc_t vr = raw_rsrc((const bf16_t*)a.vring + head, R * HD * 2);
  const __amdgpu_buffer_rsrc_t pr = raw_rsrc((const bf16_t*)a.posproj_bf + (long)h * nrel * HD, nrel * HD * 2);
#pragma unroll
  for (int c0 = 0; c0 < NS * 8; c0 += 64)  // V rows to LDS, 16 bytes per lane
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(Vs + c0 * 16), 16, (c0 + lane) * 16, 0, 0, CPOL_NT);
  // K and position rows as B operands: tile t, k-step ks -> row 16 t + l16, dims 32 ks + 8 lg ..
  u32x4_v kb[NT][2], pb[NT][2];
  {
    const int bo = l16 * HD * 2 + lg * 16;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off = bo + t * 16 * HD * 2 + ks * 64;
        kb[t][ks] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, CPOL_NT));
        pb[t][ks] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
      }
  }
  // query rows as A operands: row l16 (zero past nf), dims 32 ks + 8 lg .. + 7
  u32x4_v qa[2], qb[2];
  {
    const bool live = l16 < nf;
    const float* qp = a.q + ((long)s * nf + min(l16, nf - 1)) * a.D + h * HD + 8 * lg;
    const float* up = a.pos_u + h * HD + 8 * lg;
    const float* vp = a.pos_v + h * HD + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4_v q0 = *(const f32x4_v*)(qp + 32 * ks), q1 = *(const f32x4_v*)(qp + 32 * ks + 4);
      const f32x4_v u0 = *(const f32x4_v*)(up + 32 * ks), u1 = *(const f32x4_v*)(up + 32 * ks + 4);
      const f32x4_v v0 = *(const f32x4_v*)(vp + 32 * ks), v1 = *(const f32x4_v*)(vp + 32 * ks + 4);
      const f32x4_v a0 = q0 + u0, a1 = q1 + u1, b0 = q0 + v0, b1 = q1 + v1;
      qa[ks] = live ? u32x4_v{pack_bf2(a0.x, a0.y), pack_bf2(a0.z, a0.w), pack_bf2(a1.x, a1.y), pack_bf2(a1.z, a1.w)}
                    : u32x4_v{0u, 0u, 0u, 0u};
      qb[ks] = live ? u32x4_v{pack_bf2(b0.x, b0.y), pack_bf2(b0.z, b0.w), pack_bf2(b1.x, b1.y), pack_bf2(b1.z, b1.w)}
                    : u32x4_v{0u, 0u, 0u, 0u};
    }
  }
  // ---- the two products
  f32x4_v S[NT], T[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    S[t] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    T[t] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      S[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, qa[ks]), __builtin_bit_cast(bf16x8_v, kb[t][ks]),
                                                     S[t], 0, 0, 0);
      T[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, qb[ks]), __builtin_bit_cast(bf16x8_v, pb[t][ks]),
                                                     T[t], 0, 0, 0);
    }
  }
  // ---- ring slot positions; zero the V rows of slots without a key once the copies landed
  const int pe = pos0 + nf - 1, pm = pe % R, q_lo = max(0, pos0 - a.Lc);
  auto slot_pos = [&](int j) {  // -1: no key (also the padding slots j >= R)
    int dd = pm - j;
    dd += dd < 0 ? R : 0;
    return (j < R && pe - dd >= q_lo) ? pe - dd : -1;
  };
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  wave_sync();
#pragma unroll
  for (int j0 = 0; j0 < NS; j0 += 8) {
    const int j = j0 + (lane >> 3);
    if (slot_pos(j) < 0) *(u32x4_v*)(Vs + j * 128 + (lane & 7) * 16) = u32x4_v{0u, 0u, 0u, 0u};
  }
  // position terms to LDS (rows 4 lg + c of each tile; with NR < 4 only lanes lg = 0 hold kept
  // rows, and only their first NR)
  constexpr int CR = NR < 4 ? NR : 4;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < CR; ++c)
      if (4 * lg + c < NR) Ts[(4 * lg + c) * NS + 16 * t + l16] = T[t][c];
  wave_sync();
  // ---- scores and softmax of rows 4 lg + c
  int qk[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) qk[t] = slot_pos(16 * t + l16);
#pragma unroll
  for (int c = 0; c < CR; ++c) {
    const int m = 4 * lg + c;
    const int p = pos0 + m;
    int lo, hi;
    if (a.lookahead) { lo = p - a.Lc; hi = p + a.right; }
    else { const int cs = p - p % a.chunk; lo = cs - a.Lc; hi = cs + a.chunk - 1; }
    lo = max(lo, 0);
    if (m >= nf) hi = -1;  // rows past the call's frames see nothing
    const float* tr = Ts + min(m, NR - 1) * NS;
    float x[NT], mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int q = qk[t];
      const bool vis = q >= lo && q <= hi;  // q = -1 (no key) fails q >= lo
      x[t] = vis ? (S[t][c] + tr[vis ? p - q - a.rel_lo : 0]) * a.scale : -INFINITY;
      mx = fmaxf(mx, x[t]);
    }
    mx = row16_max(mx);
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      x[t] = mx == -INFINITY ? 0.0f : __expf(x[t] - mx);
      sum += x[t];
    }
    sum = row16_sum(sum);
    const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
    if (m < NR) {
#pragma unroll
      for (int t = 0; t < NT; ++t) Ws[m * NS + 16 * t + l16] = x[t] * inv;
    }
  }
  wave_sync();
  // ---- PV on v_mfma_f32_16x16x32_bf16: O[i][d] = sum_j W[i][j] V[j][d] over 32-slot k-steps
  // (and one 16-slot step on v_mfma_f32_16x16x16_bf16 when NT is odd), the weights rounded to
  // bf16 as the 16-row A operand (rows past NR zero) and V as the B operand in 16-dim tiles.
  // B needs consecutive slots of one dim per lane, V rows hold dims: ds_read_b64_tr_b16
  // transposes within each 16-lane group, giving lane i of the group element i % 4 of the 4
  // read by lane 4 j + i / 4 as its j-th value. So lane i reads dims d0 + 4 (i % 4) .. + 3 of
  // slot (group slot base) + i / 4, and every lane ends with dim d0 + i of 4 consecutive slots;
  // two such reads make the 8 of a 32-slot step.
  f32x4_v O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < NS / 32; ++ks) {
    const int j0 = 32 * ks + 8 * lg;  // this lane's 8 slots of the k-step (A and B alike)
    u32x4_v wa = u32x4_v{0u, 0u, 0u, 0u};
    if (l16 < NR) {
      const f32x4_v w0 = *(const f32x4_v*)(Ws + l16 * NS + j0), w1 = *(const f32x4_v*)(Ws + l16 * NS + j0 + 4);
      wa = u32x4_v{pack_bf2(w0.x, w0.y), pack_bf2(w0.z, w0.w), pack_bf2(w1.x, w1.y), pack_bf2(w1.z, w1.w)};
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const unsigned char* vb = Vs + (j0 + (l16 >> 2)) * 128 + (16 * dt + 4 * (l16 & 3)) * 2;
      const s16x4_v b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vb);
      const s16x4_v b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + 4 * 128));
      const u32x2_w p0 = __builtin_bit_cast(u32x2_w, b0), p1 = __builtin_bit_cast(u32x2_w, b1);
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, wa),
                                                      __builtin_bit_cast(bf16x8_v, u32x4_v{p0.x, p0.y, p1.x, p1.y}), O[dt], 0, 0, 0);
    }
  }
  if constexpr (NS % 32 != 0) {  // the last 16 slots: 4 per lane group
    const int j0 = NS - 16 + 4 * lg;
    u32x2_w wa = u32x2_w{0u, 0u};
    if (l16 < NR) {
      const f32x4_v w0 = *(const f32x4_v*)(Ws + l16 * NS + j0);
      wa = u32x2_w{pack_bf2(w0.x, w0.y), pack_bf2(w0.z, w0.w)};
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const unsigned char* vb = Vs + (j0 + (l16 >> 2)) * 128 + (16 * dt + 4 * (l16 & 3)) * 2;
      const s16x4_v b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vb);
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_v, wa), b0, O[dt], 0, 0, 0);
    }
  }
  // O[dt] element r of a lane: query row 4 (lane / 16) + r, dim 16 dt + lane % 16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * lg + r;
    if (i < nf && i < NR) {
      bf16_t* dst = (bf16_t*)a.o + ((long)s * nf + i) * a.D + h * HD + l16;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) dst[16 * dt] = f2bf(O[dt][r]);
    }
  }
}

template <int NT>
static const void* attn_mfma_pick_nr(int nf) {
  if (nf <= 2) return (const void*)&attn_mfma_kernel<NT, 2>;
  if (nf <= 4) return (const void*)&attn_mfma_kernel<NT, 4>;
  if (nf <= 8) return (const void*)&attn_mfma_kernel<NT, 8>;
  if (nf <= 12) return (const void*)&attn_mfma_kernel<NT, 12>;
  return (const void*)&attn_mfma_kernel<NT, 16>;
}
static int attn_mfma_nr(int nf) { return nf <= 2 ? 2 : nf <= 4 ? 4 : nf <= 8 ? 8 : nf <= 12 ? 12 : 16; }

void launch_attention(Launcher& L, const AttnArgs& a, int dtype, int hd) {
  AttnArgs args = a;
  if (dtype == DT_BF16 && hd == 64 && a.posproj_bf && a.R <= 128 && a.nrel <= 128 && a.cv.nf <= 16) {
    const int nt = (std::max(a.R, a.nrel) + 15) / 16;
    const void* fn = nullptr;
    switch (nt) {
      case 1: case 2: case 3: case 4: fn = attn_mfma_pick_nr<4>(a.cv.nf); break;
      case 5: fn = attn_mfma_pick_nr<5>(a.cv.nf); break;
      case 6: fn = attn_mfma_pick_nr<6>(a.cv.nf); break;
      case 7: fn = attn_mfma_pick_nr<7>(a.cv.nf); break;
      default: fn = attn_mfma_pick_nr<8>(a.cv.nf); break;
    }
    L.tag_name = "attention";
    L.launch(fn, dim3(a.cv.n_streams * a.H), dim3(64), attn_mfma_lds(std::max(nt, 4), attn_mfma_nr(a.cv.nf)), &args);
    return;
  }
  const size_t shm = attention_shmem(a.cv.nf, a.R, a.nrel, hd, dtype == DT_F32 ? 4 : 2);
  const void* fn = nullptr;
  const bool wide = a.R > 128;  // ring slots per lane: 2 up to R = 128, else 4 (R <= 256)
#define ATT_PICK(HDV)                                                                                     \
  fn = dtype == DT_F32 ? (wide ? (const void*)&attn_kernel<float, HDV, 4> : (const void*)&attn_kernel<float, HDV, 2>) \
                       : (wide ? (const void*)&attn_kernel<bf16_t, HDV, 4> : (const void*)&attn_kernel<bf16_t, HDV, 2>);
  if (hd == 16) { ATT_PICK(16) } else if (hd == 32) { ATT_PICK(32) } else { ATT_PICK(64) }
#undef ATT_PICK
  L.tag_name = "attention";  // the caller tags bytes and flops (it knows each stream's fill)
  L.launch(fn, dim3(a.cv.n_streams * a.H), dim3(256), shm, &args);
}

// =============================================================================== depthwise conv
// One thread per (row, 4 channels): the taps and ring rows are loaded together, positions
// before the stream start read as zero.
template <typename T>
__device__ __forceinline__ void dw_row4(const DwArgs& a, int m, int c) {
  const int s = m / a.cv.nf, i = m % a.cv.nf;
  const int id = a.cv.ids[s];
  const int p = a.cv.cpos[s] + i;
  const T* ring = (const T*)a.cring;  // 4 channels of one 32-channel block per read
  float g[16][4];
  float4 w[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int q = p - (a.K - 1) + t;
    const bool ok = t < a.K && q >= 0;
    w[t] = t < a.K ? *(const float4*)(a.w + t * a.D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (sizeof(T) == 4) {
      const float4 v = ok ? *(const float4*)(ring + cring_idx(id, q % a.Rc, c, a.D, a.Rc)) : make_float4(0.f, 0.f, 0.f, 0.f);
      g[t][0] = v.x; g[t][1] = v.y; g[t][2] = v.z; g[t][3] = v.w;
    } else {
      const uint2 v = ok ? *(const uint2*)(ring + cring_idx(id, q % a.Rc, c, a.D, a.Rc)) : make_uint2(0u, 0u);
      g[t][0] = __uint_as_float(v.x << 16); g[t][1] = __uint_as_float(v.x & 0xffff0000u);
      g[t][2] = __uint_as_float(v.y << 16); g[t][3] = __uint_as_float(v.y & 0xffff0000u);
    }
  }
  const float4 b4 = *(const float4*)(a.b + c);
  float acc[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    acc[0] += w[t].x * g[t][0]; acc[1] += w[t].y * g[t][1]; acc[2] += w[t].z * g[t][2]; acc[3] += w[t].w * g[t][3];
  }
  T* e = (T*)a.e + (long)m * a.D + c;
#pragma unroll
  for (int q = 0; q < 4; ++q) st<T>(e + q, silu_f(acc[q]));
}

template <typename T>
__global__ __launch_bounds__(256) void dw_kernel(DwArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int cg = a.D / 4;
  const long total = (long)a.cv.n_streams * a.cv.nf * cg;
  if (idx >= total) return;
  dw_row4<T>(a, (int)(idx / cg), (int)(idx % cg) * 4);
}

// The streams whose rows cross a multiple of 64 rows (one per boundary at most, the frames per
// call being at most 64): the MFMA GLU epilogue leaves their conv to this kernel, blockIdx.y
// the boundary 64 (y + 1), x over the stream's (frame, 4 channels).
__global__ __launch_bounds__(256) void dw_straddle_kernel(DwArgs a) {
  const int b = 64 * ((int)blockIdx.y + 1), nf = a.cv.nf, s = b / nf;
  if (b % nf == 0 || s >= a.cv.n_streams) return;
  const int cg = a.D / 4, idx = (int)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nf * cg) return;
  dw_row4<bf16_t>(a, s * nf + idx / cg, (idx % cg) * 4);
}

void launch_dwconv(Launcher& L, const DwArgs& a, int dtype) {
  DwArgs args = a;
  const long total = (long)a.cv.n_streams * a.cv.nf * (a.D / 4);
  const void* fn = dtype == DT_F32 ? (const void*)&dw_kernel<float> : (const void*)&dw_kernel<bf16_t>;
  L.tag_name = "dwconv";  // the caller tags bytes and flops
  L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

bool launch_dwconv_straddle(Launcher& L, const DwArgs& a) {
  const int M = a.cv.n_streams * a.cv.nf;
  if (a.cv.nf < 1 || a.cv.nf > 64 || 64 % a.cv.nf == 0 || M <= 64) return false;  // no stream crosses
  DwArgs args = a;  // the caller tags the launch
  L.launch((const void*)&dw_straddle_kernel, dim3((unsigned)((a.cv.nf * (a.D / 4) + 255) / 256), (unsigned)((M - 1) / 64)),
           dim3(256), 0, &args);
  return true;
}

// =============================================================================== input, FE window
template <typename T>
__global__ __launch_bounds__(256) void input_kernel(InputArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx < (long)a.M * a.D) a.x[idx] = ld<T>((const T*)a.in + idx);
  // the call's positions for every later kernel (they read cpos only), then the streams advance
  if (idx < a.cv.n_streams) {
    const int id = a.cv.ids[idx], p = a.pos[id];
    a.cv.cpos[idx] = p;
    a.pos[id] = p + a.adv;
  }
}
void launch_input(Launcher& L, const InputArgs& a, int dtype) {
  InputArgs args = a;
  const long total = (long)a.M * a.D;
  const void* fn = dtype == DT_F32 ? (const void*)&input_kernel<float> : (const void*)&input_kernel<bf16_t>;
  L.tag("input", (double)total * (dtype == DT_F32 ? 4 : 2), 0.0);
  L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

__global__ __launch_bounds__(256) void copy_rows_kernel(CopyRowsArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.M * a.D) return;
  const int m = (int)(idx / a.D), c = (int)(idx % a.D);
  const long row = a.omap ? (long)a.omap[m / a.ogroup] * a.ostride + m % a.ogroup : m;
  a.out[row * a.D + c] = a.x[a.amap.off(m) + c];
}
void launch_copy_rows(Launcher& L, const CopyRowsArgs& a) {
  CopyRowsArgs args = a;
  const long total = (long)a.M * a.D;
  L.tag("copy_rows", (double)total * 4, 0.0);
  L.launch((const void*)&copy_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

// One thread per (call stream, mel bin): window = [tail || new], tail <- last rows of window.
// Mel frames before the stream start are zero regardless of what the tail slot holds.
template <typename T>
__global__ __launch_bounds__(256) void fe_window_kernel(FeWindowArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.cv.n_streams * a.bins) return;
  const int s = idx / a.bins, b = idx % a.bins;
  const int id = a.cv.ids[s];
  const int pos = a.cv.pos[id];
  const bool fresh = pos == 0;
  if (b == 0) a.cv.cpos[s] = pos;
  const int nt = a.mel_tail, nn = a.mel_new, rows = nt + nn;
  T* tail = (T*)a.tail + (long)id * nt * a.bins + b;
  const T* mel = (const T*)a.mel + (long)s * nn * a.bins + b;
  T* win = (T*)a.win + (long)s * rows * a.bins + b;
  for (int r = 0; r < nt; ++r) win[(long)r * a.bins] = fresh ? T(0) : tail[(long)r * a.bins];
  for (int r = 0; r < nn; ++r) win[(long)(nt + r) * a.bins] = mel[(long)r * a.bins];
  for (int r = 0; r < nt; ++r) tail[(long)r * a.bins] = win[(long)(rows - nt + r) * a.bins];
}
// The same with one thread per (call stream, 16 bytes of bins) for windows of at most FW_MAXR
// rows: every row is loaded into registers before any is stored, so the tail rows this thread
// reads are read before it overwrites them, and all loads share one memory round trip (the
// per-bin kernel pays one per row).
constexpr int FW_MAXR = 32;
template <typename T>
__global__ __launch_bounds__(256) void fe_window_vec_kernel(FeWindowArgs a) {
  constexpr int E = 16 / sizeof(T);
  const int nch = a.bins / E;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.cv.n_streams * nch) return;
  const int s = idx / nch, ch = idx - s * nch;
  const int id = a.cv.ids[s];
  const int pos = a.cv.pos[id];
  const bool fresh = pos == 0;
  if (ch == 0) a.cv.cpos[s] = pos;
  const int nt = a.mel_tail, nn = a.mel_new, rows = nt + nn;
  u32x4_v* tail = (u32x4_v*)((T*)a.tail + (long)id * nt * a.bins) + ch;
  const u32x4_v* mel = (const u32x4_v*)((const T*)a.mel + (long)s * nn * a.bins) + ch;
  u32x4_v* win = (u32x4_v*)((T*)a.win + (long)s * rows * a.bins) + ch;
  u32x4_v v[FW_MAXR];
#pragma unroll
  for (int r = 0; r < FW_MAXR; ++r) {
    if (r < nt) v[r] = fresh ? u32x4_v{0u, 0u, 0u, 0u} : tail[r * nch];
    else if (r < rows) v[r] = mel[(r - nt) * nch];
  }
#pragma unroll
  for (int r = 0; r < FW_MAXR; ++r)
    if (r < rows) win[r * nch] = v[r];
#pragma unroll
  for (int r = 0; r < FW_MAXR; ++r)  // the last nt rows of the window become the tail
    if (r < rows && r >= rows - nt) tail[(r - (rows - nt)) * nch] = v[r];
}

void launch_fe_window(Launcher& L, const FeWindowArgs& a, int dtype) {
  FeWindowArgs args = a;
  const int esz = dtype == DT_F32 ? 4 : 2;
  L.tag("fe_window", (double)a.cv.n_streams * (a.mel_new + 2 * a.mel_tail) * a.bins * esz, 0.0);
  if ((a.bins * esz) % 16 == 0 && a.mel_tail + a.mel_new <= FW_MAXR) {
    const int total = a.cv.n_streams * (a.bins * esz / 16);
    const void* fn = dtype == DT_F32 ? (const void*)&fe_window_vec_kernel<float> : (const void*)&fe_window_vec_kernel<bf16_t>;
    L.launch(fn, dim3((total + 255) / 256), dim3(256), 0, &args);
    return;
  }
  const int total = a.cv.n_streams * a.bins;
  const void* fn = dtype == DT_F32 ? (const void*)&fe_window_kernel<float> : (const void*)&fe_window_kernel<bf16_t>;
  L.launch(fn, dim3((total + 255) / 256), dim3(256), 0, &args);
}

// One thread per (stream, output row, output column, 8 channels): 9 taps, 16-byte stores.
__global__ __launch_bounds__(256) void fe2d_kernel(Fe2dArgs a) {
  const int c8 = a.C / 8;
  long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.cv.n_streams * a.Tout * a.Fout * c8;
  if (idx >= total) return;
  const int cg = (int)(idx % c8);
  idx /= c8;
  const int f = (int)(idx % a.Fout);
  idx /= a.Fout;
  const int r = (int)(idx % a.Tout);
  const int s = (int)(idx / a.Tout);
  const int c0 = cg * 8;
  float acc[8];
  ld_f8(a.b + c0, acc);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int row = 2 * r + i;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int col = 2 * f + j - 1;
      if (col < 0 || col >= a.Fin) continue;
      float w[8];
      ld_f8(a.w + (long)(i * 3 + j) * a.C + c0, w);
      if (a.cin1) {
        const float v = bf2f(((const bf16_t*)a.in)[((long)s * a.Tin + row) * a.Fin + col]);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += w[q] * v;
      } else {
        const u32x4_v raw = *(const u32x4_v*)((const bf16_t*)a.in + (((long)s * a.Tin + row) * a.Fin + col) * a.C + c0);
        const unsigned int u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += w[2 * q] * __uint_as_float(u[q] << 16);
          acc[2 * q + 1] += w[2 * q + 1] * __uint_as_float(u[q] & 0xffff0000u);
        }
      }
    }
  }
  if (a.cin1) {
    const bool before_start = a.cv.cpos[s] == 0 && r < a.neg;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = before_start ? 0.0f : fmaxf(acc[q], 0.0f);
  }
  st_bf8((bf16_t*)a.out + (((long)s * a.Tout + r) * a.Fout + f) * a.C + c0, acc);
}

// The same stages with one thread per (stream, output row, FE2D_FG consecutive output columns,
// 8 channels): the 9 taps' weights are loaded once for the thread's FE2D_FG outputs, and the
// input pixels its outputs share (stride 2, width 3) once; threads of one pixel group differ
// in their channels only. Needs Fout a multiple of FE2D_FG.
constexpr int FE2D_FG = 4;
template <bool CIN1>
__global__ __launch_bounds__(256) void fe2d_group_kernel(Fe2dArgs a) {
  constexpr int FG = FE2D_FG, NIC = 2 * FG + 1;  // input columns 2 f0 - 1 .. 2 f0 + 2 FG - 1
  const int c8 = a.C / 8, fgs = a.Fout / FG;
  long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.cv.n_streams * a.Tout * fgs * c8;
  if (idx >= total) return;
  const int cg = (int)(idx % c8);
  idx /= c8;
  const int f0 = (int)(idx % fgs) * FG;
  idx /= fgs;
  const int r = (int)(idx % a.Tout);
  const int s = (int)(idx / a.Tout);
  const int c0 = cg * 8;
  float w[9][8], acc[FG][8];
#pragma unroll
  for (int t = 0; t < 9; ++t) ld_f8(a.w + (long)t * a.C + c0, w[t]);
  {
    float b[8];
    ld_f8(a.b + c0, b);
#pragma unroll
    for (int o = 0; o < FG; ++o)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[o][q] = b[q];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const long rowbase = (long)s * a.Tin + 2 * r + i;
    if constexpr (CIN1) {
      float v[NIC];
#pragma unroll
      for (int j = 0; j < NIC; ++j) {
        const int col = 2 * f0 - 1 + j;
        v[j] = (col >= 0 && col < a.Fin) ? bf2f(((const bf16_t*)a.in)[rowbase * a.Fin + col]) : 0.0f;
      }
#pragma unroll
      for (int o = 0; o < FG; ++o)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[o][q] += w[i * 3 + j][q] * v[2 * o + j];
    } else {
      u32x4_v raw[NIC];
#pragma unroll
      for (int j = 0; j < NIC; ++j) {
        const int col = 2 * f0 - 1 + j;
        raw[j] = (col >= 0 && col < a.Fin) ? *(const u32x4_v*)((const bf16_t*)a.in + (rowbase * a.Fin + col) * a.C + c0)
                                           : u32x4_v{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int o = 0; o < FG; ++o)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const u32x4_v u = raw[2 * o + j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[o][2 * q] += w[i * 3 + j][2 * q] * __uint_as_float(u[q] << 16);
            acc[o][2 * q + 1] += w[i * 3 + j][2 * q + 1] * __uint_as_float(u[q] & 0xffff0000u);
          }
        }
    }
  }
  const bool zero = CIN1 && a.cv.cpos[s] == 0 && r < a.neg;
#pragma unroll
  for (int o = 0; o < FG; ++o) {
    if constexpr (CIN1) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[o][q] = zero ? 0.0f : fmaxf(acc[o][q], 0.0f);
    }
    st_bf8((bf16_t*)a.out + (((long)s * a.Tout + r) * a.Fout + f0 + o) * a.C + c0, acc[o]);
  }
}

void launch_fe2d(Launcher& L, const Fe2dArgs& a) {
  Fe2dArgs args = a;
  const double outb = (double)a.cv.n_streams * a.Tout * a.Fout * a.C * 2.0;
  L.tag(a.cin1 ? "fe2d_conv1" : "fe2d_depthwise", 0.0, 2.0 * 9.0 * outb / 2.0);
  if (a.Fout % FE2D_FG == 0 && a.C % 8 == 0) {
    const long total = (long)a.cv.n_streams * a.Tout * (a.Fout / FE2D_FG) * (a.C / 8);
    const void* fn = a.cin1 ? (const void*)&fe2d_group_kernel<true> : (const void*)&fe2d_group_kernel<false>;
    L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
    return;
  }
  const long total = (long)a.cv.n_streams * a.Tout * a.Fout * (a.C / 8);
  L.launch((const void*)&fe2d_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

// Stage 1 and the depthwise stage after it for one stream and 32 channels per block: the mel
// window and the stage-1 map (bf16, rounded as the separate launches store it) sit in LDS, so
// the 11 x F1 x C stage-1 map never goes to memory (at 1024 streams, 128 bins, 256 channels it
// is 369 MB per call, which the separate stage-1 launch spent ~190 us writing). Stage 1: thread
// (column f, 8-channel group) over the rows; depthwise: thread (column, 8-channel group, row
// parity) over every other row, 16-byte stores, the block's 4 groups of a position adjacent.
constexpr int FE2D_CB = 32;
__global__ __launch_bounds__(256) void fe2d_s1dw_kernel(Fe2dS1DwArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char fe_lds[];
  bf16_t* win = (bf16_t*)fe_lds;                                     // [Tin][Fin]
  bf16_t* m1 = (bf16_t*)(fe_lds + ((a.Tin * a.Fin * 2 + 15) & ~15));  // [T1][F1][32]
  const int ncb = a.C / FE2D_CB, s = blockIdx.x / ncb, cb = blockIdx.x - s * ncb, tid = threadIdx.x;
  const int cg = tid & 3, c0 = cb * FE2D_CB + cg * 8;
  {  // the window, 16 bytes per thread
    const u32x4_v* src = (const u32x4_v*)((const bf16_t*)a.in + (long)s * a.Tin * a.Fin);
    const int n16 = a.Tin * a.Fin / 8;
    for (int k = tid; k < n16; k += 256) ((u32x4_v*)win)[k] = src[k];
  }
  float w[9][8], b[8];
#pragma unroll
  for (int t = 0; t < 9; ++t) ld_f8(a.w1 + (long)t * a.C + c0, w[t]);
  ld_f8(a.b1 + c0, b);
  const bool fresh = a.cv.cpos[s] == 0;
  __syncthreads();
  const int f = tid >> 2;
  if (f < a.F1) {
    for (int r = 0; r < a.T1; ++r) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = b[q];
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) {  // unconditional reads (clamped column), padding selected out
          const int col = 2 * f + j - 1;
          const float raw = bf2f(win[(2 * r + i) * a.Fin + min(max(col, 0), a.Fin - 1)]);
          const float v = (col >= 0 && col < a.Fin) ? raw : 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += w[i * 3 + j][q] * v;
        }
      const bool zero = fresh && r < a.neg1;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = zero ? 0.0f : fmaxf(acc[q], 0.0f);
      *(u32x4_v*)(m1 + ((r * a.F1 + f) * FE2D_CB + cg * 8)) =
          u32x4_v{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]), pack_bf2(acc[6], acc[7])};
    }
  }
#pragma unroll
  for (int t = 0; t < 9; ++t) ld_f8(a.w2 + (long)t * a.C + c0, w[t]);
  ld_f8(a.b2 + c0, b);
  __syncthreads();
  const int f2 = (tid >> 2) & 31, rh = tid >> 7;
  if (f2 >= a.F2) return;
  for (int r2 = rh; r2 < a.T2; r2 += 2) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = b[q];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int col = 2 * f2 + j - 1;
        const u32x4_v raw = *(const u32x4_v*)(m1 + (((2 * r2 + i) * a.F1 + min(max(col, 0), a.F1 - 1)) * FE2D_CB + cg * 8));
        const u32x4_v u = (col >= 0 && col < a.F1) ? raw : u32x4_v{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += w[i * 3 + j][2 * q] * __uint_as_float(u[q] << 16);
          acc[2 * q + 1] += w[i * 3 + j][2 * q + 1] * __uint_as_float(u[q] & 0xffff0000u);
        }
      }
    st_bf8((bf16_t*)a.out + (((long)s * a.T2 + r2) * a.F2 + f2) * a.C + c0, acc);
  }
}

bool launch_fe2d_s1dw(Launcher& L, const Fe2dS1DwArgs& a) {
  if (a.C % FE2D_CB || a.F1 > 64 || a.F2 > 32 || (a.Tin * a.Fin) % 8 || 2 * a.T2 + 1 > a.T1 || 2 * a.T1 + 1 > a.Tin)
    return false;
  Fe2dS1DwArgs args = a;
  const size_t lds = (size_t)((a.Tin * a.Fin * 2 + 15) & ~15) + (size_t)a.T1 * a.F1 * FE2D_CB * 2;
  if (lds > 64 * 1024) return false;
  const double n = a.cv.n_streams;
  L.tag("fe2d_conv1_depthwise", n * a.T2 * a.F2 * a.C * 2.0, 2.0 * 9.0 * n * (a.T1 * a.F1 + a.T2 * a.F2) * a.C);
  L.launch((const void*)&fe2d_s1dw_kernel, dim3((unsigned)(a.cv.n_streams * (a.C / FE2D_CB))), dim3(256), lds, &args);
  return true;
}

// =============================================================================== positions
__global__ void advance_kernel(AdvanceArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.n) return;
  const int id = a.ids[s];
  a.pos[id] += a.adv;
  if (a.pend) a.pend[id] += a.dpend;
}
void launch_advance(Launcher& L, const AdvanceArgs& a) {
  AdvanceArgs args = a;
  L.tag("advance", 0.0, 0.0);
  L.launch((const void*)&advance_kernel, dim3((a.n + 255) / 256), dim3(256), 0, &args);
}

__global__ __launch_bounds__(256) void fill_kernel(FillArgs a) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < a.n; i += (long)gridDim.x * 256) a.p[i] = a.v;
}

void launch_fill(Launcher& L, const FillArgs& a) {
  FillArgs args = a;
  L.tag("fill", 0.0, 0.0);
  L.launch((const void*)&fill_kernel, dim3((unsigned)std::min<long>((a.n + 255) / 256, 4096)), dim3(256), 0, &args);
}

// =============================================================================== position table
// Block per (layer, relative offset): the sinusoid row PE(rel) is formed once in LDS (double
// precision), then each thread owns one output column of PE(rel) @ Wpos_l.
__global__ __launch_bounds__(512) void posproj_kernel(PosProjArgs a) {
  extern __shared__ double pe[];
  const int l = blockIdx.y, r = blockIdx.x;
  const double rel = (double)(a.rel_lo + r);
  for (int e = threadIdx.x; e < a.D; e += blockDim.x) {
    const int m = e >> 1;
    const double ang = rel * pow(10000.0, -2.0 * m / (double)a.D);
    pe[e] = (e & 1) ? cos(ang) : sin(ang);
  }
  __syncthreads();
  const float* w = a.wpos + (long)l * a.D * a.D;
  for (int col = threadIdx.x; col < a.D; col += blockDim.x) {
    double acc = 0.0;
    for (int e = 0; e < a.D; ++e) acc += pe[e] * (double)w[(long)e * a.D + col];
    const int h = col / a.hd, d = col % a.hd;
    a.table[(((long)l * a.H + h) * a.nrel + r) * a.hd + d] = (float)acc;
  }
}
void launch_posproj(Launcher& L, const PosProjArgs& a) {
  PosProjArgs args = a;
  L.tag("posproj", 0.0, 0.0);
  L.launch((const void*)&posproj_kernel, dim3(a.nrel, a.L), dim3(512), (size_t)a.D * sizeof(double), &args);
}

// =============================================================================== stream state
// Flattened per-stream state: K ring rows, V ring rows, conv ring, mel tail, pending ring.
// op 0: reset (0 or NaN), op 1: import from the canonical blob, op 2: export to it.
template <typename T>
__device__ __forceinline__ T fill_val(int poison) {
  return poison ? (T)NAN : (T)0;
}
template <>
__device__ __forceinline__ bf16_t fill_val<bf16_t>(int poison) {
  return poison ? (bf16_t)0x7fc0 : (bf16_t)0;
}

template <typename T>
__global__ __launch_bounds__(256) void state_reset_kernel(StateArgs a) {
  const int s = blockIdx.y;
  const int id = a.ids[s];
  const long kv = (long)a.H * a.R * a.hd;    // per (layer, stream) in each K/V ring
  const long cv = (long)a.Rc * a.D;          // per (layer, stream) in the conv ring
  const long tl = (long)a.tail_rows * a.bins;
  const long x0 = (long)a.Rx * a.D;
  const long per = a.L * (2 * kv + cv) + tl + x0;
  const T fv = fill_val<T>(a.poison);
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < per; e += (long)gridDim.x * 256) {
    long r = e;
    if (r < a.L * kv) { long l = r / kv, o = r % kv; ((T*)a.kring)[(l * a.S + id) * kv + o] = fv; continue; }
    r -= a.L * kv;
    if (r < a.L * kv) { long l = r / kv, o = r % kv; ((T*)a.vring)[(l * a.S + id) * kv + o] = fv; continue; }
    r -= a.L * kv;
    if (r < a.L * cv) { long l = r / cv, o = r % cv; ((T*)a.cring)[(l * a.S + id) * cv + o] = fv; continue; }
    r -= a.L * cv;
    if (r < tl) { ((T*)a.tail)[id * tl + r] = fv; continue; }
    r -= tl;
    ((T*)a.x0)[id * x0 + r] = fv;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) { a.pos[id] = 0; a.pend[id] = 0; }
}

// Canonical blob of one stream (floats): header [STATE_HDR] (32-bit words), K [L][Lc][D],
// V [L][Lc][D], conv [L][Kc][D], tail [tail_rows][bins], x0 [nla][D]. Export writes the
// header; import leaves it to the host, which has checked it.
template <typename T, bool IMPORT>
__global__ __launch_bounds__(256) void state_xfer_kernel(StateArgs a) {
  const int s = blockIdx.y;
  const int id = a.ids[s];
  const int pos = a.hpos[s];
  const int pend = a.hpend ? a.hpend[s] : 0;
  float* blob = a.blob + (long)s * a.state_floats + STATE_HDR;
  if (!IMPORT && blockIdx.x == 0 && threadIdx.x < STATE_HDR) ((uint32_t*)blob)[(int)threadIdx.x - STATE_HDR] = a.hdr[threadIdx.x];
  const long kvn = (long)a.L * a.Lc * a.D, cvn = (long)a.L * a.Kc * a.D;
  const long tln = (long)a.tail_rows * a.bins;
  const long body = a.state_floats - STATE_HDR;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < body; e += (long)gridDim.x * 256) {
    long r = e;
    T* dst = nullptr;
    bool valid = false;
    if (r < 2 * kvn) {
      const int which = r >= kvn;
      if (which) r -= kvn;
      const long l = r / ((long)a.Lc * a.D), row = (r / a.D) % a.Lc, c = r % a.D;
      const int q = pos - a.Lc + (int)row;
      valid = q >= 0;
      if (valid) {
        const int h = (int)(c / a.hd), d = (int)(c % a.hd);
        T* ring = (T*)(which ? a.vring : a.kring);
        dst = ring + ((((l * a.S + id) * a.H + h) * a.R) + q % a.R) * a.hd + d;
      }
    } else if ((r -= 2 * kvn) < cvn) {
      const long l = r / ((long)a.Kc * a.D), j = (r / a.D) % a.Kc, c = r % a.D;
      const int q = pos - a.Kc + (int)j;
      valid = q >= 0;
      if (valid) dst = (T*)a.cring + cring_idx(l * a.S + id, q % a.Rc, (int)c, a.D, a.Rc);
    } else if ((r -= cvn) < tln) {
      valid = true;
      dst = (T*)a.tail + id * tln + r;
    } else {
      r -= tln;
      const long j = r / a.D, c = r % a.D;
      valid = j < pend;
      if (valid) dst = (T*)a.x0 + ((long)id * a.Rx + (pos + j) % a.Rx) * a.D + c;
    }
    if (IMPORT) {
      if (valid) st<T>(dst, blob[e]);
    } else {
      blob[e] = valid ? ld<T>(dst) : 0.0f;
    }
  }
  if (IMPORT && blockIdx.x == 0 && threadIdx.x == 0) { a.pos[id] = pos; a.pend[id] = pend; }
}

void launch_state(Launcher& L, const StateArgs& a, int op) {
  StateArgs args = a;
  const bool f32 = a.dtype == DT_F32;
  const void* fn;
  if (op == 0) fn = f32 ? (const void*)&state_reset_kernel<float> : (const void*)&state_reset_kernel<bf16_t>;
  else if (op == 1) fn = f32 ? (const void*)&state_xfer_kernel<float, true> : (const void*)&state_xfer_kernel<bf16_t, true>;
  else fn = f32 ? (const void*)&state_xfer_kernel<float, false> : (const void*)&state_xfer_kernel<bf16_t, false>;
  L.tag("state", 0.0, 0.0);
  L.launch(fn, dim3(64, a.n), dim3(256), 0, &args);
}

// =============================================================================== lookahead inputs
template <typename T>
__global__ __launch_bounds__(256) void la_store_kernel(LaStoreArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.cv.n_streams * a.cv.nf * a.D) return;
  const int m = (int)(idx / a.D), c = (int)(idx % a.D);
  const int s = m / a.cv.nf, i = m % a.cv.nf;
  const int id = a.cv.ids[s];
  const int slot = (a.cv.pos[id] + a.pend[id] + i) % a.Rx;
  ((T*)a.x0)[((long)id * a.Rx + slot) * a.D + c] = ((const T*)a.in)[idx];
}
template <typename T>
__global__ __launch_bounds__(256) void la_gather_kernel(LaGatherArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.cv.n_streams * a.cv.nf * a.D) return;
  const int m = (int)(idx / a.D), c = (int)(idx % a.D);
  const int s = m / a.cv.nf, i = m % a.cv.nf;
  const int id = a.cv.ids[s];
  const int pos = a.cv.pos[id];
  const int slot = (pos + i) % a.Rx;
  a.x[idx] = ld<T>((const T*)a.x0 + ((long)id * a.Rx + slot) * a.D + c);
  if (i == 0 && c == 0) a.cv.cpos[s] = pos;
}
void launch_la_store(Launcher& L, const LaStoreArgs& a, int dtype) {
  LaStoreArgs args = a;
  const long total = (long)a.cv.n_streams * a.cv.nf * a.D;
  const void* fn = dtype == DT_F32 ? (const void*)&la_store_kernel<float> : (const void*)&la_store_kernel<bf16_t>;
  L.tag("lookahead_store", (double)total * 2 * (dtype == DT_F32 ? 4 : 2), 0.0);
  L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}
void launch_la_gather(Launcher& L, const LaGatherArgs& a, int dtype) {
  LaGatherArgs args = a;
  const long total = (long)a.cv.n_streams * a.cv.nf * a.D;
  const void* fn = dtype == DT_F32 ? (const void*)&la_gather_kernel<float> : (const void*)&la_gather_kernel<bf16_t>;
  L.tag("lookahead_gather", (double)total * (dtype == DT_F32 ? 4 : 2), 0.0);
  L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

// =============================================================================== init
// Kernels with dynamic LDS may use up to the CU's 160 KB.
void kernels_init() {
  static bool done = false;
  if (done) return;
  done = true;
  const int lds = 160 * 1024;
  std::vector<const void*> fns = {

      (const void*)&attn_kernel<float, 16, 2>, (const void*)&attn_kernel<float, 32, 2>, (const void*)&attn_kernel<float, 64, 2>,
      (const void*)&attn_kernel<bf16_t, 16, 2>, (const void*)&attn_kernel<bf16_t, 32, 2>, (const void*)&attn_kernel<bf16_t, 64, 2>,
      (const void*)&attn_kernel<float, 16, 4>, (const void*)&attn_kernel<float, 32, 4>, (const void*)&attn_kernel<float, 64, 4>,
      (const void*)&attn_kernel<bf16_t, 16, 4>, (const void*)&attn_kernel<bf16_t, 32, 4>, (const void*)&attn_kernel<bf16_t, 64, 4>,
  };
  for (int kch : {0, 1, 2, 3, 4, 6, 8})
    for (bool glu : {false, true}) {
      fns.push_back(gemv_pick_kch<float, float, 2>(kch, glu));
      fns.push_back(gemv_pick_kch<float, float, 8>(kch, glu));
      fns.push_back(gemv_pick_kch<bf16_t, float, 2>(kch, glu));
      fns.push_back(gemv_pick_kch<bf16_t, float, 8>(kch, glu));
      fns.push_back(gemv_pick_kch<bf16_t, bf16_t, 2>(kch, glu));
      fns.push_back(gemv_pick_kch<bf16_t, bf16_t, 8>(kch, glu));
    }
  for (int ek : {(int)EPI_STORE, (int)EPI_SILU, (int)EPI_SILU_KEEP, (int)EPI_RELU_FE, (int)EPI_RESID, (int)EPI_RESID_KEEP,
                 (int)EPI_F32, (int)EPI_QKV, (int)EPI_GLU, (int)EPI_PART, (int)EPI_RESID_LNS, EPI_SILU | EPI_LNC,
                 EPI_SILU_KEEP | EPI_LNC, EPI_QKV | EPI_LNC, EPI_GLU | EPI_LNC, (int)EPI_GLU_DW, EPI_GLU_DW | EPI_LNC}) {
    for (int t = 1; t <= 8; ++t) fns.push_back(kMfmaTiles[t].pick(ek));
  }
  for (const void* f : fns)
    if (f) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

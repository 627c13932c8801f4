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

void Launcher::launch(const void* fn, dim3 grid, dim3 block, size_t shmem, void* args) {
  if (err != hipSuccess) return;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return;
  void* kp[1] = {args};
  if (!graph) {
    if (prof) {
      hipEvent_t a = prof->get(), b = prof->get();
      if (a && b) err = hipEventRecord(a, stream);
      if (err == hipSuccess) err = hipLaunchKernel(fn, grid, block, kp, shmem, stream);
      if (err == hipSuccess && a && b) err = hipEventRecord(b, stream);
      if (err == hipSuccess && a && b) prof->pending.push_back({prof->name_id(tag_name), tag_bytes, tag_flops, a, b});
      tag_bytes = tag_flops = 0.0;
      return;
    }
    err = hipLaunchKernel(fn, grid, block, kp, shmem, stream);
    tag_bytes = tag_flops = 0.0;
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
  if (err == hipSuccess) last = last_node = node;
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
      bool before_start = e.cv.pos[e.cv.ids[s]] == 0 && j < e.fe_neg_rows;
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
        int slot = (e.cv.pos[id] + i) % e.R;
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
  int slot = (e.cv.pos[id] + i) % e.Rc;
  st<T>((T*)e.cring + ((long)id * e.Rc + slot) * e.D + c, g);
}

// GLU packing: packed column (c / 32) * 64 + c % 32 holds value channel c, +32 its gate.
__device__ __forceinline__ int glu_a_col(int c) { return (c >> 5) * 64 + (c & 31); }

// =============================================================================== small-M GEMM
// C[M][N] = A[M][K] W[N][K]^T for M up to a few rows per block. The block's MR rows of A sit
// in LDS as float (optionally LayerNorm'ed, and rounded to bf16 when the weights are bf16);
// each wave owns whole output columns and streams their weight rows once with 16-byte loads.
template <typename TW, int VEC> struct WLoad;
template <> struct WLoad<float, 4> {
  static __device__ __forceinline__ void get(const float* p, float* w) {
    float4 v = *(const float4*)p; w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
};
template <> struct WLoad<float, 1> {
  static __device__ __forceinline__ void get(const float* p, float* w) { w[0] = *p; }
};
template <> struct WLoad<bf16_t, 8> {
  static __device__ __forceinline__ void get(const bf16_t* p, float* w) {
    uint4 v = *(const uint4*)p;
    uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[2 * i] = __uint_as_float(u[i] << 16); w[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u); }
  }
};
template <> struct WLoad<bf16_t, 1> {
  static __device__ __forceinline__ void get(const bf16_t* p, float* w) { w[0] = bf2f(*p); }
};

template <typename TW, typename TA, int MR, int VEC>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs a) {
  const int units_per_block = a.upb;
  extern __shared__ float sA[];  // [MR][K]
  const int K = a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * MR;
  const int mr = min(MR, a.M - m0);
  for (int idx = tid; idx < MR * K; idx += 256) {
    int r = idx / K, k = idx - r * K;
    float v = 0.0f;
    if (r < mr) v = ld<TA>((const TA*)a.A + a.amap.off(m0 + r) + k);
    sA[idx] = v;
  }
  __syncthreads();
  // bf16 weights with a float32 A: the operand is rounded to bf16 (after LayerNorm, if any)
  constexpr bool round_bf16 = sizeof(TW) == 2 && sizeof(TA) == 4;
  if (round_bf16 && !a.ln_g) {
    for (int idx = tid; idx < MR * K; idx += 256) sA[idx] = bf2f(f2bf(sA[idx]));
    __syncthreads();
  }
  if (a.ln_g) {
    for (int r = wave; r < mr; r += 4) {
      float* row = sA + r * K;
      float s = 0.0f;
      for (int k = lane; k < K; k += 64) s += row[k];
      const float mean = wave_sum(s) / (float)K;
      float q = 0.0f;
      for (int k = lane; k < K; k += 64) { float d = row[k] - mean; q += d * d; }
      const float rstd = rsqrtf(wave_sum(q) / (float)K + 1e-5f);
      for (int k = lane; k < K; k += 64) {
        float y = (row[k] - mean) * rstd * a.ln_g[k] + a.ln_b[k];
        row[k] = round_bf16 ? bf2f(f2bf(y)) : y;
      }
    }
    __syncthreads();
  }
  const bool glu = a.epi.kind == EPI_GLU;
  const int units = glu ? a.N / 2 : a.N;
  const int u_end = min(units, (int)(blockIdx.x + 1) * units_per_block);
  const TW* W = (const TW*)a.W;
  for (int u = blockIdx.x * units_per_block + wave; u < u_end; u += 4) {
    const int ncol = glu ? 2 : 1;
    const int col0 = glu ? glu_a_col(u) : u;
    float acc[2][MR];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < MR; ++r) acc[c][r] = 0.0f;
    for (int c = 0; c < ncol; ++c) {
      const TW* wrow = W + (long)(col0 + 32 * c) * K;
#pragma unroll 4
      for (int k0 = lane * VEC; k0 < K; k0 += 64 * VEC) {
        float w[VEC];
        WLoad<TW, VEC>::get(wrow + k0, w);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          const float* ar = sA + r * K + k0;
          float s = 0.0f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) s += w[v] * ar[v];
          acc[c][r] += s;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < MR; ++r) acc[c][r] = wave_sum(acc[c][r]);
    if (lane < mr) {
      float va = 0.0f, vb = 0.0f;
#pragma unroll
      for (int r = 0; r < MR; ++r)
        if (r == lane) { va = acc[0][r]; vb = acc[1][r]; }
      if (glu) epi_glu<TW>(a.epi, m0 + lane, u, va, vb);
      else epi_one<TW>(a.epi, m0 + lane, u, va);
    }
  }
}

// =============================================================================== MFMA GEMM (bf16)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;

// Block tile BM x BN, k-step 32, 4 waves as WM x WN, each wave (BM/WM) x (BN/WN) made of
// 32x32 MFMA fragments. A and W tiles are staged through LDS (row stride padded to 40 bf16);
// the next k-tile is fetched into registers while the current one is multiplied.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a) {
  constexpr int BK = 32, LDK = BK + 8;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int A_PER_T = BM * 4 / 256, B_PER_T = BN * 4 / 256;
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int bm0 = blockIdx.y * BM, bn0 = blockIdx.x * BN;
  const int M = a.M, N = a.N, K = a.K;
  const bf16_t* A = (const bf16_t*)a.A;
  const bf16_t* W = (const bf16_t*)a.W;

  const bf16_t* aptr[A_PER_T];
  const bf16_t* bptr[B_PER_T];
  int aoff_s[A_PER_T], boff_s[B_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    int c = tid + i * 256, row = c >> 2, kc = (c & 3) * 8;
    int m = min(bm0 + row, M - 1);
    aptr[i] = A + a.amap.off(m) + kc;
    aoff_s[i] = row * LDK + kc;
  }
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    int c = tid + i * 256, row = c >> 2, kc = (c & 3) * 8;
    int n = min(bn0 + row, N - 1);
    bptr[i] = W + (long)n * K + kc;
    boff_s[i] = row * LDK + kc;
  }
  uint4 ra[A_PER_T], rb[B_PER_T];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) ra[i] = *(const uint4*)(aptr[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) rb[i] = *(const uint4*)(bptr[i] + kt * BK);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) *(uint4*)(As + aoff_s[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) *(uint4*)(Bs + boff_s[i]) = rb[i];
  };

  f32x16_v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = K / BK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_v af[FM], bfv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8_v*)(As + (wm * TM + i * 32 + (lane & 31)) * LDK + kk + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfv[j] = *(const bf16x8_v*)(Bs + (wn * TN + j * 32 + (lane & 31)) * LDK + kk + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < KT) {
      sstore();
      __syncthreads();
    }
  }

  // fragment element r of lane: row 8*(r/4) + 4*(lane/32) + r%4, column lane%32
  const bool glu = a.epi.kind == EPI_GLU;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = bm0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= M) continue;
      if (glu) {
        // wave tile holds 32-column pairs: fragment 2j = values, 2j+1 = gates
#pragma unroll
        for (int j = 0; j + 1 < FN; j += 2) {
          const int pcol = bn0 + wn * TN + j * 32;  // multiple of 64
          const int c = (pcol >> 6) * 32 + (lane & 31);
          if (pcol < N) epi_glu<bf16_t>(a.epi, row, c, acc[i][j][r], acc[i][j + 1][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = bn0 + wn * TN + j * 32 + (lane & 31);
          if (col < N) epi_one<bf16_t>(a.epi, row, col, acc[i][j][r]);
        }
      }
    }
  }
}

// =============================================================================== LayerNorm
template <typename TO>
__global__ __launch_bounds__(256) void ln_kernel(LnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.M) return;
  const float* x = a.x + (long)row * a.D;
  float s = 0.0f;
  for (int k = lane; k < a.D; k += 64) s += x[k];
  const float mean = wave_sum(s) / (float)a.D;
  float q = 0.0f;
  for (int k = lane; k < a.D; k += 64) { float d = x[k] - mean; q += d * d; }
  const float rstd = rsqrtf(wave_sum(q) / (float)a.D + 1e-5f);
  TO* y = (TO*)a.y + (long)row * a.D;
  for (int k = lane; k < a.D; k += 64) st<TO>(y + k, (x[k] - mean) * rstd * a.g[k] + a.b[k]);
}

// =============================================================================== dense dispatch
// Algorithmic HBM bytes of one dense product: the weights once, plus what its epilogue writes
// to per-stream state (K/V rows, depthwise input rows) or to the caller's output. Activations
// that stay on chip or in the last-level cache are not counted.
static double gemm_bytes(const GemmArgs& a, size_t wsz) {
  double b = (double)a.N * a.K * wsz;
  const double esz = (double)wsz;
  switch (a.epi.kind) {
    case EPI_QKV: b += (double)a.M * 2.0 * a.epi.D * esz; break;
    case EPI_GLU: b += (double)a.M * (a.N / 2) * esz; break;
    case EPI_F32: if (a.epi.ldo != a.epi.D || a.epi.omap) b += (double)a.M * a.N * 4.0; break;
    default: break;
  }
  return b;
}

template <typename TW, typename TA>
static void gemv_dispatch(Launcher& L, const GemmArgs& a) {
  const int units = a.epi.kind == EPI_GLU ? a.N / 2 : a.N;
  int upb = std::max(4, (units + 255) / 256);
  upb = (upb + 3) / 4 * 4;
  GemmArgs args = a;
  args.upb = upb;
  // MR rows per block; weights are re-streamed once per block row
  const int MR = a.M <= 2 ? 2 : (a.M <= 4 ? 4 : 8);
  const size_t shm = (size_t)MR * a.K * sizeof(float);
  constexpr int VW = sizeof(TW) == 4 ? 4 : 8;
  const bool vec = a.K % (64 * VW) == 0;
  const void* fn = nullptr;
#define GEMV_PICK(mr) \
  fn = vec ? (const void*)&gemv_kernel<TW, TA, mr, VW> : (const void*)&gemv_kernel<TW, TA, mr, 1>;
  if (MR == 2) { GEMV_PICK(2) } else if (MR == 4) { GEMV_PICK(4) } else { GEMV_PICK(8) }
#undef GEMV_PICK
  L.tag(sizeof(TW) == 4 ? "gemm_small_m_f32" : "gemm_small_m_bf16", gemm_bytes(a, sizeof(TW)), 2.0 * a.M * a.N * a.K);
  L.launch(fn, dim3((units + upb - 1) / upb, (a.M + MR - 1) / MR), dim3(256), shm, &args);
}

static void mfma_dispatch(Launcher& L, const GemmArgs& a) {
  const bool glu = a.epi.kind == EPI_GLU;
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  GemmArgs args = a;
  const void* fn;
  dim3 grid;
  L.tag("gemm_mfma_bf16", gemm_bytes(a, 2), 2.0 * a.M * a.N * a.K);
  // largest tile that still yields >= 256 workgroups; GLU needs 64-column wave tiles
  if (tiles(128, 128) >= 256) {
    fn = (const void*)&gemm_mfma_kernel<128, 128, 2, 2>;
    grid = dim3((a.N + 127) / 128, (a.M + 127) / 128);
  } else if (glu || tiles(64, 64) < 128) {
    if (tiles(128, 64) >= tiles(64, 128) * 3 / 4 && a.M >= 128) {
      fn = (const void*)&gemm_mfma_kernel<128, 64, 4, 1>;
      grid = dim3((a.N + 63) / 64, (a.M + 127) / 128);
    } else {
      fn = (const void*)&gemm_mfma_kernel<64, 128, 2, 2>;
      grid = dim3((a.N + 127) / 128, (a.M + 63) / 64);
    }
  } else {
    fn = (const void*)&gemm_mfma_kernel<64, 64, 2, 2>;
    grid = dim3((a.N + 63) / 64, (a.M + 63) / 64);
  }
  L.launch(fn, grid, dim3(256), 0, &args);
}

__global__ __launch_bounds__(256) void cvt_kernel(CvtArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.M * a.K) return;
  const int m = (int)(idx / a.K), k = (int)(idx % a.K);
  ((bf16_t*)a.y)[idx] = f2bf(a.x[a.amap.off(m) + k]);
}

void launch_gemm(Launcher& L, const GemmArgs& a, int dtype, int path) {
  if (dtype == DT_F32) {
    gemv_dispatch<float, float>(L, a);
    return;
  }
  const bool small = path == 1 || (path == 0 && a.M <= 8);
  if (small) {
    if (a.a_f32) gemv_dispatch<bf16_t, float>(L, a);
    else gemv_dispatch<bf16_t, bf16_t>(L, a);
    return;
  }
  GemmArgs g = a;
  if (a.a_f32) {
    // materialise the bf16 operand first: LayerNorm rows, or a rounded (gathered) copy
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
    g.A = a.a_scratch;
    g.amap = RowMap{INT_MAX, 0, a.K};
    g.a_f32 = 0;
    g.ln_g = g.ln_b = nullptr;
  }
  mfma_dispatch(L, g);
}

void launch_ln(Launcher& L, const LnArgs& a, int dtype) {
  LnArgs args = a;
  const void* fn = (a.out_f32 || dtype == DT_F32) ? (const void*)&ln_kernel<float> : (const void*)&ln_kernel<bf16_t>;
  L.tag("layernorm", 0.0, 0.0);
  L.launch(fn, dim3((a.M + 3) / 4), dim3(256), 0, &args);
}

// =============================================================================== attention
// One wave per (call stream, head). Keys are the ring rows of positions
// [max(0, pos0 - Lc), pos0 + nf - 1]; the rows of this call were written by the QKV epilogue.
// score(i, j) = ((q_i + u) . k_j + (q_i + v) . P[p_i - q_j]) * scale on visible keys,
// with the position term taken from a per-wave table bd[i][rel] = (q_i + v) . P[rel].
size_t attention_shmem(int nf, int nk_max, int nrel, int hd) {
  return (size_t)4 * sizeof(float) * (2 * nf * hd + nf * nrel + nf * nk_max);
}

__device__ __forceinline__ bool att_visible(const AttnArgs& a, int p, int q) {
  if (q < 0) return false;
  if (a.lookahead) return q >= p - a.Lc && q <= p + a.right;
  const int cs = p - p % a.chunk;
  return q >= cs - a.Lc && q <= cs + a.chunk - 1;
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nf = a.cv.nf, nrel = a.nrel, nkmax = a.Lc + nf;
  const int per_wave = 2 * nf * HD + nf * nrel + nf * nkmax;
  float* qu = sm + wave * per_wave;
  float* qv = qu + nf * HD;
  float* bd = qv + nf * HD;
  float* sc = bd + nf * nrel;
  const int pair = blockIdx.x * 4 + wave;
  const bool active = pair < a.cv.n_streams * a.H;
  const int s = active ? pair / a.H : 0, h = active ? pair % a.H : 0;
  const int id = a.cv.ids[s];
  const int pos0 = a.cv.pos[id];
  const int q_lo = max(0, pos0 - a.Lc), q_hi = pos0 + nf - 1, nk = q_hi - q_lo + 1;

  if (active) {
    for (int idx = lane; idx < nf * HD; idx += 64) {
      const int i = idx / HD, d = idx - i * HD;
      const float q = a.q[(long)(s * nf + i) * a.D + h * HD + d];
      qu[idx] = q + a.pos_u[h * HD + d];
      qv[idx] = q + a.pos_v[h * HD + d];
    }
  }
  __syncthreads();
  if (active) {
    // position term table
    for (int r = lane; r < nrel; r += 64) {
      const float* prow = a.posproj + ((long)h * nrel + r) * HD;
      float pr[HD];
#pragma unroll
      for (int d = 0; d < HD; d += 4) {
        float4 v = *(const float4*)(prow + d);
        pr[d] = v.x; pr[d + 1] = v.y; pr[d + 2] = v.z; pr[d + 3] = v.w;
      }
      for (int i = 0; i < nf; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc += qv[i * HD + d] * pr[d];
        bd[i * nrel + r] = acc;
      }
    }
  }
  __syncthreads();
  if (active) {
    const T* kbase = (const T*)a.kring + ((long)id * a.H + h) * a.R * HD;
    for (int j = lane; j < nk; j += 64) {
      const int qk = q_lo + j;
      const T* krow = kbase + (long)(qk % a.R) * HD;
      float kr[HD];
#pragma unroll
      for (int d = 0; d < HD; ++d) kr[d] = ld<T>(krow + d);
      for (int i = 0; i < nf; ++i) {
        const int p = pos0 + i;
        float sv = -INFINITY;
        if (att_visible(a, p, qk)) {
          float acc = 0.0f;
#pragma unroll
          for (int d = 0; d < HD; ++d) acc += qu[i * HD + d] * kr[d];
          sv = (acc + bd[i * nrel + (p - qk - a.rel_lo)]) * a.scale;
        }
        sc[i * nkmax + j] = sv;
      }
    }
  }
  __syncthreads();
  if (active) {
    for (int i = 0; i < nf; ++i) {
      float mx = -INFINITY;
      for (int j = lane; j < nk; j += 64) mx = fmaxf(mx, sc[i * nkmax + j]);
      mx = wave_max(mx);
      float sum = 0.0f;
      for (int j = lane; j < nk; j += 64) {
        const float e = __expf(sc[i * nkmax + j] - mx);
        sc[i * nkmax + j] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      const float inv = 1.0f / sum;
      for (int j = lane; j < nk; j += 64) sc[i * nkmax + j] *= inv;
    }
  }
  __syncthreads();
  if (active && lane < HD) {
    const T* vbase = (const T*)a.vring + ((long)id * a.H + h) * a.R * HD;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int j = 0; j < nk; ++j) {
      const float vv = ld<T>(vbase + (long)((q_lo + j) % a.R) * HD + lane);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < nf) acc[i] += sc[i * nkmax + j] * vv;
    }
    for (int i = 0; i < nf; ++i) st<T>((T*)a.o + (long)(s * nf + i) * a.D + h * HD + lane, acc[i]);
  }
}

void launch_attention(Launcher& L, const AttnArgs& a, int dtype, int hd) {
  AttnArgs args = a;
  const int pairs = a.cv.n_streams * a.H;
  const size_t shm = attention_shmem(a.cv.nf, a.Lc + a.cv.nf, a.nrel, hd);
  const void* fn = nullptr;
#define ATT_PICK(HDV)                                                                   \
  fn = dtype == DT_F32 ? (const void*)&attn_kernel<float, HDV> : (const void*)&attn_kernel<bf16_t, HDV>;
  if (hd == 16) { ATT_PICK(16) } else if (hd == 32) { ATT_PICK(32) } else { ATT_PICK(64) }
#undef ATT_PICK
  L.tag_name = "attention";  // the caller tags bytes and flops (it knows each stream's fill)
  L.launch(fn, dim3((pairs + 3) / 4), dim3(256), shm, &args);
}

// =============================================================================== depthwise conv
template <typename T>
__global__ __launch_bounds__(256) void dw_kernel(DwArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.cv.n_streams * a.cv.nf * a.D;
  if (idx >= total) return;
  const int m = (int)(idx / a.D), c = (int)(idx % a.D);
  const int s = m / a.cv.nf, i = m % a.cv.nf;
  const int id = a.cv.ids[s];
  const int p = a.cv.pos[id] + i;
  const T* ring = (const T*)a.cring + (long)id * a.Rc * a.D;
  float acc = a.b[c];
  for (int k = 0; k < a.K; ++k) {
    const int q = p - (a.K - 1) + k;
    if (q >= 0) acc += a.w[k * a.D + c] * ld<T>(ring + (long)(q % a.Rc) * a.D + c);
  }
  st<T>((T*)a.e + (long)m * a.D + c, silu_f(acc));
}

void launch_dwconv(Launcher& L, const DwArgs& a, int dtype) {
  DwArgs args = a;
  const long total = (long)a.cv.n_streams * a.cv.nf * a.D;
  const void* fn = dtype == DT_F32 ? (const void*)&dw_kernel<float> : (const void*)&dw_kernel<bf16_t>;
  L.tag_name = "dwconv";  // the caller tags bytes and flops
  L.launch(fn, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, &args);
}

// =============================================================================== input, FE window
template <typename T>
__global__ __launch_bounds__(256) void input_kernel(InputArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx < (long)a.M * a.D) a.x[idx] = ld<T>((const T*)a.in + idx);
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
  const bool fresh = a.cv.pos[id] == 0;
  const int nt = a.mel_tail, nn = a.mel_new, rows = nt + nn;
  T* tail = (T*)a.tail + (long)id * nt * a.bins + b;
  const T* mel = (const T*)a.mel + (long)s * nn * a.bins + b;
  T* win = (T*)a.win + (long)s * rows * a.bins + b;
  for (int r = 0; r < nt; ++r) win[(long)r * a.bins] = fresh ? T(0) : tail[(long)r * a.bins];
  for (int r = 0; r < nn; ++r) win[(long)(nt + r) * a.bins] = mel[(long)r * a.bins];
  for (int r = 0; r < nt; ++r) tail[(long)r * a.bins] = win[(long)(rows - nt + r) * a.bins];
}
void launch_fe_window(Launcher& L, const FeWindowArgs& a, int dtype) {
  FeWindowArgs args = a;
  const int total = a.cv.n_streams * a.bins;
  const void* fn = dtype == DT_F32 ? (const void*)&fe_window_kernel<float> : (const void*)&fe_window_kernel<bf16_t>;
  L.tag("fe_window", (double)a.cv.n_streams * (a.mel_new + 2 * a.mel_tail) * a.bins * (dtype == DT_F32 ? 4 : 2), 0.0);
  L.launch(fn, dim3((total + 255) / 256), dim3(256), 0, &args);
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

// Canonical blob of one stream (floats): K [L][Lc][D], V [L][Lc][D], conv [L][Kc][D],
// tail [tail_rows][bins], x0 [nla][D].
template <typename T, bool IMPORT>
__global__ __launch_bounds__(256) void state_xfer_kernel(StateArgs a) {
  const int s = blockIdx.y;
  const int id = a.ids[s];
  const int pos = a.hpos[s];
  const int pend = a.hpend ? a.hpend[s] : 0;
  float* blob = a.blob + (long)s * a.state_floats;
  const long kvn = (long)a.L * a.Lc * a.D, cvn = (long)a.L * a.Kc * a.D;
  const long tln = (long)a.tail_rows * a.bins, x0n = (long)a.nla * a.D;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < a.state_floats; e += (long)gridDim.x * 256) {
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
      if (valid) dst = (T*)a.cring + ((l * a.S + id) * a.Rc + q % a.Rc) * a.D + c;
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
  const int slot = (a.cv.pos[id] + i) % a.Rx;
  a.x[idx] = ld<T>((const T*)a.x0 + ((long)id * a.Rx + slot) * a.D + c);
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
  const void* fns[] = {
      (const void*)&gemv_kernel<float, float, 2, 4>, (const void*)&gemv_kernel<float, float, 4, 4>,
      (const void*)&gemv_kernel<float, float, 8, 4>, (const void*)&gemv_kernel<float, float, 2, 1>,
      (const void*)&gemv_kernel<float, float, 4, 1>, (const void*)&gemv_kernel<float, float, 8, 1>,
      (const void*)&gemv_kernel<bf16_t, float, 2, 8>, (const void*)&gemv_kernel<bf16_t, float, 4, 8>,
      (const void*)&gemv_kernel<bf16_t, float, 8, 8>, (const void*)&gemv_kernel<bf16_t, float, 2, 1>,
      (const void*)&gemv_kernel<bf16_t, float, 4, 1>, (const void*)&gemv_kernel<bf16_t, float, 8, 1>,
      (const void*)&gemv_kernel<bf16_t, bf16_t, 2, 8>, (const void*)&gemv_kernel<bf16_t, bf16_t, 4, 8>,
      (const void*)&gemv_kernel<bf16_t, bf16_t, 8, 8>, (const void*)&gemv_kernel<bf16_t, bf16_t, 2, 1>,
      (const void*)&gemv_kernel<bf16_t, bf16_t, 4, 1>, (const void*)&gemv_kernel<bf16_t, bf16_t, 8, 1>,
      (const void*)&attn_kernel<float, 16>, (const void*)&attn_kernel<float, 32>, (const void*)&attn_kernel<float, 64>,
      (const void*)&attn_kernel<bf16_t, 16>, (const void*)&attn_kernel<bf16_t, 32>, (const void*)&attn_kernel<bf16_t, 64>,
  };
  for (const void* f : fns) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

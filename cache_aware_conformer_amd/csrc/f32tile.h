// One 64 x 64 float32 output tile of a row-gathered product on v_mfma_f32_32x32x2f32, shared by
// the greedy and beam decoders' dense kernels (prediction network, projection, joint).
#pragma once

#include <hip/hip_runtime.h>

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int F32T_BK = 64;                    // k per step
constexpr int F32T_S = 68;                     // LDS row stride (floats): 64 k + 4 pad
constexpr int F32T_DEPTH = 3;                  // k-steps whose operands are loaded ahead
// two k-step buffers of A [64][68] and W [64][68]; afterwards the output tile Ct[64][65]
constexpr size_t F32T_LDS = (size_t)2 * 2 * 64 * F32T_S * sizeof(float);  // 68 KB

// A 256-thread block computes rows [row0, row0 + 64) x columns [col0, col0 + 64) of A W^T with
// W stored [N][ldw] (row n holds output column n's K weights, k contiguous; K a multiple of 64).
// Thread t loads the 16 A values k = (t % 4) * 16 .. + 15 of tile row t / 4 (plus multiples
// of 64) through src(k), which returns 4 consecutive values of that thread's own row, and the
// same 16 k of W row col0 + t / 4. Both tiles sit in LDS k-contiguous per row. Each of the
// four waves owns a 32 x 32 quarter; within a k-step of 64 the MFMA j of a wave takes k = j
// on its lanes 0-31 and k = 32 + j on lanes 32-63 (the two k rows of the 32x32x2 operands), so
// a lane's operands for the whole step are 32 consecutive floats of one LDS row: eight 16-byte
// reads per operand instead of one 4-byte read per MFMA.
// k0 offsets the contraction (the block covers k0 .. k0 + K - 1 of both operands).
// On return the tile is in Ct[64][65] (LDS, float (*)[65] over lds) and the block is synchronised.
template <class Src>
__device__ __forceinline__ void f32_tile(const Src& src, const float* __restrict__ W, int ldw, int K, int col0,
                                         float* lds, int k0 = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int lr = tid >> 2, lk = (tid & 3) * 16;         // loader: tile row / W row lr, k lk .. lk+15
  const float* wrow = W + (long)(col0 + lr) * ldw + k0 + lk;
  const int KT = K / F32T_BK;
  // operands of the next F32T_DEPTH k-steps in flight in registers (set s holds step kt with
  // kt % F32T_DEPTH == s), so each load has that many steps of MFMA work to arrive behind
  f32x4_t ra[F32T_DEPTH][4], rb[F32T_DEPTH][4];
#pragma unroll
  for (int s = 0; s < F32T_DEPTH; ++s)
    if (s < KT) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra[s][q] = src(k0 + s * F32T_BK + lk + 4 * q);
        rb[s][q] = *(const f32x4_t*)(wrow + s * F32T_BK + 4 * q);
      }
    }
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  const int ar = wm * 32 + (lane & 31), bc = wn * 32 + (lane & 31), kh = (lane >> 5) * 32;
  for (int kt0 = 0; kt0 < KT; kt0 += F32T_DEPTH) {
#pragma unroll
    for (int s = 0; s < F32T_DEPTH; ++s) {
      const int kt = kt0 + s;
      if (kt >= KT) break;
      float* As = lds + (kt & 1) * 2 * 64 * F32T_S;
      float* Bs = As + 64 * F32T_S;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *(f32x4_t*)&As[lr * F32T_S + lk + 4 * q] = ra[s][q];
        *(f32x4_t*)&Bs[lr * F32T_S + lk + 4 * q] = rb[s][q];
      }
      __syncthreads();
      if (kt + F32T_DEPTH < KT) {
        const int k1 = (kt + F32T_DEPTH) * F32T_BK;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ra[s][q] = src(k0 + k1 + lk + 4 * q);
          rb[s][q] = *(const f32x4_t*)(wrow + k1 + 4 * q);
        }
      }
      f32x4_t fa[8], fb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        fa[q] = *(const f32x4_t*)&As[ar * F32T_S + kh + 4 * q];
        fb[q] = *(const f32x4_t*)&Bs[bc * F32T_S + kh + 4 * q];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].x, fb[q].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].y, fb[q].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].z, fb[q].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].w, fb[q].w, acc, 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the k-step buffers
  float (*Ct)[65] = (float (*)[65])lds;
  // accumulator element r of a lane: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) Ct[wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][wn * 32 + (lane & 31)] = acc[r];
  __syncthreads();
}

// One wave's 32 x 32 output tile over k-steps [ks0, ks1) of 64, both operands loaded straight
// from memory into the MFMA operand registers (no LDS). Lane l holds tile row / W row l % 32;
// within a k-step its 32 consecutive k (0-31 on lanes 0-31, 32-63 on lanes 32-63) feed the 32
// MFMAs of the step, k = j (lanes 0-31) and 32 + j (lanes 32-63) in MFMA j. src(k) returns 4
// consecutive A values of the lane's row; wrow points at the lane's W row (k contiguous). The
// next step's operands are loaded while this step's MFMAs run.
template <class Src>
__device__ __forceinline__ f32x16_t f32_wave_tile(const Src& src, const float* __restrict__ wrow, int ks0, int ks1) {
  const int kh = ((threadIdx.x & 63) >> 5) * 32;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  if (ks0 >= ks1) return acc;
  f32x4_t a0[8], b0[8], a1[8], b1[8];
  auto load = [&](f32x4_t (&ar)[8], f32x4_t (&br)[8], int ks) {
    const int k = ks * 64 + kh;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ar[q] = src(k + 4 * q);
      br[q] = *(const f32x4_t*)(wrow + k + 4 * q);
    }
  };
  auto mma = [&](const f32x4_t (&ar)[8], const f32x4_t (&br)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[q].x, br[q].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[q].y, br[q].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[q].z, br[q].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[q].w, br[q].w, acc, 0, 0, 0);
    }
  };
  load(a0, b0, ks0);
  for (int ks = ks0; ks < ks1; ks += 2) {
    if (ks + 1 < ks1) load(a1, b1, ks + 1);
    mma(a0, b0);
    if (ks + 1 >= ks1) break;
    if (ks + 2 < ks1) load(a0, b0, ks + 2);
    mma(a1, b1);
  }
  return acc;
}

// NW waves share one 32 x 32 output tile, each over its share of the k-steps; their partial
// tiles are added in LDS (wave order, so the sum does not depend on timing) into Ct[32][33].
// red must hold NW * 32 * 33 floats; the block has 64 NW threads. On return the block is
// synchronised.
template <int NW, class Src>
__device__ __forceinline__ void f32_tile32(const Src& src, const float* __restrict__ wrow, int K, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KT = K / 64;
  const f32x16_t acc = f32_wave_tile(src, wrow, wave * KT / NW, (wave + 1) * KT / NW);
  float (*P)[32][33] = (float (*)[32][33])red;
  // accumulator element r of a lane: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) P[wave][8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = acc[r];
  __syncthreads();
  float (*Ct)[33] = (float (*)[33])red;   // over P[0]: each thread reads its sums first
  constexpr int PER = 1024 / (64 * NW);
  float v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int idx = tid + 64 * NW * q, r = idx >> 5, c = idx & 31;
    float x = P[0][r][c];
#pragma unroll
    for (int w = 1; w < NW; ++w) x += P[w][r][c];
    v[q] = x;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int idx = tid + 64 * NW * q;
    Ct[idx >> 5][idx & 31] = v[q];
  }
  __syncthreads();
}

// One 64 x 64 float32 output tile of a row-gathered product on v_mfma_f32_32x32x2f32, shared by
// the greedy and beam decoders' dense kernels (prediction network, projection, joint).
#pragma once

#include <hip/hip_runtime.h>

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int F32T_BK = 64;                    // k per step
constexpr int F32T_AS = 65, F32T_BS = 68;      // LDS row strides (A k-major, W row-major)
// two k-tile buffers; after the k-loop the first 64 x 65 floats hold the output tile
constexpr size_t F32T_LDS = (size_t)2 * F32T_BK * (F32T_AS + F32T_BS) * sizeof(float);  // 68 KB

// A 256-thread block computes rows [row0, row0 + 64) x columns [col0, col0 + 64) of A W, W
// [K][N] row-major (K a multiple of 64, col0 + 64 <= N). Thread t loads the 16 A values
// k = (t % 4) * 16 .. + 15 of tile row t / 4 (plus multiples of 64) through src(k), which
// returns 4 consecutive values of that thread's own row. Four waves each own a 32 x 32 quarter.
// On return the tile is in Ct[64][65] (LDS, float (*)[65] over lds) and the block is synchronised.
template <class Src>
__device__ __forceinline__ void f32_tile(const Src& src, const float* __restrict__ W, int N, int K, int col0,
                                         float* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int lr = tid >> 2, lk = (tid & 3) * 16;         // A loader: row lr, k lk .. lk+15
  const int bk = tid >> 2, bn = (tid & 3) * 16;         // W loader: k bk, columns bn .. bn+15
  const int KT = K / F32T_BK;
  f32x4_t ra[4], rb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ra[q] = src(lk + 4 * q);
    rb[q] = *(const f32x4_t*)(W + (long)bk * N + col0 + bn + 4 * q);
  }
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  for (int kt = 0; kt < KT; ++kt) {
    float* As = lds + (kt & 1) * F32T_BK * (F32T_AS + F32T_BS);
    float* Bs = As + F32T_BK * F32T_AS;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      As[(lk + 4 * q + 0) * F32T_AS + lr] = ra[q].x;
      As[(lk + 4 * q + 1) * F32T_AS + lr] = ra[q].y;
      As[(lk + 4 * q + 2) * F32T_AS + lr] = ra[q].z;
      As[(lk + 4 * q + 3) * F32T_AS + lr] = ra[q].w;
      *(f32x4_t*)&Bs[bk * F32T_BS + bn + 4 * q] = rb[q];
    }
    __syncthreads();
    if (kt + 1 < KT) {
      const int k1 = (kt + 1) * F32T_BK;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra[q] = src(k1 + lk + 4 * q);
        rb[q] = *(const f32x4_t*)(W + (long)(k1 + bk) * N + col0 + bn + 4 * q);
      }
    }
#pragma unroll
    for (int kk = 0; kk < F32T_BK; kk += 2) {
      const float av = As[(kk + (lane >> 5)) * F32T_AS + wm * 32 + (lane & 31)];
      const float bv = Bs[(kk + (lane >> 5)) * F32T_BS + wn * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the k-tile buffers
  float (*Ct)[65] = (float (*)[65])lds;
  // accumulator element r of a lane: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) Ct[wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][wn * 32 + (lane & 31)] = acc[r];
  __syncthreads();
}

// Plain LDS-tiled FMA GEMM C = A B^T (fp32 accumulate), for the fp32 path.
// 64x64 output tile per 256-thread block, 4x4 outputs per thread, K step 16.
#include "kernels.hpp"

namespace lb {

template <typename T>
__global__ __launch_bounds__(256) void k_gemm_simt(const T* __restrict__ A, const T* __restrict__ B,
                                                   float* __restrict__ C, int M, int N, int K) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    // 64 rows x 16 k of A and of B: 1024 values each, 4 per thread
    for (int i = threadIdx.x; i < 1024; i += 256) {
      int r = i >> 4, c = i & 15;
      int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      As[c][r] = (gm < M && gk < K) ? Elt<T>::load(A, (size_t)gm * K + gk) : 0.f;
      Bs[c][r] = (gn < N && gk < K) ? Elt<T>::load(B, (size_t)gn * K + gk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int gn = n0 + tx * 4 + j;
      if (gn < N) C[(size_t)gm * N + gn] = acc[i][j];
    }
  }
}

template <typename T>
void launch_gemm_simt(const T* A, const T* B, float* C, int M, int N, int K, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(k_gemm_simt<T>, grid, dim3(256), 0, s, A, B, C, M, N, K);
}

template void launch_gemm_simt<float>(const float*, const float*, float*, int, int, int, hipStream_t);
template void launch_gemm_simt<bf16_t>(const bf16_t*, const bf16_t*, float*, int, int, int, hipStream_t);

}  // namespace lb

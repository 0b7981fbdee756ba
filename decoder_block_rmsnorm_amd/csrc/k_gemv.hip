// Decode-time projections (one token per sequence, M = batch <= 64): every
// weight byte is read exactly once per step, so these kernels are HBM-bound.
//
// k_gemv_bf16: split-K skinny GEMM on v_mfma_f32_16x16x32_bf16.  A block owns
//   NW*64 output columns and one K slice; each wavefront streams its 16*NW
//   weight rows straight from HBM into MFMA B-operand registers with 128-bit
//   loads (8 per lane in flight per 256-wide K chunk, prefetched one chunk
//   ahead), while the activations of the chunk sit in LDS for all four
//   wavefronts.  fp32 partials [ks][M][N] go to a reduce-and-finish kernel,
//   or, unsplit (ks = 1), the W1/W3 product is finished in place: RMSNorm row
//   scale and silu(gate) * up (EPI_SWIGLU).
//
// k_gemv_q4: 4-bit group-affine weights (group 64 along the input dim, the MLX
//   quantization config of "模型配置"): W = s * code + b.  Per 8-code word,
//   one shift and four three-input bit operations turn nibble pairs into fp16 pairs
//   (1024 + code or 1024 + 16 code, exact), v_dot2_f32_f16 multiplies them with
//   pre-scaled fp16 activations; the 1024 offset and the bias are removed per
//   32-code chunk with precomputed activation sums:
//       sum_k W x = sum_chunks  s * (A - 1024 * Xh) + b * X.
#include "kernels.hpp"

namespace lb {

__device__ inline bf16x8 v_as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

namespace gv {
constexpr int KC = 256;         // K chunk per pipeline step
constexpr int XST = KC + 8;     // LDS row stride (bf16)
}  // namespace gv

// Pipeline per block: the weight rows of chunk c+2 and the activations of chunk
// c+1 are in flight while chunk c is multiplied.  Program order is chosen for
// the in-order vmcnt counter: the activations of c+1 are requested before the
// weights of c+2, so waiting for them never waits for the newer weights.
// Every load of the steady-state loop is unconditional (out-of-range addresses
// are clamped, and the values they bring are multiplied by zeros), so the
// compiler can count outstanding loads exactly and never has to drain them.
//
// W is in the tiled layout (TILED: each wavefront load instruction reads one
// contiguous kilobyte; the padding of the last chunk is zero) or row-major
// [N][K].  K slice ksi of ks covers the 256-column chunks
// [ksi * nchk / ks, (ksi + 1) * nchk / ks).  K is a multiple of 8.
template <int NW, int MT, bool TILED, bool SS, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemv_bf16(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, float* __restrict__ part, int M, int N, int K, int ks,
    float* __restrict__ ss_out, GemvSwiglu e) {
  using namespace gv;
  constexpr int ROWS = MT * 16;
  constexpr int XL = ROWS * (KC / 8) / 256;   // 16-byte activation pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][ROWS * XST];
  // SS: the first column-block of each K slice also sums x^2 of the rows it
  // stages (the RMSNorm statistic of the input, reduced over slices by its
  // consumer); each thread accumulates the squares of its own activation pieces
  const bool do_ss = SS && blockIdx.x == 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, hg = lane >> 4;
  float ssp[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) ssp[i] = 0.f;
  const int ksi = blockIdx.y;
  const int nchk = (K + KC - 1) / KC;
  const int c0 = ksi * nchk / ks, c1 = (ksi + 1) * nchk / ks;
  const int kb = c0 * KC;
  const int nch = c1 - c0;
  const int nrow0 = blockIdx.x * (64 * NW) + wave * (16 * NW);

  f32x4 acc[MT][NW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[i][j] = (f32x4){};

  uint4 w0[NW][8], w1[NW][8], xr[XL];
  auto wload = [&](int c, uint4(&w)[NW][8]) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if constexpr (TILED) {
        const bf16_t* t = W + ((size_t)(c0 + c) * (N >> 4) + (nrow0 >> 4) + j) * kTileElems + lane * 8;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) w[j][kc] = ld16(t + 512 * kc);
      } else {
        const bf16_t* wrow = W + (size_t)(nrow0 + j * 16 + l16) * K;
        const int k0 = kb + c * KC + 8 * hg;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) w[j][kc] = ld16(wrow + min(k0 + 32 * kc, K - 8));
      }
    }
  };
  // piece p of a chunk: row p / 32, 8 columns at 8 * (p % 32); rows >= M
  // repeat row M - 1 (their products are never stored), columns >= K are zero
  auto xload = [&](int c) {
    const int k0 = kb + c * KC;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int p = tid + 256 * i, r = min(p >> 5, M - 1), col = k0 + (p & 31) * 8;
      const uint32_t keep = col < K ? 0xffffffffu : 0u;
      uint4 v = ld16(X + (size_t)r * K + min(col, K - 8));
      v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
      xr[i] = v;
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int p = tid + 256 * i, r = p >> 5, col = (p & 31) * 8;
      st16(&xs[buf][r * XST + col], xr[i]);
      if (do_ss) {
        const bf16x8 v = v_as_bf16x8(xr[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = (float)v[e];
          ssp[i] += f * f;
        }
      }
    }
  };
  auto compute = [&](int buf, const uint4(&w)[NW][8]) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 xa = v_as_bf16x8(ld16(&xs[buf][(mt * 16 + l16) * XST + 32 * kc + 8 * hg]));
#pragma unroll
        for (int j = 0; j < NW; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, v_as_bf16x8(w[j][kc]), acc[mt][j], 0, 0, 0);
      }
    }
  };

  // buffer reuse: a chunk's activations are stored into the LDS buffer read
  // two computes earlier, with a barrier in between
  // EPI_SWIGLU: 1/rms of the input rows, from the producer's partial sums of
  // squares (four threads per row, each over every fourth partial, combined in
  // a fixed order), requested once the first chunks are on their way
  __shared__ float s_r[ROWS];
  auto row_scale = [&]() {
    const int m = tid >> 2, qq = tid & 3;
    float t = 0.f;
    if (m < M) {
      if (e.stat.inv) {
        if (qq == 0) t = e.stat.inv[m];
      } else {
        for (int b = qq; b < e.stat.nb; b += 4) t += e.stat.ss[(size_t)b * e.stat.M + m];
      }
    }
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    if (m < ROWS && qq == 0) s_r[m] = e.stat.inv ? t : 1.0f / sqrtf(t / (float)e.stat.n + e.stat.eps);
  };

  if (nch >= 2) {
    xload(0);
    wload(0, w0);
    wload(1, w1);
    if constexpr (EPI == EPI_SWIGLU) row_scale();
    xstore(0);
    __syncthreads();
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      xload(c + 1);
      compute(0, w0);
      wload(c + 2, w0);
      xstore(1);
      __syncthreads();
      xload(c + 2);
      compute(1, w1);
      wload(c + 3, w1);
      xstore(0);
      __syncthreads();
    }
    // two or three chunks left: w0 holds chunk c, w1 chunk c + 1
    xload(c + 1);
    compute(0, w0);
    if (c + 2 < nch) wload(c + 2, w0);
    xstore(1);
    __syncthreads();
    if (c + 2 < nch) {
      xload(c + 2);
      compute(1, w1);
      xstore(0);
      __syncthreads();
      compute(0, w0);
    } else {
      compute(1, w1);
    }
  } else if (nch == 1) {
    xload(0);
    wload(0, w0);
    if constexpr (EPI == EPI_SWIGLU) row_scale();
    xstore(0);
    __syncthreads();
    compute(0, w0);
  }
  if (do_ss) {
    // the 32 pieces of row (tid + 256 i) / 32 sit in 32 adjacent lanes
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      float t = ssp[i];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) t += __shfl_xor(t, o, 32);
      const int r = (tid + 256 * i) >> 5;
      if ((tid & 31) == 0 && r < M) ss_out[(size_t)ksi * M + r] = t;
    }
  }
  // lane: C[m = 16*mt + 4*hg + i][n = nrow0 + 16*j + l16]
  if constexpr (EPI == EPI_F32) {
    float* pp = part + (size_t)ksi * M * N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * hg + i;
        if (m < M) {
#pragma unroll
          for (int j = 0; j < NW; ++j) pp[(size_t)m * N + nrow0 + 16 * j + l16] = acc[mt][j][i];
        }
      }
    }
  } else {
    // the block's 64*NW rows hold whole (w1 block, w3 block) pairs of ib rows:
    // stage them as [row][m] (padded) in the activation buffers' LDS
    constexpr int LS = ROWS + 1;
    float* stage = reinterpret_cast<float*>(&xs[0][0]);
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(16 * NW * wave + 16 * j + l16) * LS + mt * 16 + 4 * hg + i] = acc[mt][j][i];
    __syncthreads();
    constexpr int OUT = 32 * NW;  // outputs per row from this block
    const int F = N >> 1, ib = e.ib, j0 = blockIdx.x * OUT, r0 = blockIdx.x * 64 * NW;
    for (int p = tid; p < OUT * M; p += 256) {
      const int m = p / OUT, jg = j0 + p % OUT;
      const int ra = (jg / ib) * 2 * ib + jg % ib - r0;
      const float r = s_r[m];
      const float a = stage[ra * LS + m] * r, b = stage[(ra + ib) * LS + m] * r;
      Elt<bf16_t>::store(e.g_out, (size_t)m * F + jg, silu_f(a) * b);
    }
  }
}

int gemv_cols(int M, int N) { return (M > 16 && (N % 128) == 0) ? 128 : 64; }

template <int NW, bool TILED, bool SS, int EPI>
static void gemv_mt(const bf16_t* X, const bf16_t* W, float* partial, int M, int N, int K, int ks, float* ss_out,
                    const GemvSwiglu& e, hipStream_t s) {
  dim3 grid(N / (64 * NW), ks);
  plan_log("gemv M %d N %d K %d: %d columns per block, split-K %d (%d blocks), %s weights%s%s", M, N, K, 64 * NW, ks,
           (int)(grid.x * grid.y), TILED ? "tiled" : "row-strip", SS ? ", x statistic" : "",
           EPI == EPI_SWIGLU ? ", SwiGLU in the kernel" : "");
  if (M <= 16)
    hipLaunchKernelGGL((k_gemv_bf16<NW, 1, TILED, SS, EPI>), grid, dim3(256), 0, s, X, W, partial, M, N, K, ks,
                       ss_out, e);
  else if (M <= 32)
    hipLaunchKernelGGL((k_gemv_bf16<NW, 2, TILED, SS, EPI>), grid, dim3(256), 0, s, X, W, partial, M, N, K, ks,
                       ss_out, e);
  else
    hipLaunchKernelGGL((k_gemv_bf16<NW, 4, TILED, SS, EPI>), grid, dim3(256), 0, s, X, W, partial, M, N, K, ks,
                       ss_out, e);
}

template <bool TILED, bool SS>
static void gemv_nw(const bf16_t* X, const bf16_t* W, float* partial, int M, int N, int K, int ks, float* ss_out,
                    hipStream_t s) {
  const GemvSwiglu none{};
  if (gemv_cols(M, N) == 128) gemv_mt<2, TILED, SS, EPI_F32>(X, W, partial, M, N, K, ks, ss_out, none, s);
  else gemv_mt<1, TILED, SS, EPI_F32>(X, W, partial, M, N, K, ks, ss_out, none, s);
}

void launch_gemv_bf16(const bf16_t* X, const bf16_t* W, bool tiled, float* partial, int M, int N, int K, int ks,
                      float* ss_out, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (tiled) {
    if (ss_out) gemv_nw<true, true>(X, W, partial, M, N, K, ks, ss_out, s);
    else gemv_nw<true, false>(X, W, partial, M, N, K, ks, ss_out, s);
  } else {
    gemv_nw<false, false>(X, W, partial, M, N, K, ks, nullptr, s);
  }
}

void launch_gemv_swiglu(const bf16_t* X, const bf16_t* W, int M, int N, int K, const GemvSwiglu& e,
                        hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (gemv_cols(M, N) == 128) gemv_mt<2, true, false, EPI_SWIGLU>(X, W, nullptr, M, N, K, 1, nullptr, e, s);
  else gemv_mt<1, true, false, EPI_SWIGLU>(X, W, nullptr, M, N, K, 1, nullptr, e, s);
}

// ===========================================================================
// 4-bit GEMV
// ===========================================================================
// Activation preparation, once per call: one block per row m computes
//   xh  [M][K] fp16 in word-pair order: for the 8 codes k0..k0+7 of one word,
//        (x0, x4), (x1/16, x5/16), (x2, x6), (x3/16, x7/16);
//   xsum[M][K/32][2] = (sum of the xh values of the chunk, sum of x of the chunk)
// with x = x_in * r * gamma_k when an RMSNorm feeds the projection (norm 1: r
// from this row's own mean square; norm 2: r from the producer's statistic).
__global__ __launch_bounds__(1024) void k_q4_prep(const bf16_t* X, int norm, RowStat stat, float eps,
                                                  const float* gamma, int M, int K, _Float16* xh, float* xsum) {
  const int m = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bf16_t* xr = X + (size_t)m * K;
  float r = 1.0f;
  if (norm == 1) {
    __shared__ float red[16];
    float t = 0.f;
    for (int k = threadIdx.x; k < K; k += 1024) {
      const float v = bf16_to_f32(xr[k]);
      t += v * v;
    }
    t = warp_sum(t);
    if (lane == 0) red[wave] = t;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < 16; ++w) tot += red[w];
    r = 1.0f / sqrtf(tot / (float)K + eps);
  } else if (norm == 2) {
    r = stat.get_block(m);
  }
  for (int chunk = wave; chunk < K / 32; chunk += 16) {
    float x = 0.f, h = 0.f;
    if (lane < 32) {
      const int k = chunk * 32 + lane;
      x = bf16_to_f32(xr[k]);
      if (norm) x *= r * gamma[k];
      const int j = k & 7;                 // code position inside its word
      const _Float16 hv = (_Float16)(x * ((j & 1) ? (1.0f / 16.0f) : 1.0f));
      h = (float)hv;
      // slot inside the word's 8 fp16: pair p = j % 4, half j / 4
      xh[(size_t)m * K + (k & ~7) + 2 * (j & 3) + (j >> 2)] = hv;
    }
    const float hs = warp_sum(h);
    const float xsv = warp_sum(x);
    if (lane == 0) {
      xsum[((size_t)m * (K / 32) + chunk) * 2 + 0] = hs;
      xsum[((size_t)m * (K / 32) + chunk) * 2 + 1] = xsv;
    }
  }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline half2_t u32_as_h2(uint32_t u) {
  half2_t r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

template <int MR>
__global__ __launch_bounds__(256) void k_gemv_q4(const _Float16* __restrict__ xh, const float* __restrict__ xsum,
                                                const uint32_t* __restrict__ words, const bf16_t* __restrict__ scales,
                                                const bf16_t* __restrict__ biases, float* __restrict__ y, int M, int N,
                                                int K, int gs, int rows_per_wave) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nchunk = K / 32;
  const int ngrp = K / gs;
  const int cpg = gs / 32;  // chunks per group
  const int row0 = (blockIdx.x * 4 + wave) * rows_per_wave;
  for (int rr = 0; rr < rows_per_wave; ++rr) {
    const int n = row0 + rr;
    if (n >= N) return;
    const uint32_t* wrow = words + (size_t)n * (K / 8);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      const uint4 w = ld16(wrow + c * 4);
      const int g = c / cpg;
      const float s = bf16_to_f32(scales[(size_t)n * ngrp + g]);
      const float b = bf16_to_f32(biases[(size_t)n * ngrp + g]);
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
      uint32_t qp[16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t u = wv[t], u8 = wv[t] >> 8;
        qp[4 * t + 0] = (u & 0x000F000Fu) | 0x64006400u;
        qp[4 * t + 1] = (u & 0x00F000F0u) | 0x64006400u;
        qp[4 * t + 2] = (u8 & 0x000F000Fu) | 0x64006400u;
        qp[4 * t + 3] = (u8 & 0x00F000F0u) | 0x64006400u;
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < M) {
          const uint4* xp = reinterpret_cast<const uint4*>(xh + (size_t)m * K + c * 32);
          float a = 0.f;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint4 xv = xp[t];
            a = __builtin_amdgcn_fdot2(u32_as_h2(qp[4 * t + 0]), u32_as_h2(xv.x), a, false);
            a = __builtin_amdgcn_fdot2(u32_as_h2(qp[4 * t + 1]), u32_as_h2(xv.y), a, false);
            a = __builtin_amdgcn_fdot2(u32_as_h2(qp[4 * t + 2]), u32_as_h2(xv.z), a, false);
            a = __builtin_amdgcn_fdot2(u32_as_h2(qp[4 * t + 3]), u32_as_h2(xv.w), a, false);
          }
          const float* xsm = xsum + ((size_t)m * nchunk + c) * 2;
          acc[m] += s * (a - 1024.0f * xsm[0]) + b * xsm[1];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        float v = warp_sum(acc[m]);
        if (lane == 0) y[(size_t)m * N + n] = v;
      }
    }
  }
}

// One row of activations (M = 1, the single-sequence decode of the stack),
// with what follows the projection in the block done in the same kernel.
// No preparation pass: the block's 4 wavefronts form 4 / kp row sets, each
// split over kp parts of K; lane l of a wavefront owns the 32-code chunks
// c0 + l + 64 i (i < NI) of its part and keeps x-hat for them in registers
// (gamma applied, fp16 pairs in the word order of the nibble trick, the two
// chunk sums) for all the rows of its set; the wavefronts of a part convert a
// share of it each and exchange it through LDS.  A wavefront's rows (RW of
// them, unrolled) go through a ring of D + 1 register buffers; each lane keeps
// a partial sum per row and one transposed reduction at the end leaves every
// row's sum in one lane.  Row sums land in LDS; after one barrier the
// block applies the RMSNorm row scale (a per-row scalar, so it multiplies the
// sum) and its epilogue, one thread per output element:
//   Q4E_PLAIN : y[n] = the projection (fp32);
//   Q4E_QKV   : q/k/v with RoPE, k and v appended to the cache (the block's
//               rows are RoPE pairs (i, i + d/2) of whole heads);
//   Q4E_RESID : out = resid + projection, the next RMSNorm's partial sum of
//               squares per block, optional branch copy and cache-length bump;
//   Q4E_SWIGLU: g = silu(w1 n) * (w3 n) (the block's rows are w1/w3 pairs).
constexpr int kQ4MaxRB = 256;   // rows per block at most

// f(integral_constant<int, i>) for i = I .. N-1, unrolled at compile time
template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One 8-code unit of x-hat = x * gamma (word t of a chunk covers codes 8t ..
// 8t+7): the fp16 pairs (x0, x4), (x1/16, x5/16), (x2, x6), (x3/16, x7/16) in
// the word order of the nibble trick, the sum of those fp16 values (hsum) and
// of the fp32 ones (xsum); adds the unit's x^2 (before gamma) to ssq.
__device__ inline void q4_unit(uint4 xraw, bool use_g, f32x4 g0, f32x4 g1, uint32_t (&w)[4], float& hsum,
                               float& xsum, float& ssq) {
  const bf16x8 xb = v_as_bf16x8(xraw);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = (float)xb[e];
    ssq += v[e] * v[e];
  }
  if (use_g) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] *= g0[e];
      v[e + 4] *= g1[e];
    }
  }
  hsum = 0.f;
  xsum = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float sc = (p & 1) ? (1.0f / 16.0f) : 1.0f;
    const _Float16 lo = (_Float16)(v[p] * sc), hi = (_Float16)(v[p + 4] * sc);
    hsum += (float)lo + (float)hi;
    xsum += v[p] + v[p + 4];
    uint16_t l16, h16;
    __builtin_memcpy(&l16, &lo, 2);
    __builtin_memcpy(&h16, &hi, 2);
    w[p] = (uint32_t)l16 | ((uint32_t)h16 << 16);
  }
}

// lane's chunks c0 + lane + 64 i (i < NI, c < c1; zero past c1) of x-hat:
// xw[i][4t + p] = word p of unit t, hs / xs = chunk sums.  Returns the lane's
// sum of x^2.
template <int NI>
__device__ inline float q4_xhat(const bf16_t* __restrict__ X, const float* __restrict__ gamma, int c0, int c1,
                                int lane, uint32_t (&xw)[NI][16], float (&hs)[NI], float (&xs)[NI]) {
  float ssq = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = c0 + lane + 64 * i;
    hs[i] = 0.f;
    xs[i] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 xr = make_uint4(0, 0, 0, 0);
      f32x4 g0 = {1.f, 1.f, 1.f, 1.f}, g1 = g0;
      if (c < c1) {
        const int k0 = c * 32 + 8 * t;
        xr = ld16(X + k0);
        if (gamma) {
          g0 = *reinterpret_cast<const f32x4*>(gamma + k0);
          g1 = *reinterpret_cast<const f32x4*>(gamma + k0 + 4);
        }
      }
      uint32_t w[4];
      float h, x;
      q4_unit(xr, gamma != nullptr, g0, g1, w, h, x, ssq);
      hs[i] += h;
      xs[i] += x;
#pragma unroll
      for (int p = 0; p < 4; ++p) xw[i][4 * t + p] = w[p];
    }
  }
  return ssq;
}

// weight row of the block's local row lr (ok: it exists)
template <int EPI>
__device__ inline int q4_row(const Q4Fused& e, int RB, int lr, bool& ok) {
  if (EPI == Q4E_PLAIN || EPI == Q4E_RESID) {
    const int n = blockIdx.x * RB + lr;
    ok = n < e.N;
    return n;
  }
  const int half = RB >> 1, hi = lr >= half ? 1 : 0, p = blockIdx.x * half + lr - hi * half;
  ok = p < (e.N >> 1);
  if (EPI == Q4E_SWIGLU) return (p / e.ib) * 2 * e.ib + p % e.ib + hi * e.ib;
  const int hd = e.kv.d >> 1;
  return (p / hd) * e.kv.d + p % hd + hi * hd;
}

// One step of a transposed wavefront reduction: lanes with bit M set keep the
// rows of `hi`, the others those of `lo`, and each adds its partner's copy of
// the rows it keeps (two row sets summed over a lane pair in one exchange).
template <int M>
__device__ inline float reduce_split(float lo, float hi, int lane) {
  if constexpr (M >= 16) {
    // vdst = lo, src = hi: afterwards the first result holds lo of the pair in
    // the even rows and hi of the partner in the odd rows, the second the
    // partner's lo in the even rows and hi in the odd rows
    const auto p = M == 16 ? __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi),
                                                              false, false)
                           : __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi),
                                                              false, false);
    return __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
  } else {
    const bool up = lane & M;
    return (up ? hi : lo) + xor_lane<M>(up ? lo : hi, lane);
  }
}

// Sums each of the wavefront's RW row accumulators over the 64 lanes: log2(RW)
// split steps (lane bits 5, 4, ...) leave one value per lane, the remaining
// lane bits are summed plainly.  Returns the sum of row `row` (same in every
// lane whose low 6 - log2(RW) bits are zero).
template <int RW>
__device__ inline float reduce_rows(float (&v)[RW], int lane, int& row) {
  constexpr int LG = RW == 1 ? 0 : RW == 2 ? 1 : RW == 4 ? 2 : RW == 8 ? 3 : 4;
  static_assert((1 << LG) == RW, "rows per wavefront: a power of two up to 16");
  static_for<0, LG>([&](auto sc) {
    constexpr int s = decltype(sc)::value, M = 32 >> s, H = RW >> (s + 1);
    static_for<0, H>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      v[j] = reduce_split<M>(v[j], v[j + H], lane);
    });
  });
  static_for<LG, 6>([&](auto sc) {
    constexpr int M = 32 >> decltype(sc)::value;
    v[0] += xor_lane<M>(v[0], lane);
  });
  row = 0;
#pragma unroll
  for (int s = 0; s < LG; ++s) row += ((lane >> (5 - s)) & 1) * (RW >> (s + 1));
  return v[0];
}

// Block: 4 wavefronts = KP K parts x NSETS = 4 / KP row sets of RW rows (RB =
// NSETS * RW rows per block).  A wavefront's rows are unrolled at compile time:
// the codes and scale/bias of row r + D are requested before row r is
// multiplied (a ring of D + 1 rows in registers), so every wait is a partial
// count and nothing is loaded past the last row.  Row bases are wave-uniform
// (scalar); each lane's chunk offsets are fixed for all rows.  Each lane keeps
// one partial sum per row; one transposed reduction at the end.
template <int NI, int KP, int RW, int D, int EPI>
__global__ __launch_bounds__(256) void k_q4_fused(const bf16_t* __restrict__ X, const uint32_t* __restrict__ words,
                                                 const bf16_t* __restrict__ scales,
                                                 const bf16_t* __restrict__ biases, Q4Fused e) {
  constexpr int NSETS = 4 / KP, RB = NSETS * RW, half = RB / 2;
  static_assert(RB <= kQ4MaxRB, "rows per block");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = e.K, nchunk = K / 32, ngrp = K / 64;
  const int kpi = wave % KP, rs = wave / KP;
  const int c0 = kpi * nchunk / KP, c1 = (kpi + 1) * nchunk / KP;
  // (a residual epilogue's projection takes no RMSNorm: its input is the
  // attention output or the SwiGLU product)
  constexpr bool NORMED = EPI != Q4E_RESID;
  const int norm = NORMED ? e.norm : 0;
  const float* gamma = norm ? e.gamma : nullptr;
  __shared__ float ys[KP][RB];
  __shared__ float ssq_w[4];
  __shared__ float red[4];
  // x-hat shared by the wavefronts of a part: unit (i, t) of lane l
  constexpr int NSH = NSETS > 1 ? KP * NI * 4 * 64 : 1;
  __shared__ uint4 xl[NSH];
  __shared__ float2 hl[NSH];
  // norm 2: the producer's partial sums of squares (lane l: partials l + 64 u,
  // clamped, unconditional so that no wait below covers later loads),
  // requested before everything else and summed after the rows
  constexpr int SU = 8;
  float sp[SU];
  float r_inv = 1.f;
  if (norm == 2) {
    if (e.stat.inv) {
      r_inv = e.stat.inv[0];
    } else if (e.stat.ss) {
#pragma unroll
      for (int u = 0; u < SU; ++u) sp[u] = e.stat.ss[(size_t)min(lane + 64 * u, e.stat.nb - 1) * e.stat.M];
    }
  }
  // with several row sets per part, set rs converts units t = rs * KP + tt of
  // every chunk of the part (tt < KP); its x and gamma go out before the codes
  uint4 xr[NI][KP];
  f32x4 gr[NI][KP][2];
  if constexpr (NSETS > 1) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = c0 + lane + 64 * i;
#pragma unroll
      for (int tt = 0; tt < KP; ++tt) {
        // (lanes past the part read its last chunk and convert zeros)
        const int k0 = min(c, c1 - 1) * 32 + 8 * (rs * KP + tt);
        xr[i][tt] = ld16(X + k0);
        gr[i][tt][0] = gr[i][tt][1] = f32x4{1.f, 1.f, 1.f, 1.f};
        if (gamma) {
          gr[i][tt][0] = *reinterpret_cast<const f32x4*>(gamma + k0);
          gr[i][tt][1] = *reinterpret_cast<const f32x4*>(gamma + k0 + 4);
        }
      }
    }
  }
  // the lane's chunks (lanes past the part repeat its last chunk: loaded, and
  // multiplied by zero activations)
  uint32_t offw[NI], offs[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = min(c0 + lane + 64 * i, c1 - 1);
    offw[i] = (uint32_t)c * 16;
    offs[i] = (uint32_t)(c >> 1) * 2;
  }
  // the wavefront's weight rows, lane j computing row j's index once (rows
  // that do not exist read the block's first); row r is read back into a
  // scalar register where it is used
  int n_lane;
  {
    bool ok;
    n_lane = q4_row<EPI>(e, RB, rs * RW + min(lane, RW - 1), ok);
    if (!ok) n_lane = q4_row<EPI>(e, RB, 0, ok);
  }
  uint4 wc[D + 1][NI];
  uint32_t sv[D + 1][NI], bv[D + 1][NI];
  auto load_row = [&](auto rc) {
    constexpr int r = decltype(rc)::value, b = r % (D + 1);
    const int n = __builtin_amdgcn_readlane(n_lane, r);
    const char* wrow = reinterpret_cast<const char*>(words) + (size_t)n * (K / 2);
    const char* srow = reinterpret_cast<const char*>(scales) + (size_t)n * ngrp * 2;
    const char* brow = reinterpret_cast<const char*>(biases) + (size_t)n * ngrp * 2;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      wc[b][i] = ld16(wrow + offw[i]);
      sv[b][i] = *reinterpret_cast<const uint16_t*>(srow + offs[i]);
      bv[b][i] = *reinterpret_cast<const uint16_t*>(brow + offs[i]);
    }
  };
  static_for<0, (D < RW ? D : RW)>([&](auto j) { load_row(j); });
  // (loads with clamped indices, not under a condition: a conditional load is
  // waited for at once, and that wait would cover the codes requested above)
  bool own_ok = false;
  int own_row = 0;
  bf16_t rv = 0;
  float2 cs = make_float2(1.f, 0.f);
  int pos = 0;
  if (EPI == Q4E_RESID) {
    own_row = blockIdx.x * RB + tid;
    own_ok = tid < RB && own_row < e.N;
    rv = e.resid[min(own_row, e.N - 1)];
  } else if (EPI == Q4E_QKV) {
    const int hd = e.kv.d >> 1;
    own_row = blockIdx.x * half + tid;   // pair index
    own_ok = tid < half && own_row < (e.N >> 1);
    pos = e.kv.lens[0];
    cs = e.rope[(size_t)pos * hd + own_row % hd];
  }
  // everything above is requested before the conversion below starts
  __builtin_amdgcn_sched_barrier(0);
  uint32_t xw[NI][16];
  float hs[NI], xs[NI];
  float ssq = 0.f;
  if constexpr (NSETS > 1) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool inpart = c0 + lane + 64 * i < c1;
#pragma unroll
      for (int tt = 0; tt < KP; ++tt) {
        uint32_t w[4];
        float h, x;
        q4_unit(inpart ? xr[i][tt] : make_uint4(0, 0, 0, 0), gamma != nullptr, gr[i][tt][0], gr[i][tt][1], w, h,
                x, ssq);
        const int u = ((kpi * NI + i) * 4 + rs * KP + tt) * 64 + lane;
        xl[u] = make_uint4(w[0], w[1], w[2], w[3]);
        hl[u] = make_float2(h, x);
      }
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      hs[i] = 0.f;
      xs[i] = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = ((kpi * NI + i) * 4 + t) * 64 + lane;
        const uint4 w = xl[u];
        const float2 h = hl[u];
        xw[i][4 * t + 0] = w.x;
        xw[i][4 * t + 1] = w.y;
        xw[i][4 * t + 2] = w.z;
        xw[i][4 * t + 3] = w.w;
        hs[i] += h.x;
        xs[i] += h.y;
      }
    }
  } else {
    ssq = q4_xhat<NI>(X, gamma, c0, c1, lane, xw, hs, xs);
  }
  // every wavefront's x^2 covers a disjoint share of K, together all of it
  if (norm == 1) {
    ssq = warp_sum(ssq);
    if (lane == 0) ssq_w[wave] = ssq;
  }
  // nibble masks and the fp16 exponent pattern in registers (opaque to the
  // compiler), so each (code & mask) | 0x6400 pair is one three-input bit op
  uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
  asm("" : "+v"(m_lo), "+v"(m_hi), "+v"(magic));
  float acc[RW];
  static_for<0, RW>([&](auto rc) {
    constexpr int r = decltype(rc)::value, b = r % (D + 1);
    if constexpr (r + D < RW) load_row(std::integral_constant<int, r + D>{});
    float a_row = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t wv4[4] = {wc[b][i].x, wc[b][i].y, wc[b][i].z, wc[b][i].w};
      float a = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t u = wv4[t], u8 = wv4[t] >> 8;
        a = __builtin_amdgcn_fdot2(u32_as_h2((u & m_lo) | (magic & ~m_lo)), u32_as_h2(xw[i][4 * t + 0]), a, false);
        a = __builtin_amdgcn_fdot2(u32_as_h2((u & m_hi) | (magic & ~m_hi)), u32_as_h2(xw[i][4 * t + 1]), a, false);
        a = __builtin_amdgcn_fdot2(u32_as_h2((u8 & m_lo) | (magic & ~m_lo)), u32_as_h2(xw[i][4 * t + 2]), a, false);
        a = __builtin_amdgcn_fdot2(u32_as_h2((u8 & m_hi) | (magic & ~m_hi)), u32_as_h2(xw[i][4 * t + 3]), a, false);
      }
      const float s = __builtin_bit_cast(float, sv[b][i] << 16), bi = __builtin_bit_cast(float, bv[b][i] << 16);
      a_row += s * (a - 1024.0f * hs[i]) + bi * xs[i];
    }
    acc[r] = a_row;
  });
  {
    int row;
    const float v = reduce_rows<RW>(acc, lane, row);
    if ((lane & (64 / RW - 1)) == 0) ys[kpi][rs * RW + row] = v;
  }
  __syncthreads();
  // row scale: 1 (norm 0), from the row's mean square over all of K (norm 1),
  // or from the producer's statistic (norm 2)
  float r = 1.0f;
  if (norm == 1) {
    r = 1.0f / sqrtf(((ssq_w[0] + ssq_w[1]) + (ssq_w[2] + ssq_w[3])) / (float)K + e.eps);
  } else if (norm == 2) {
    if (e.stat.inv) {
      r = r_inv;
    } else if (e.stat.ss) {
      // (every wavefront reduces the same values in the same order)
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (lane + 64 * u < e.stat.nb) v += sp[u];
      for (int j = lane + 64 * SU; j < e.stat.nb; j += 64) v += e.stat.ss[(size_t)j * e.stat.M];
      r = 1.0f / sqrtf(warp_sum(v) / (float)e.stat.n + e.stat.eps);
    }
  }
  auto sum_row = [&](int lr) {
    float v = 0.f;
    for (int k = 0; k < KP; ++k) v += ys[k][lr];
    return v * r;
  };
  if (EPI == Q4E_PLAIN) {
    bool ok;
    const int n = q4_row<EPI>(e, RB, tid, ok);
    if (tid < RB && ok) e.y[n] = sum_row(tid);
  } else if (EPI == Q4E_RESID) {
    float o = 0.f;
    if (own_ok) {
      const float f = sum_row(tid);
      if (e.branch) e.branch[own_row] = f32_to_bf16(f);
      o = Elt<bf16_t>::round(bf16_to_f32(rv) + f);
      e.out[own_row] = f32_to_bf16(o);
    }
    if (e.ss_out) {
      const float t = warp_sum(o * o);
      if (lane == 0) red[wave] = t;
      __syncthreads();
      if (tid == 0) e.ss_out[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    }
    if (e.lens_add && blockIdx.x == 0 && tid == 0) e.lens_add[0] += 1;
  } else if (EPI == Q4E_SWIGLU) {
    const int j = blockIdx.x * half + tid;
    if (tid < half && j < (e.N >> 1)) e.g_out[j] = f32_to_bf16(silu_f(sum_row(tid)) * sum_row(tid + half));
  } else if (EPI == Q4E_QKV) {
    if (own_ok) {
      const int d = e.kv.d, hd = d >> 1;
      const int head = own_row / hd, i = own_row % hd, cb0 = head * d;
      float a = sum_row(tid), b = sum_row(tid + half);
      if (cb0 < e.Nq + e.Nkv) {
        const float a2 = a * cs.x - b * cs.y, b2 = b * cs.x + a * cs.y;
        a = a2;
        b = b2;
      }
      const int ca = e.traditional ? 2 * i : i, cb = e.traditional ? 2 * i + 1 : i + hd;
      if (cb0 < e.Nq) {
        e.q_out[cb0 + ca] = f32_to_bf16(a);
        e.q_out[cb0 + cb] = f32_to_bf16(b);
      } else if (cb0 < e.Nq + e.Nkv) {
        const int g = (cb0 - e.Nq) / d;
        bf16_t* Kc = (bf16_t*)e.kv.k;
        Kc[e.kv.k_off(0, pos, g, ca)] = f32_to_bf16(a);
        Kc[e.kv.k_off(0, pos, g, cb)] = f32_to_bf16(b);
      } else {
        const int g = (cb0 - e.Nq - e.Nkv) / d;
        bf16_t* Vc = (bf16_t*)e.kv.v;
        Vc[e.kv.v_off(0, pos, g, i)] = f32_to_bf16(a);
        Vc[e.kv.v_off(0, pos, g, i + hd)] = f32_to_bf16(b);
      }
    }
  }
}

// K parts per block, chunks per lane and rows per wavefront of the single-row
// kernel; false when K is too long for one block (more than 1024 chunks)
static bool q4_fused_shape(int N, int K, int& kp, int& ni, int& rw) {
  const int nchunk = K / 32;
  if (nchunk < 1 || nchunk > 1024) return false;
  kp = nchunk <= 256 ? 1 : nchunk <= 512 ? 2 : 4;
  ni = ((nchunk + kp - 1) / kp + 63) / 64;
  // rows per wavefront: the fewest of 4, 8 and 16 that keep the grid at most
  // 512 blocks, two per compute unit (fewer rows convert x more often for the
  // same weights; more blocks than that measured slower)
  const int sets = 4 / kp;
  rw = 4;
  while (rw < 16 && (N + sets * rw - 1) / (sets * rw) > 512) rw *= 2;
  return true;
}

int q4_fused_blocks(int N, int K) {
  int kp, ni, rw;
  if (!q4_fused_shape(N, K, kp, ni, rw)) return 0;
  const int RB = 4 / kp * rw;
  return (N + RB - 1) / RB;
}

// rows requested ahead of the one being multiplied: 3 with 16 rows per
// wavefront, else 2 (measured: deeper rings were slower at every shape of the
// 13B-width layer, and 2 beat 3 for the shorter wavefronts)
template <int RW>
constexpr int q4_depth() { return RW >= 16 ? 3 : 2; }

bool launch_q4_fused(const bf16_t* X, const uint32_t* words, const bf16_t* scales, const bf16_t* biases,
                     Q4Fused e, hipStream_t s) {
  int kp, ni, rw;
  if (e.N <= 0) return true;
  if (!q4_fused_shape(e.N, e.K, kp, ni, rw)) return false;
  if (e.epi != Q4E_PLAIN && e.epi != Q4E_RESID && (e.N & 1)) return false;
  if (e.epi == Q4E_RESID && e.norm != 0) return false;
  e.kp = kp;
  e.rpw = rw;
  const dim3 grid(q4_fused_blocks(e.N, e.K));
  plan_log("4-bit gemv (one row) N %d K %d: %d blocks, %d rows per wavefront, %d K parts, %d chunks per lane, "
           "epilogue %d", e.N, e.K, (int)grid.x, rw, kp, ni, e.epi);
#define Q4L(n, k, r, E) \
  hipLaunchKernelGGL((k_q4_fused<n, k, r, q4_depth<r>(), E>), grid, dim3(256), 0, s, X, words, scales, biases, e)
#define Q4F(n, k, E)               \
  if (ni == n && kp == k) {        \
    if (rw == 4)                   \
      Q4L(n, k, 4, E);             \
    else if (rw == 8)              \
      Q4L(n, k, 8, E);             \
    else                           \
      Q4L(n, k, 16, E);            \
    return true;                   \
  }
  // (a part of more than 256 chunks is split further, so parts of kp > 1
  // hold more than 128 chunks: 3 or 4 per lane)
#define Q4FE(E)                                                                                     \
  case E:                                                                                           \
    Q4F(1, 1, E) Q4F(2, 1, E) Q4F(3, 1, E) Q4F(4, 1, E) Q4F(3, 2, E) Q4F(4, 2, E) Q4F(3, 4, E) Q4F(4, 4, E) \
    break;
  switch (e.epi) { Q4FE(Q4E_PLAIN) Q4FE(Q4E_QKV) Q4FE(Q4E_RESID) Q4FE(Q4E_SWIGLU) }
#undef Q4FE
#undef Q4F
#undef Q4L
  return false;
}

void launch_gemv_q4(const bf16_t* X, int norm, RowStat stat, float eps, const float* gamma,
                    const uint32_t* words, const bf16_t* scales, const bf16_t* biases, float* y, int M, int N,
                    int K, int gs, _Float16* xh_buf, float* xsum_buf, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (M == 1) {
    Q4Fused e{};
    e.epi = Q4E_PLAIN;
    e.N = N;
    e.K = K;
    e.norm = norm;
    e.stat = stat;
    e.eps = eps;
    e.gamma = gamma;
    e.y = y;
    if (launch_q4_fused(X, words, scales, biases, e, s)) return;
  }
  hipLaunchKernelGGL(k_q4_prep, dim3(M), dim3(1024), 0, s, X, norm, stat, eps, gamma, M, K, xh_buf, xsum_buf);
  const int rpw = 2;
  const int blocks = (N + 4 * rpw - 1) / (4 * rpw);
  plan_log("4-bit gemv M %d N %d K %d: prepared activations, %d blocks of %d rows", M, N, K, blocks, 4 * rpw);
  if (M == 1)
    hipLaunchKernelGGL(k_gemv_q4<1>, dim3(blocks), dim3(256), 0, s, xh_buf, xsum_buf, words, scales, biases, y, M,
                       N, K, gs, rpw);
  else
    hipLaunchKernelGGL(k_gemv_q4<4>, dim3(blocks), dim3(256), 0, s, xh_buf, xsum_buf, words, scales, biases, y, M,
                       N, K, gs, rpw);
}

}  // namespace lb

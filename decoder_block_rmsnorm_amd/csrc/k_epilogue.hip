// Reduce-and-finish kernels behind the split-K decode GEMMs and the fp32 GEMM.
// Each sums the fp32 partials [ks][M][N] in a fixed order (deterministic, no
// atomics) and applies what follows the projection in the block:
//   qkv   : RMSNorm row scale, RoPE on q and k, cache append of k and v;
//   resid : residual add (+ the next RMSNorm's partial statistics, + the
//           feed-forward branch diagnostic, + the cache-length bump);
//   swiglu: RMSNorm row scale, silu(gate) * up.
#include "kernels.hpp"

namespace lb {

// slices summed in order; loads issued four at a time
__device__ inline float sum_parts(const float* part, int ks, size_t stride, size_t idx) {
  float v = 0.f;
  int s = 0;
  for (; s + 4 <= ks; s += 4) {
    const float a = part[(size_t)s * stride + idx], b = part[(size_t)(s + 1) * stride + idx];
    const float c = part[(size_t)(s + 2) * stride + idx], e = part[(size_t)(s + 3) * stride + idx];
    v += a;
    v += b;
    v += c;
    v += e;
  }
  for (; s < ks; ++s) v += part[(size_t)s * stride + idx];
  return v;
}

// ---------------------------------------------------------------------------
// q/k/v finish.  Columns come in the repacked order: per head, pair i is
// (i, i + d/2).  For the interleaved ("traditional") layout the wq/wk rows were
// permuted at creation so that adjacent pairs (2i, 2i+1) land at (i, i + d/2);
// the write below puts them back.  RoPE as in LLaMARoPE (page 二) with the
// angle table built in float64 on the host; the cache offset is the number of
// tokens already cached ("2. 注意力机制" KV-cache fragment, MLX page).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_epi_qkv(const float* part, int ks, int M, int Nq, int Nkv, RowStat stat,
                                                int L, const float2* rope, int traditional, T* q_out, KVView kv) {
  int m = blockIdx.x;
  int head = blockIdx.y;          // 0..H-1 q, H..H+G-1 k, then v
  int d = kv.d, half = d >> 1;
  int i = threadIdx.x;
  const bool act = i < half;
  int N = Nq + 2 * Nkv;
  size_t stride = (size_t)M * N;
  int c0 = head * d;
  int bseq = kv.seq_of_row(m, L), l = m - kv.first_row(bseq, L);
  int pos = kv.lens[bseq] + l;
  int H = Nq / d;
  // the statistic's partials, the slices and the rotation factors are
  // requested together, then the row scale is shared
  const float pv = stat.pre(m);
  float a = 0.f, b = 0.f;
  float2 cs = make_float2(1.f, 0.f);
  if (act) {
    a = sum_parts(part, ks, stride, (size_t)m * N + c0 + i);
    b = sum_parts(part, ks, stride, (size_t)m * N + c0 + i + half);
    if (c0 < Nq + Nkv) cs = rope[(size_t)pos * half + i];
  }
  const float r = stat.finish_block(pv);
  if (!act) return;
  a *= r;
  b *= r;
  if (c0 < Nq + Nkv) {
    float a2 = a * cs.x - b * cs.y;
    float b2 = b * cs.x + a * cs.y;
    a = a2;
    b = b2;
  }
  int ca = traditional ? 2 * i : i;
  int cb = traditional ? 2 * i + 1 : i + half;
  if (c0 < Nq) {
    Elt<T>::store(q_out, (size_t)m * Nq + c0 + ca, a);
    Elt<T>::store(q_out, (size_t)m * Nq + c0 + cb, b);
  } else if (c0 < Nq + Nkv) {
    int g = head - H;
    T* K = (T*)kv.k;
    Elt<T>::store(K, kv.k_off(bseq, pos, g, ca), a);
    Elt<T>::store(K, kv.k_off(bseq, pos, g, cb), b);
  } else {
    int g = head - H - Nkv / d;
    T* V = (T*)kv.v;
    Elt<T>::store(V, kv.v_off(bseq, pos, g, i), a);
    Elt<T>::store(V, kv.v_off(bseq, pos, g, i + half), b);
  }
}

template <typename T>
void launch_epi_qkv(const float* part, int ks, int M, int Nq, int Nkv, RowStat stat, int L, const float2* rope,
                    int traditional, T* q_out, KVView kv, hipStream_t s) {
  if (M <= 0) return;
  dim3 grid(M, (Nq + 2 * Nkv) / kv.d);
  hipLaunchKernelGGL(k_epi_qkv<T>, grid, dim3(64), 0, s, part, ks, M, Nq, Nkv, stat, L, rope, traditional, q_out,
                     kv);
}

// ---------------------------------------------------------------------------
// Residual add: out = resid + sum(partials) (LLaMABlock, page 二; "数据流动"),
// rounded to the storage type.  One thread per column, blocks over (256-column
// chunk, row); optionally each block's sum of squares of the stored values (the
// next RMSNorm's statistic, reduced by its consumer), the feed-forward branch
// itself, and the cache-length bump after the block.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_epi_resid(const float* part, int ks, int M, int N, const T* resid, T* out,
                                                   float* ss_out, int32_t* lens_add, int lens_inc, int n_seq,
                                                   T* branch, const int32_t* lens_cu, int ss_128,
                                                   _Float16* out16, const float* gamma16) {
  const int m = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)M * N;
  float v = 0.f;
  if (c < N) {
    const size_t idx = (size_t)m * N + c;
    const float f = sum_parts(part, ks, stride, idx);
    if (branch) Elt<T>::store(branch, idx, f);
    v = Elt<T>::round(Elt<T>::load(resid, idx) + f);
    Elt<T>::store(out, idx, v);
    // (optional) the stored value times the next RMSNorm's weight, in fp16: the
    // A operand of a 4-bit GEMM, rounded as its copy kernel would round it
    if (out16) out16[idx] = (_Float16)(v * gamma16[c]);
  }
  if (ss_out) {
    __shared__ float red[4];
    const float ss = warp_sum(v * v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      if (!ss_128) {
        ss_out[(size_t)blockIdx.x * M + m] = (red[0] + red[1]) + (red[2] + red[3]);
      } else {
        // one partial per 128 columns (two wavefronts each)
        ss_out[(size_t)(2 * blockIdx.x) * M + m] = red[0] + red[1];
        if ((2 * blockIdx.x + 1) * 128 < N) ss_out[(size_t)(2 * blockIdx.x + 1) * M + m] = red[2] + red[3];
      }
    }
  }
  if (lens_add && m == 0 && blockIdx.x == 0 && (int)threadIdx.x < n_seq)
    lens_add[threadIdx.x] += lens_cu ? lens_cu[threadIdx.x + 1] - lens_cu[threadIdx.x] : lens_inc;
}

template <typename T>
void launch_epi_resid(const float* part, int ks, int M, int N, const T* resid, T* out, float* ss_out,
                      int32_t* lens_add, int lens_inc, int n_seq, T* branch, hipStream_t s, const int32_t* lens_cu,
                      int ss_128, _Float16* out16, const float* gamma16) {
  if (M <= 0) return;
  dim3 grid((N + 255) / 256, M);
  hipLaunchKernelGGL(k_epi_resid<T>, grid, dim3(256), 0, s, part, ks, M, N, resid, out, ss_out, lens_add,
                     lens_inc, n_seq, branch, lens_cu, ss_128, out16, gamma16);
}

// ---------------------------------------------------------------------------
// SwiGLU: g = silu(w1 n) * (w3 n) ("3. 前馈网络", MLX page; LLaMAMLP, page 二).
// w1/w3 rows are interleaved in blocks of ib: block 2j holds w1 rows
// j*ib .. j*ib+ib-1, block 2j+1 the same w3 rows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_epi_swiglu(const float* part, int ks, int M, int F2, int ib, RowStat stat,
                                                    T* g_out) {
  int m = blockIdx.y;
  int F = F2 >> 1;
  int j = blockIdx.x * 256 + threadIdx.x;
  size_t stride = (size_t)M * F2;
  int jb = j / ib, w = j % ib;
  int cg = jb * 2 * ib + w;
  const float pv = stat.pre(m);
  float a = 0.f, b = 0.f;
  if (j < F) {
    a = sum_parts(part, ks, stride, (size_t)m * F2 + cg);
    b = sum_parts(part, ks, stride, (size_t)m * F2 + cg + ib);
  }
  const float r = stat.finish_block(pv);
  if (j >= F) return;
  Elt<T>::store(g_out, (size_t)m * F + j, silu_f(a * r) * (b * r));
}

template <typename T>
void launch_epi_swiglu(const float* part, int ks, int M, int F2, int ib, RowStat stat, T* g_out, hipStream_t s) {
  if (M <= 0) return;
  dim3 grid((F2 / 2 + 255) / 256, M);
  hipLaunchKernelGGL(k_epi_swiglu<T>, grid, dim3(256), 0, s, part, ks, M, F2, ib, stat, g_out);
}

__global__ __launch_bounds__(256) void k_reduce_f32(const float* part, int ks, int M, int N, float* out) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  size_t total = (size_t)M * N;
  if (i < total) out[i] = sum_parts(part, ks, total, i);
}

void launch_reduce_f32(const float* part, int ks, int M, int N, float* out, hipStream_t s) {
  size_t total = (size_t)M * N;
  if (!total) return;
  hipLaunchKernelGGL(k_reduce_f32, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, ks, M, N, out);
}

#define INST(T)                                                                                                 \
  template void launch_epi_qkv<T>(const float*, int, int, int, int, RowStat, int, const float2*, int, T*, KVView, \
                                  hipStream_t);                                                                 \
  template void launch_epi_resid<T>(const float*, int, int, int, const T*, T*, float*, int32_t*, int, int, T*,    \
                                    hipStream_t, const int32_t*, int, _Float16*, const float*);                 \
  template void launch_epi_swiglu<T>(const float*, int, int, int, int, RowStat, T*, hipStream_t);
INST(float)
INST(bf16_t)
#undef INST

}  // namespace lb

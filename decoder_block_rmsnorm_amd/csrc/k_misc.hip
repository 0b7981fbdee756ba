// Small kernels: RMSNorm statistics, embedding gather, argmax, cache copies,
// weight repacking and 4-bit dequantisation.
#include "kernels.hpp"

namespace lb {

// ---------------------------------------------------------------------------
// RMSNorm statistics -- "4. RMSNorm" of the MLX page / LLaMARMSNorm of page 二:
// inv = 1 / sqrt(mean(x^2) + eps).  One wavefront per row, fp32 sum of squares
// reduced across the 64 lanes.  The gamma multiply is folded elsewhere (into the
// next GEMM's weights, or applied by rmsnorm_apply).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float row_sumsq(const T* row, int D, int lane) {
  float ss = 0.f;
  for (int i = lane; i < D; i += 64) {
    float v = Elt<T>::load(row, i);
    ss += v * v;
  }
  return warp_sum(ss);
}

template <>
__device__ inline float row_sumsq<bf16_t>(const bf16_t* row, int D, int lane) {
  float ss = 0.f;
  if ((D & 7) == 0) {
    for (int i = lane * 8; i < D; i += 512) {
      uint4 w = ld16(row + i);
      uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = bf16_to_f32((bf16_t)(u[j] & 0xffff));
        float b = bf16_to_f32((bf16_t)(u[j] >> 16));
        ss += a * a + b * b;
      }
    }
  } else {
    for (int i = lane; i < D; i += 64) {
      float v = bf16_to_f32(row[i]);
      ss += v * v;
    }
  }
  return warp_sum(ss);
}

template <typename T>
__global__ __launch_bounds__(256) void k_rms_inv(const T* x, int rows, int D, float eps, float* inv) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float ss = row_sumsq<T>(x + (size_t)row * D, D, lane);
  if (lane == 0) inv[row] = 1.0f / sqrtf(ss / (float)D + eps);
}

template <typename T>
void launch_rms_inv(const T* x, int rows, int D, float eps, float* inv, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_rms_inv<T>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, D, eps, inv);
}

template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_apply(const T* x, const T* gamma, int rows, int D,
                                                       float eps, T* out) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* xr = x + (size_t)row * D;
  float ss = row_sumsq<T>(xr, D, lane);
  float r = 1.0f / sqrtf(ss / (float)D + eps);
  for (int i = lane; i < D; i += 64)
    Elt<T>::store(out, (size_t)row * D + i, Elt<T>::load(xr, i) * r * Elt<T>::load(gamma, i));
}

template <typename T>
void launch_rmsnorm_apply(const T* x, const T* gamma, int rows, int D, float eps, T* out, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_rmsnorm_apply<T>, dim3((rows + 3) / 4), dim3(256), 0, s, x, gamma, rows, D, eps, out);
}

// ---------------------------------------------------------------------------
// Embedding lookup -- "1. 嵌入层" of the MLX page: out[i] = table[ids[i]].
// ss_out (optional): the rows' sums of squares per 128 columns, [ceil(D/128)][n]
// (the statistic of the first block's RMSNorm)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const T* table, int vocab, int D, const int32_t* ids, T* out,
                                               float* ss_out, int n) {
  int i = blockIdx.x;
  int id = ids[i];
  bool ok = id >= 0 && id < vocab;
  __shared__ float red[4];
  for (int c0 = 0; c0 < D; c0 += 256) {
    const int c = c0 + threadIdx.x;
    float v = 0.f;
    if (c < D) {
      const T e = ok ? table[(size_t)id * D + c] : T(0);
      out[(size_t)i * D + c] = e;
      v = Elt<T>::to_f(e);
    }
    if (ss_out) {
      const float t = warp_sum(v * v);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
      __syncthreads();
      if (threadIdx.x == 0) {
        ss_out[(size_t)(c0 / 128) * n + i] = red[0] + red[1];
        if (c0 + 128 < D) ss_out[(size_t)(c0 / 128 + 1) * n + i] = red[2] + red[3];
      }
      __syncthreads();
    }
  }
}

template <typename T>
void launch_embed(const T* table, int vocab, int D, const int32_t* ids, int n, T* out, hipStream_t s, float* ss_out) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_embed<T>, dim3(n), dim3(256), 0, s, table, vocab, D, ids, out, ss_out, n);
}

// ---------------------------------------------------------------------------
// Greedy choice -- argmax at temperature 0 ("生成过程", MLX page): the first
// index holding the largest logit.  Block reduction keeps (value, index) with
// the lower index on equal values, so the result is deterministic.
// ---------------------------------------------------------------------------
__device__ inline void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(1024) void k_argmax(const float* logits, int vocab, int32_t* ids) {
  const float* row = logits + (size_t)blockIdx.x * vocab;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < vocab; i += 1024) better(bv, bi, row[i], i);
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    better(bv, bi, ov, oi);
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = sv[0];
    int id = si[0];
    for (int k = 1; k < 16; ++k) better(v, id, sv[k], si[k]);
    ids[blockIdx.x] = (id == 0x7fffffff) ? 0 : id;
  }
}

void launch_argmax(const float* logits, int rows, int vocab, int32_t* ids, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(1024), 0, s, logits, vocab, ids);
}

// ---------------------------------------------------------------------------
// Sampled next id ("生成过程", MLX page: a multinomial draw from
// softmax(logits / T) when T > 0; LLaMA.generate, page 二: limited to the
// nucleus, the most probable tokens up to and including the first at which
// their cumulative probability exceeds top_p).  One block per row, 1024 threads.
//   e_i = 2^((z_i - max) * log2(e) / T), kept in LDS up to kSampleLds tokens,
//   else recomputed by the same instructions in every pass (so every pass sees
//   the same values; no scratch);
//   nucleus: the kept tokens are e_i >= thr, thr = the largest e value whose
//   tail mass (the sum of all e_j >= it) exceeds top_p * sum(e), found by
//   bisection over the bit patterns of positive floats (ordered like their
//   values); tokens tied with it are kept;
//   draw: the first index, in vocabulary order, at which the cumulative kept
//   mass exceeds u * (kept mass), u = u[*u_off or row].  Each thread sums one
//   contiguous 1/1024 of the row, the first wavefront chains the 1024 sums
//   into prefixes in order, so the chunks' intervals [prefix, next prefix) tile
//   [0, total) and one chunk holds the crossing.
// ---------------------------------------------------------------------------
constexpr int kSampleThreads = 1024;
constexpr int kSampleLds = 36864;   // e values kept in LDS (144 KB) up to this vocabulary

__device__ inline float block_reduce_s(float v, bool is_max, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  __syncthreads();   // red is reused by consecutive reductions
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kSampleThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// CACHE: e_i computed once into LDS (vocab <= kSampleLds), else recomputed
// by the same instructions in every pass
template <bool CACHE>
__global__ __launch_bounds__(kSampleThreads) void k_sample(const float* logits, int vocab, float temperature,
                                                           float top_p, const float* u, const int32_t* u_off,
                                                           int32_t* ids) {
  extern __shared__ float e_s[];
  const float* z = logits + (size_t)blockIdx.x * vocab;
  const int tid = threadIdx.x;
  constexpr int NT = kSampleThreads;
  __shared__ float red[NT / 64];
  __shared__ float pre[NT + 1];
  __shared__ int found, last_kept;
  float m = -INFINITY;
  for (int i = tid; i < vocab; i += NT) m = fmaxf(m, z[i]);
  m = block_reduce_s(m, true, red);
  const float k2 = 1.4426950408889634f / temperature;
  auto e_calc = [&](int i) { return __builtin_amdgcn_exp2f((z[i] - m) * k2); };
  if constexpr (CACHE) {
    for (int i = tid; i < vocab; i += NT) e_s[i] = e_calc(i);
    __syncthreads();
  }
  auto e_of = [&](int i) { return CACHE ? e_s[i] : e_calc(i); };
  float thr = 0.f;
  if (top_p < 1.f) {
    float tot = 0.f;
    for (int i = tid; i < vocab; i += NT) tot += e_of(i);
    const float target = top_p * block_reduce_s(tot, false, red);
    // invariant: tail(lo) > target >= tail(hi); e <= 1, so tail(1 + ulp) = 0
    uint32_t lo = 0u, hi = 0x3f800001u;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      const float t = __uint_as_float(mid);
      float sm = 0.f;
      for (int i = tid; i < vocab; i += NT) {
        const float e = e_of(i);
        if (e >= t) sm += e;
      }
      if (block_reduce_s(sm, false, red) > target) lo = mid;
      else hi = mid;
    }
    thr = __uint_as_float(lo);
  }
  const int C = (vocab + NT - 1) / NT;
  const int i0 = min(vocab, tid * C), i1 = min(vocab, i0 + C);
  float cs = 0.f;
  int lk = -1;
  for (int i = i0; i < i1; ++i) {
    const float e = e_of(i);
    if (e >= thr) {
      cs += e;
      lk = i;
    }
  }
  pre[tid] = cs;
  if (tid == 0) {
    found = 0x7fffffff;
    last_kept = -1;
  }
  __syncthreads();
  // prefixes in chunk order by the first wavefront: lane l sums chunks
  // 16 l .. 16 l + 15, the 64 lane sums are chained in order, then each lane
  // writes its 16 prefixes from its start, one chunk sum at a time.  (Where a
  // lane's last prefix and the next lane's start differ by rounding, two
  // chunks' intervals may overlap but never leave a gap; the lower index wins.)
  if (tid < 64) {
    constexpr int PER = NT / 64;
    float ls = 0.f;
    for (int j = 0; j < PER; ++j) ls = ls + pre[tid * PER + j];
    float base = 0.f;
    for (int l = 0; l < 64; ++l) {
      const float v = __shfl(ls, l, 64);
      if (l == tid) ls = base;   // this lane's starting prefix
      base = base + v;
    }
    float run = ls;
    for (int j = 0; j < PER; ++j) {
      const float c = pre[tid * PER + j];
      pre[tid * PER + j] = run;
      run = run + c;
    }
    if (tid == 63) pre[NT] = run;
  }
  atomicMax(&last_kept, lk);
  __syncthreads();
  const float target = u[u_off ? *u_off : blockIdx.x] * pre[NT];
  if (pre[tid] <= target && target < pre[tid + 1]) {
    // the chunk holding the crossing (its own running sum may round short of
    // it: then its last kept token)
    float run = pre[tid];
    int pick = lk;
    for (int i = i0; i < i1; ++i) {
      const float e = e_of(i);
      if (e >= thr) {
        run += e;
        if (run > target) {
          pick = i;
          break;
        }
      }
    }
    atomicMin(&found, pick);
  }
  __syncthreads();
  // (u * total rounded up to total: the last kept token)
  if (tid == 0) ids[blockIdx.x] = found != 0x7fffffff ? found : max(last_kept, 0);
}

void launch_sample(const float* logits, int rows, int vocab, float temperature, float top_p, const float* u,
                   const int32_t* u_off, int32_t* ids, hipStream_t s) {
  if (rows <= 0) return;
  if (temperature <= 0.f) return launch_argmax(logits, rows, vocab, ids, s);
  if (vocab <= kSampleLds) {
    static bool attr = false;
    const size_t lds = (size_t)kSampleLds * sizeof(float);
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)k_sample<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      attr = true;
    }
    hipLaunchKernelGGL(k_sample<true>, dim3(rows), dim3(kSampleThreads), (size_t)vocab * sizeof(float), s, logits,
                       vocab, temperature, top_p, u, u_off, ids);
  } else {
    hipLaunchKernelGGL(k_sample<false>, dim3(rows), dim3(kSampleThreads), 0, s, logits, vocab, temperature, top_p,
                       u, u_off, ids);
  }
}

// ---------------------------------------------------------------------------
// Paged cache <-> canonical [n, G, d] copies (cache pre-fill and read-back).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_kv_copy(KVView kv, int seq, int pos0, int n, const T* kin,
                                                 const T* vin, T* kout, T* vout) {
  size_t total = (size_t)n * kv.G * kv.d;
  T* K = (T*)kv.k;
  T* V = (T*)kv.v;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    int e = (int)(i % kv.d);
    int g = (int)((i / kv.d) % kv.G);
    int t = (int)(i / ((size_t)kv.d * kv.G));
    int pos = pos0 + t;
    size_t ko = kv.k_off(seq, pos, g, e), vo = kv.v_off(seq, pos, g, e);
    if (kin) {
      K[ko] = kin[i];
      V[vo] = vin[i];
    } else {
      kout[i] = K[ko];
      vout[i] = V[vo];
    }
  }
}

template <typename T>
void launch_kv_write(KVView kv, int seq, int pos0, int n, const T* k, const T* v, hipStream_t s) {
  size_t total = (size_t)n * kv.G * kv.d;
  if (!total) return;
  int blocks = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_kv_copy<T>, dim3(blocks), dim3(256), 0, s, kv, seq, pos0, n, k, v, (T*)nullptr,
                     (T*)nullptr);
}

template <typename T>
void launch_kv_read(KVView kv, int seq, int pos0, int n, T* k, T* v, hipStream_t s) {
  size_t total = (size_t)n * kv.G * kv.d;
  if (!total) return;
  int blocks = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_kv_copy<T>, dim3(blocks), dim3(256), 0, s, kv, seq, pos0, n, (const T*)nullptr,
                     (const T*)nullptr, k, v);
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
void launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
}

struct I32Vals {
  int32_t n;
  int32_t v[kMaxSetI32];
};
__global__ __launch_bounds__(256) void k_set_i32(I32Vals a, int32_t* dst) {
  for (int i = threadIdx.x; i < a.n; i += 256) dst[i] = a.v[i];
}
void launch_set_i32(const int32_t* vals, int n, int32_t* dst, hipStream_t s) {
  if (n <= 0) return;
  I32Vals a{};
  a.n = n < kMaxSetI32 ? n : kMaxSetI32;
  for (int i = 0; i < a.n; ++i) a.v[i] = vals[i];
  hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(256), 0, s, a, dst);
}

// ---------------------------------------------------------------------------
// Weight repacking (runs once at block creation).
// ---------------------------------------------------------------------------
__device__ inline int repack_dst_row(int r, int row0, int ib, int ib_stride, int perm_d) {
  if (perm_d > 0) {
    int local = r % perm_d;
    int dl = (local & 1) ? (perm_d / 2 + local / 2) : (local / 2);
    r = (r / perm_d) * perm_d + dl;
  }
  return row0 + (r / ib) * ib_stride + (r % ib);
}

// tiled != 0: destination in the tiled layout (row-major otherwise)
template <typename T>
__global__ __launch_bounds__(256) void k_repack_rows(T* dst, const T* src, int rows, int K, const T* gamma,
                                                     int row0, int ib, int ib_stride, int perm_d, int tgroups) {
  int r = blockIdx.x;
  int dr = repack_dst_row(r, row0, ib, ib_stride, perm_d);
  // tgroups > 0: tiled layout of a [16 * tgroups][K] matrix, whose padding past
  // K is written as zeros (readers may take whole chunks)
  const int kend = tgroups ? tiled_chunks(K) * kTileK : K;
  for (int c = threadIdx.x; c < kend; c += 256) {
    float v = 0.f;
    if (c < K) {
      v = Elt<T>::load(src, (size_t)r * K + c);
      if (gamma) v *= Elt<T>::load(gamma, c);
    }
    Elt<T>::store(dst, tgroups ? tiled_off(dr, c, tgroups) : (size_t)dr * K + c, v);
  }
}

template <typename T>
void launch_repack_rows(T* dst, const T* src, int rows, int K, const T* gamma, int row0, int ib, int ib_stride,
                        int perm_d, int tgroups, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_repack_rows<T>, dim3(rows), dim3(256), 0, s, dst, src, rows, K, gamma, row0, ib,
                     ib_stride, perm_d, tgroups);
}

__global__ __launch_bounds__(256) void k_repack_bytes(uint8_t* dst, const uint8_t* src, int rows, int rb,
                                                      int row0, int ib, int ib_stride, int perm_d) {
  int r = blockIdx.x;
  int dr = repack_dst_row(r, row0, ib, ib_stride, perm_d);
  for (int c = threadIdx.x; c < rb; c += 256) dst[(size_t)dr * rb + c] = src[(size_t)r * rb + c];
}

void launch_repack_bytes(uint8_t* dst, const uint8_t* src, int rows, int row_bytes, int row0, int ib,
                         int ib_stride, int perm_d, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_repack_bytes, dim3(rows), dim3(256), 0, s, dst, src, rows, row_bytes, row0, ib,
                     ib_stride, perm_d);
}

// ---------------------------------------------------------------------------
// 4-bit group-affine dequantisation to fp16 (prompt pass of the quantized
// stack): W[o, k] = scale[o, k/gs] * code[o, k] + bias[o, k/gs], the 4-bit /
// group-64 format of the MLX quantization config ("模型配置").  The norm weight
// of the following RMSNorm-fed GEMM is folded in (gamma_k) before the single
// rounding to fp16 (11 significant bits: 4x finer than bf16).  Row-major
// (one block per row), or in the tiled layout of the dense weights (one block
// per 16-row x 256-column tile, written as one contiguous 8 KB run; zeros past
// K up to the chunk boundary); one word of 8 codes -> one 16-byte store.
// ---------------------------------------------------------------------------
__device__ inline uint4 q4_dequant_word(const uint32_t* words, const bf16_t* scales, const bf16_t* biases, int row,
                                        int K, int gs, const float* gamma, int k0) {
  const uint32_t u = words[(size_t)row * (K / 8) + k0 / 8];
  const int g = k0 / gs;
  const float sc = bf16_to_f32(scales[(size_t)row * (K / gs) + g]);
  const float bi = bf16_to_f32(biases[(size_t)row * (K / gs) + g]);
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = sc * (float)((u >> (8 * j)) & 15u) + bi;
    float b = sc * (float)((u >> (8 * j + 4)) & 15u) + bi;
    if (gamma) { a *= gamma[k0 + 2 * j]; b *= gamma[k0 + 2 * j + 1]; }
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    uint16_t ua, ub;
    __builtin_memcpy(&ua, &ha, 2);
    __builtin_memcpy(&ub, &hb, 2);
    o[j] = (uint32_t)ua | ((uint32_t)ub << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ __launch_bounds__(256) void k_q4_dequant(const uint32_t* words, const bf16_t* scales,
                                                    const bf16_t* biases, int N, int K, int gs,
                                                    const float* gamma, _Float16* out) {
  const int row = blockIdx.x;
  for (int w = threadIdx.x; w < K / 8; w += 256)
    st16(out + (size_t)row * K + w * 8, q4_dequant_word(words, scales, biases, row, K, gs, gamma, w * 8));
}

// tile (16-row group blockIdx.x, 256-column chunk blockIdx.y), 128 threads:
// thread (r = t % 16, 32-column block kb = t / 16) expands 32 codes of row
// 16 g + r (one 16-byte load) into the four 16-byte pieces kb * 64 + 16 j + r
// of the tile, so that each store instruction writes 256 contiguous bytes per
// 16 lanes
__global__ __launch_bounds__(128) void k_q4_dequant_tiled(const uint32_t* words, const bf16_t* scales,
                                                          const bf16_t* biases, int N, int K, int gs,
                                                          const float* gamma, _Float16* out) {
  const int g = blockIdx.x, c = blockIdx.y;
  const int r = threadIdx.x & 15, kb = threadIdx.x >> 4;
  const int row = g * 16 + r, kbase = c * kTileK + kb * 32;
  _Float16* tile = out + ((size_t)c * (N >> 4) + g) * kTileElems;
  uint32_t u[4] = {0u, 0u, 0u, 0u};
  float sc = 0.f, bi = 0.f;
  const bool in = kbase < K;   // (K % 32 == 0: a block is inside K or past it)
  if (in) {
    const uint4 w = ld16(words + (size_t)row * (K / 8) + kbase / 8);
    u[0] = w.x; u[1] = w.y; u[2] = w.z; u[3] = w.w;
    sc = bf16_to_f32(scales[(size_t)row * (K / gs) + kbase / gs]);
    bi = bf16_to_f32(biases[(size_t)row * (K / gs) + kbase / gs]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (in) {
      const int k0 = kbase + 8 * j;
      float gm[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
      if (gamma) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + k0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + k0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gm[e] = g0[e];
          gm[e + 4] = g1[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = (sc * (float)((u[j] >> (8 * e)) & 15u) + bi) * gm[2 * e];
        const float b = (sc * (float)((u[j] >> (8 * e + 4)) & 15u) + bi) * gm[2 * e + 1];
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        uint16_t ua, ub;
        __builtin_memcpy(&ua, &ha, 2);
        __builtin_memcpy(&ub, &hb, 2);
        o[e] = (uint32_t)ua | ((uint32_t)ub << 16);
      }
    }
    st16(tile + (kb * 64 + 16 * j + r) * 8, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

void launch_q4_dequant(const uint32_t* words, const bf16_t* scales, const bf16_t* biases, int N, int K, int gs,
                       const float* gamma, bool tiled, _Float16* out, hipStream_t s) {
  if (N <= 0) return;
  if (tiled)
    hipLaunchKernelGGL(k_q4_dequant_tiled, dim3(N >> 4, tiled_chunks(K)), dim3(128), 0, s, words, scales, biases, N,
                       K, gs, gamma, out);
  else
    hipLaunchKernelGGL(k_q4_dequant, dim3(N), dim3(256), 0, s, words, scales, biases, N, K, gs, gamma, out);
}

// fp16 copy of bf16 values, 8 per thread (n % 8 == 0; |v| < 65504 on its
// uses), times gamma[column] for rows of K columns when gamma is given (the
// RMSNorm weight of a 4-bit GEMM's input; one rounding of the exact product)
__global__ __launch_bounds__(256) void k_bf16_to_f16(const bf16_t* src, _Float16* dst, size_t n8, const float* gamma,
                                                     int K) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = ld16(src + i * 8);
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  float gm[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if (gamma) {
    const int c0 = (int)((i * 8) % (size_t)K);   // (K % 8 == 0: the 8 values share a row)
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + c0);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + c0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gm[e] = g0[e];
      gm[e + 4] = g1[e];
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)(__uint_as_float(in[j] << 16) * gm[2 * j]);
    const _Float16 hi = (_Float16)(__uint_as_float(in[j] & 0xffff0000u) * gm[2 * j + 1]);
    uint16_t l, h;
    __builtin_memcpy(&l, &lo, 2);
    __builtin_memcpy(&h, &hi, 2);
    o[j] = (uint32_t)l | ((uint32_t)h << 16);
  }
  st16(dst + i * 8, make_uint4(o[0], o[1], o[2], o[3]));
}

void launch_bf16_to_f16(const bf16_t* src, _Float16* dst, size_t n, hipStream_t s, const float* gamma, int K) {
  const size_t n8 = n / 8;
  if (!n8) return;
  hipLaunchKernelGGL(k_bf16_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, src, dst, n8, gamma, K);
}

// Group scale/bias pairs transposed to [G][N], one 32-bit word per (group,
// row): the 4-bit prompt-pass GEMM loads a group's pairs for 256 rows at once.
__global__ __launch_bounds__(256) void k_q4_pairs(const bf16_t* scales, const bf16_t* biases, int N, int G,
                                                  uint32_t* pairs) {
  const int n = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y;
  if (n >= N) return;
  pairs[(size_t)g * N + n] = (uint32_t)scales[(size_t)n * G + g] | ((uint32_t)biases[(size_t)n * G + g] << 16);
}

void launch_q4_pairs(const bf16_t* scales, const bf16_t* biases, int N, int G, uint32_t* pairs, hipStream_t s) {
  if (N <= 0 || G <= 0) return;
  hipLaunchKernelGGL(k_q4_pairs, dim3((N + 255) / 256, G), dim3(256), 0, s, scales, biases, N, G, pairs);
}

template <typename T>
__global__ void k_to_f32(const T* src, float* dst, int n) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = Elt<T>::load(src, i);
}
template <typename T>
void launch_to_f32(const T* src, float* dst, int n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_to_f32<T>, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
}

// ---------------------------------------------------------------------------
// Generation bookkeeping: ids_out[*cursor] = *cur_id (and the logits row),
// then *cursor += 1.  Keeps the emitted ids on the device between steps.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(const int32_t* cur_id, int32_t* ids_out, int32_t* cursor,
                                              const float* logits, float* logits_out, int V) {
  const int c = *cursor;
  if (threadIdx.x == 0) ids_out[c] = *cur_id;
  if (logits_out)
    for (int i = threadIdx.x; i < V; i += 256) logits_out[(size_t)c * V + i] = logits[i];
  __syncthreads();
  if (threadIdx.x == 0) *cursor = c + 1;
}

// p[i * stride] = v for i < n (one lens entry per cache layer)
__global__ __launch_bounds__(64) void k_fill_strided_i32(int32_t* p, int n, int stride, int32_t v) {
  for (int i = threadIdx.x; i < n; i += 64) p[(size_t)i * stride] = v;
}

void launch_fill_strided_i32(int32_t* p, int n, int stride, int32_t v, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_fill_strided_i32, dim3(1), dim3(64), 0, s, p, n, stride, v);
}

void launch_emit(const int32_t* cur_id, int32_t* ids_out, int32_t* cursor, const float* logits, float* logits_out,
                 int V, hipStream_t s) {
  hipLaunchKernelGGL(k_emit, dim3(1), dim3(256), 0, s, cur_id, ids_out, cursor, logits, logits_out, V);
}

// explicit instantiations
#define INST(T)                                                                                     \
  template void launch_rms_inv<T>(const T*, int, int, float, float*, hipStream_t);                  \
  template void launch_rmsnorm_apply<T>(const T*, const T*, int, int, float, T*, hipStream_t);      \
  template void launch_embed<T>(const T*, int, int, const int32_t*, int, T*, hipStream_t, float*);  \
  template void launch_kv_write<T>(KVView, int, int, int, const T*, const T*, hipStream_t);         \
  template void launch_kv_read<T>(KVView, int, int, int, T*, T*, hipStream_t);                      \
  template void launch_repack_rows<T>(T*, const T*, int, int, const T*, int, int, int, int, int, hipStream_t); \
  template void launch_to_f32<T>(const T*, float*, int, hipStream_t);
INST(float)
INST(bf16_t)
#undef INST

}  // namespace lb

// Host-side launchers of the gfx950 kernels (one definition per .hip file).
#pragma once
#include "common.hpp"
#include "trace.hpp"

namespace lb {

// RMSNorm row statistic of row m, from whichever source a producer left:
//   inv[m] directly, or partial sums of squares ss[j * M + m] (j < nb) over the
//   n elements of the row, reduced here in a fixed order; neither: 1.
struct RowStat {
  const float* inv = nullptr;
  const float* ss = nullptr;
  int nb = 0, M = 0, n = 1;
  float eps = 0.f;
  // 1/rms of row m, computed by the first wavefront of the block (its lanes
  // sum the nb partials) and shared: every thread of the block must call it,
  // with the same m, before any thread leaves.  In two halves so that a caller
  // can request its own loads in between: pre() requests this thread's share
  // of the partials, finish_block() reduces them and shares the result through
  // LDS (a barrier that waits for LDS traffic only, not for loads in flight).
  __device__ inline float pre(int m) const {
    float v = 0.f;
    if (threadIdx.x < 64) {
      if (inv) {
        if (threadIdx.x == 0) v = inv[m];
      } else if (ss) {
        if ((int)threadIdx.x < nb) v = ss[(size_t)threadIdx.x * M + m];
        for (int j = threadIdx.x + 64; j < nb; j += 64) v += ss[(size_t)j * M + m];
      }
    }
    return v;
  }
  __device__ inline float finish_block(float v) const {
    __shared__ float s_r;
    if (threadIdx.x < 64) {
      float r = 1.0f;
      if (inv) r = warp_sum(v);
      else if (ss) r = 1.0f / sqrtf(warp_sum(v) / (float)n + eps);
      if (threadIdx.x == 0) s_r = r;
    }
    lds_barrier();
    return s_r;
  }
  __device__ inline float get_block(int m) const { return finish_block(pre(m)); }
};

// Launch-attached timing events (profiling aid).  When set, the prefill GEMM
// launch records `start` and `stop` in its own dispatch, and the decode
// attention records `start` with its main kernel and `stop` with its merge
// kernel; each launcher clears what it used.  No extra stream packets, so the
// timed phase adds no gap to the stream.
struct LaunchClock {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchClock g_clock;

// ---------------------------------------------------------------- k_misc.hip
// inv_rms[r] = 1 / sqrt(mean(x[r,:]^2) + eps) for rows of x [rows, D].
template <typename T>
void launch_rms_inv(const T* x, int rows, int D, float eps, float* inv_rms, hipStream_t s);
// out[r,:] = x[r,:] * inv_rms(x[r]) * gamma  (act dtype out)
template <typename T>
void launch_rmsnorm_apply(const T* x, const T* gamma, int rows, int D, float eps, T* out, hipStream_t s);
template <typename T>
void launch_embed(const T* table, int vocab, int D, const int32_t* ids, int n, T* out, hipStream_t s,
                  float* ss_out = nullptr);
// ids[r] = first index of the max of logits[r, :vocab]
void launch_argmax(const float* logits, int rows, int vocab, int32_t* ids, hipStream_t s);
// ids[r] = sampled id of row r (temperature <= 0: argmax), draw u[*u_off] when
// u_off is given (one row), else u[r]
void launch_sample(const float* logits, int rows, int vocab, float temperature, float top_p, const float* u,
                   const int32_t* u_off, int32_t* ids, hipStream_t s);
// canonical [n, G, d] <-> paged
template <typename T>
void launch_kv_write(KVView kv, int seq, int pos0, int n, const T* k, const T* v, hipStream_t s);
template <typename T>
void launch_kv_read(KVView kv, int seq, int pos0, int n, T* k, T* v, hipStream_t s);
void launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
// dst[0 .. n) = vals[0 .. n) (host values, n <= kMaxSetI32), carried in the
// kernel's arguments: no host buffer has to outlive the call
constexpr int kMaxSetI32 = 257;
void launch_set_i32(const int32_t* vals, int n, int32_t* dst, hipStream_t s);
void launch_fill_strided_i32(int32_t* p, int n, int stride, int32_t v, hipStream_t s);
// Row repack.  Source row r first moves inside its head when perm_d > 0
// (local index j -> j/2 for even j, perm_d/2 + j/2 for odd j: interleaved pairs
// become (i, i + d/2) pairs), then lands at dst row row0 + (r'/ib)*ib_stride + r'%ib.
// gamma (optional, length K) scales the columns (norm weight folding).
// tgroups > 0: dst is in the tiled layout of a [16 * tgroups][K] matrix.
template <typename T>
void launch_repack_rows(T* dst, const T* src, int rows, int K, const T* gamma, int row0, int ib,
                        int ib_stride, int perm_d, int tgroups, hipStream_t s);
void launch_repack_bytes(uint8_t* dst, const uint8_t* src, int rows, int row_bytes, int row0, int ib,
                         int ib_stride, int perm_d, hipStream_t s);
// fp16 (scale * code + bias) * gamma_k (gamma may be null): row-major [N, K], or
// (tiled) in the tiled layout of an [N, K] weight (N % 16 == 0, tiled_chunks(K) *
// 256 columns, zero past K)
void launch_q4_dequant(const uint32_t* words, const bf16_t* scales, const bf16_t* biases, int N, int K,
                       int gs, const float* gamma, bool tiled, _Float16* out, hipStream_t s);
// dst = fp16(src), or fp16(src * gamma[column]) for rows of K columns when gamma is given
void launch_bf16_to_f16(const bf16_t* src, _Float16* dst, size_t n, hipStream_t s, const float* gamma = nullptr,
                        int K = 0);
// pairs[g][n] = scales[n][g] | biases[n][g] << 16 (bf16 bit patterns), G groups per row
void launch_q4_pairs(const bf16_t* scales, const bf16_t* biases, int N, int G, uint32_t* pairs, hipStream_t s);
template <typename T>
void launch_to_f32(const T* src, float* dst, int n, hipStream_t s);
// ids_out[*cursor] = *cur_id; logits_out[*cursor] = logits (if logits_out); ++*cursor
void launch_emit(const int32_t* cur_id, int32_t* ids_out, int32_t* cursor, const float* logits, float* logits_out,
                 int V, hipStream_t s);

// ----------------------------------------------------------- k_gemm_simt.hip
// C[M, N] (fp32) = A[M, K] * B[N, K]^T   (generic; used by the fp32 path)
template <typename T>
void launch_gemm_simt(const T* A, const T* B, float* C, int M, int N, int K, hipStream_t s);

// ----------------------------------------------------------- k_gemm_mfma.hip
enum GemmEpi { EPI_F32 = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_RESID = 3 };
struct GemmArgs {
  const bf16_t* A;  // [M, K] bf16
  const bf16_t* B;  // [N, K] bf16, or fp16 bit patterns when b_f16
  int M, N, K;
  int b_f16;        // B is fp16 and the MFMA runs on fp16: B row-major, A (bf16)
                    // converted on the way into LDS; or, with a_f16, A fp16 and
                    // B fp16 in the tiled layout (gemm_f16_direct_ok shapes)
  int a_f16;
  int ksplit;       // EPI_F32 only: K split into ksplit slices, slice s -> C + s*M*N
  // EPI_F32
  float* C;
  // row scale (QKV / SWIGLU): inv_rms[M], or, when inv_rms is null, 1/rms from
  // rstat's partial sums of squares (rstat.ss[j * rstat.M + m], j < rstat.nb <=
  // kGemmMaxRowPartials), reduced once per block
  const float* inv_rms;
  RowStat rstat;
  // EPI_QKV
  bf16_t* q_out;          // [M, Nq]
  int Nq, Nkv, L;         // row m = b * L + l (or the ragged rows of kv.cu)
  const float2* rope;     // [max_seq][64] (cos, sin)
  int traditional;
  KVView kv;
  // EPI_SWIGLU
  bf16_t* g_out;          // [M, N/2]
  // EPI_RESID
  const bf16_t* resid;    // [M, N]
  bf16_t* out;            // [M, N]
  int32_t* lens_add;      // if non-null: lens_add[b] += lens_inc for b < n_seq (block 0),
  int lens_inc, n_seq;    // or += lens_cu[b + 1] - lens_cu[b] when lens_cu is set
  const int32_t* lens_cu;
  bf16_t* branch;         // if non-null: the product before the residual add [M, N]
  float* ss_out;          // if non-null: sums of squares of the stored rows, one per
                          // 128-column block: ss_out[(col / 128) * M + row]
  // 4-bit B (with b_f16 and a_f16, gemm_q4_direct_ok shapes): B dequantized in
  // the kernel from codes q4w [N][K/8] words (code k at bits 4*(k%8)) and group
  // scale/bias pairs q4sb [K/64][N] (scale in the low 16 bits, bias in the
  // high, bf16): B[n][k] = fp16(scale * code + bias); B itself is unused
  const uint32_t* q4w;
  const uint32_t* q4sb;
  // columns [n_lo, n_hi) of the product only (n_hi = 0: up to N); set by the
  // launcher when it splits one product over two tile shapes
  int n_lo, n_hi;
};
constexpr int kGemmMaxRowPartials = 64;
void launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t s);
// K slices (1, 2 or 4) for an [M, N] x K product (B in fp16 when b_f16) whose
// tile grid alone leaves the chip short of work; slice s writes fp32 partials
// at C + s*M*N
constexpr int kMaxSplitK = 4;
int gemm_split_k(int M, int N, int K, bool b_f16);
// 4-bit weights dequantized inside the GEMM: any slice count up to
// kMaxSplitKQ4 (slices x 256 x 256 tiles within one round of 256 blocks)
constexpr int kMaxSplitKQ4 = 8;
int gemm_split_k_q4(int M, int N, int K);
// shapes whose fp16 GEMM can take A fp16 and B tiled (direct-to-LDS tiles)
bool gemm_f16_direct_ok(int M, int N, int K);
// shapes whose fp16 GEMM can take 4-bit B dequantized in the kernel
bool gemm_q4_direct_ok(int M, int N, int K);

// ---------------------------------------------------------------- k_gemv.hip
// partial[ks][M][N] (fp32) = X[M, kslice] * W[N, kslice]^T (bf16, M <= 64),
// W tiled (tiled_off) or row-major; slice s = 256-column chunks
// [s * nchk / ks, (s + 1) * nchk / ks), nchk = tiled_chunks(K).
// ss_out (optional): sum of squares of each X row over each K slice, [ks][M].
void launch_gemv_bf16(const bf16_t* X, const bf16_t* W, bool tiled, float* partial, int M, int N, int K, int ks,
                      float* ss_out, hipStream_t s);
// columns of W per GEMV block (64 or 128)
int gemv_cols(int M, int N);
// g[M][N/2] (bf16) = silu(y1 * r) * (y3 * r) for y = X W^T over all of K
// (W tiled, rows interleaved in blocks of ib: w1 rows, then the same w3 rows),
// r = 1/rms of row m from stat.  No scratch.
struct GemvSwiglu {
  RowStat stat;
  int ib;
  bf16_t* g_out;
};
void launch_gemv_swiglu(const bf16_t* X, const bf16_t* W, int M, int N, int K, const GemvSwiglu& e,
                        hipStream_t s);
// y[M][N] (fp32) = xhat W^T, W 4-bit group affine, xhat = x * r * gamma, M <= 4.
// norm: 0 = no RMSNorm (r = 1, gamma unused), 1 = r from the row itself (eps),
// 2 = r from `stat`.  xh_buf: fp16 [M, K]; xsum_buf: fp32 [M, K/32, 2] (scratch,
// used unless M = 1 and K <= 32768).
void launch_gemv_q4(const bf16_t* X, int norm, RowStat stat, float eps, const float* gamma,
                    const uint32_t* words, const bf16_t* scales, const bf16_t* biases, float* y, int M, int N,
                    int K, int gs, _Float16* xh_buf, float* xsum_buf, hipStream_t s);
// Single-row (M = 1) 4-bit projection X W^T (W: N rows, K inputs, groups of 64)
// with its epilogue in the same kernel, bf16 activations.  r and gamma as in
// launch_gemv_q4.
enum Q4Epi { Q4E_PLAIN = 0, Q4E_QKV = 1, Q4E_RESID = 2, Q4E_SWIGLU = 3 };
struct Q4Fused {
  int epi, N, K;
  int kp, rpw;            // set by the launcher
  int norm;
  RowStat stat;
  float eps;
  const float* gamma;
  float* y;               // PLAIN: [N]
  // QKV (rows in the repacked order: per head, RoPE pair i is (i, i + d/2)):
  // q_out [Nq]; k, v appended at position kv.lens[0] of sequence 0
  int Nq, Nkv;
  const float2* rope;
  int traditional;
  bf16_t* q_out;
  KVView kv;
  // RESID: out = resid + y [N]; ss_out (optional): one sum of squares of the
  // stored values per block [q4_fused_blocks]; branch (optional): y in bf16;
  // lens_add (optional): lens_add[0] += 1
  const bf16_t* resid;
  bf16_t* out;
  float* ss_out;
  int32_t* lens_add;
  bf16_t* branch;
  // SWIGLU: rows interleaved in blocks of ib (w1 rows, then the same w3 rows);
  // g_out [N/2]
  int ib;
  bf16_t* g_out;
};
// false (nothing launched) when K > 32768, a paired epilogue has odd N or a
// residual epilogue asks for a norm
bool launch_q4_fused(const bf16_t* X, const uint32_t* words, const bf16_t* scales, const bf16_t* biases,
                     Q4Fused e, hipStream_t s);
// blocks of the single-row kernel for [N, K] (0: not supported)
int q4_fused_blocks(int N, int K);

// ------------------------------------------------------------ k_epilogue.hip
// All take fp32 partials [ks][M][N] and reduce them in a fixed order.
template <typename T>
void launch_epi_qkv(const float* part, int ks, int M, int Nq, int Nkv, RowStat stat, int L,
                    const float2* rope, int traditional, T* q_out, KVView kv, hipStream_t s);
// out = resid + sum(part); ss_out (optional): per-256-column-block sums of squares of
// the stored rows, [ceil(N/256)][M] (a RowStat source for the next RMSNorm), or per
// 128 columns, [ceil(N/128)][M], with ss_128.
// lens_add (optional): lens_add[b] += lens_inc, or lens_cu[b + 1] - lens_cu[b]
// when lens_cu is given, for b < n_seq.
template <typename T>
void launch_epi_resid(const float* part, int ks, int M, int N, const T* resid, T* out, float* ss_out,
                      int32_t* lens_add, int lens_inc, int n_seq, T* branch, hipStream_t s,
                      const int32_t* lens_cu = nullptr, int ss_128 = 0, _Float16* out16 = nullptr,
                      const float* gamma16 = nullptr);
template <typename T>
void launch_epi_swiglu(const float* part, int ks, int M, int F2, int ib, RowStat stat, T* g_out,
                       hipStream_t s);
// logits[M][N] = sum_ks part
void launch_reduce_f32(const float* part, int ks, int M, int N, float* out, hipStream_t s);

// ---------------------------------------------------------------- k_attn.hip
// generic causal attention over the paged cache (fp32 path):
// q [M, H*d] with row m = b*L + l (or the ragged rows of kv.cu) at position
// lens_before[b] + l; out [M, H*d]
template <typename T>
void launch_attn_simt(const T* q, KVView kv, int M, int L, int H, int G, int d, T* out, hipStream_t s);
// bf16 flash prefill (d = 128); L = new tokens per sequence, or the most of any
// sequence of a ragged call (kv.cu)
void launch_attn_prefill_bf16(const bf16_t* q, KVView kv, int B, int L, int H, int G, bf16_t* out,
                              hipStream_t s);
// bf16 split-K decode (d = 128): one token per sequence at position lens[b] (already appended)
void launch_attn_decode_bf16(const bf16_t* q, KVView kv, int B, int H, int G, int n_splits, int split_len,
                             float* part_o, float* part_ml, bf16_t* out, hipStream_t s);

}  // namespace lb

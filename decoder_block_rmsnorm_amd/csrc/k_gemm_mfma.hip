// bf16 MFMA GEMM for the prompt pass:  C[M, N] = A[M, K] * B[N, K]^T
// (A = activations, B = repacked nn.Linear weights, both K-contiguous), fp32
// accumulation on v_mfma_f32_32x32x16_bf16, with the block's element-wise work
// fused into the epilogue so no fp32 intermediate reaches HBM:
//   EPI_F32    : plain fp32 store;
//   EPI_QKV    : RMSNorm row scale (gamma is folded into the weights), RoPE on
//                q and k, q to a [M, Nq] buffer, k and v appended to the pages;
//   EPI_SWIGLU : RMSNorm row scale, silu(w1 n) * (w3 n) on interleaved columns;
//   EPI_RESID  : residual add (wo and w2).
//
// Tiling: BM x BN block tile (BM, BN in {128, 256}), K step 64, four wavefronts,
// each owning a (BM / WM) x 128 tile so that one wavefront always holds whole
// 128-wide heads (the RoPE partner columns i and i + 64 sit in the same lane).
// Global -> registers -> LDS with the next K step prefetched during the MFMAs;
// LDS rows padded to 72 bf16 (144 B) against bank conflicts; two LDS buffers,
// one barrier per K step.  Blocks are renumbered XCD-major and walked in
// GROUP_M-row bands so that co-resident blocks of one XCD share A and B tiles
// in that XCD's L2.
#include "kernels.hpp"

namespace lb {

namespace gm {
constexpr int BK = 64;
constexpr int LDS_ST = BK + 8;  // bf16 per LDS row
constexpr int GROUP_M = 8;
}  // namespace gm

__device__ inline bf16x8 u4_as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_mfma(GemmArgs a) {
  using namespace gm;
  constexpr int WN = BN / 128;
  constexpr int WM = 4 / WN;
  constexpr int WTM = BM / WM;
  constexpr int MI = WTM / 32;
  constexpr int A_CH = BM * 8 / 256;  // 16-byte chunks per thread per K step
  constexpr int B_CH = BN * 8 / 256;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  // buffer b: A tile at lds + b * (BM + BN) * LDS_ST, B tile right after it
  auto As = [&](int b) { return lds + b * (BM + BN) * LDS_ST; };
  auto Bs = [&](int b) { return lds + b * (BM + BN) * LDS_ST + BM * LDS_ST; };

  const int M = a.M, N = a.N, K = a.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  // XCD-major renumbering, then grouped ordering
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (bid % per_group) % gsz;
  const int tn = (bid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hg = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  const bf16_t* Ag = a.A;
  const bf16_t* Bg = a.B;
  uint4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + 256 * i;
      int r = c >> 3, kc = c & 7;
      int gr = min(m0 + r, M - 1);
      ra[i] = ld16(Ag + (size_t)gr * K + k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + 256 * i;
      int r = c >> 3, kc = c & 7;
      rb[i] = ld16(Bg + (size_t)(n0 + r) * K + k0 + kc * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + 256 * i;
      st16(As(buf) + (c >> 3) * LDS_ST + (c & 7) * 8, ra[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + 256 * i;
      st16(Bs(buf) + (c >> 3) * LDS_ST + (c & 7) * 8, rb[i]);
    }
  };

  f32x16 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  const int KT = K / BK;
  gload(0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    lstore(buf);
    __syncthreads();
    if (kt + 1 < KT) gload(kt + 1);
    const bf16_t* as = As(buf) + (wm * WTM + l32) * LDS_ST + hg * 8;
    const bf16_t* bs = Bs(buf) + (wn * 128 + l32) * LDS_ST + hg * 8;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[MI], bfr[4];
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = u4_as_bf16x8(ld16(as + i * 32 * LDS_ST + kk * 16));
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = u4_as_bf16x8(ld16(bs + j * 32 * LDS_ST + kk * 16));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---------------- epilogue: lane holds column l32 of each 32x32 subtile,
  // rows 8*(r/4) + 4*hg + r%4 for register r.
  const int wcol0 = n0 + wn * 128;  // first column of this wavefront (head aligned)
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hg + (r & 3);
      if (row >= M) continue;
      if constexpr (EPI == EPI_F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a.C[(size_t)row * N + wcol0 + j * 32 + l32] = acc[i][j][r];
      } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          size_t idx = (size_t)row * N + wcol0 + j * 32 + l32;
          if (a.branch) a.branch[idx] = f32_to_bf16(acc[i][j][r]);
          a.out[idx] = f32_to_bf16(bf16_to_f32(a.resid[idx]) + acc[i][j][r]);
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        const float rs = a.inv_rms[row];
        const int F = N >> 1;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          // interleave block of 32: columns wcol0 + 64*jp .. +31 are w1 rows,
          // the next 32 the matching w3 rows
          const int blk = (wcol0 + 64 * jp) >> 5;
          const int j = (blk >> 1) * 32 + l32;
          float gt = acc[i][2 * jp][r] * rs, up = acc[i][2 * jp + 1][r] * rs;
          a.g_out[(size_t)row * F + j] = f32_to_bf16(silu_f(gt) * up);
        }
      } else {  // EPI_QKV
        const float rs = a.inv_rms[row];
        const int bseq = row / a.L, l = row - bseq * a.L;
        const int pos = a.kv.lens[bseq] + l;
        const bool is_q = wcol0 < a.Nq;
        const bool is_k = !is_q && wcol0 < a.Nq + a.Nkv;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const int pi = jp * 32 + l32;  // pair index: columns pi and pi + 64 of the head
          float x0 = acc[i][jp][r] * rs, x1 = acc[i][jp + 2][r] * rs;
          if (is_q || is_k) {
            float2 cs = a.rope[(size_t)pos * 64 + pi];
            float y0 = x0 * cs.x - x1 * cs.y;
            float y1 = x1 * cs.x + x0 * cs.y;
            x0 = y0;
            x1 = y1;
          }
          if (is_q) {
            const int ca = a.traditional ? 2 * pi : pi;
            const int cb = a.traditional ? 2 * pi + 1 : pi + 64;
            bf16_t* qr = a.q_out + (size_t)row * a.Nq + wcol0;
            qr[ca] = f32_to_bf16(x0);
            qr[cb] = f32_to_bf16(x1);
          } else if (is_k) {
            const int ca = a.traditional ? 2 * pi : pi;
            const int cb = a.traditional ? 2 * pi + 1 : pi + 64;
            const int g = (wcol0 - a.Nq) >> 7;
            bf16_t* Kc = (bf16_t*)a.kv.k;
            Kc[a.kv.k_off(bseq, pos, g, ca)] = f32_to_bf16(x0);
            Kc[a.kv.k_off(bseq, pos, g, cb)] = f32_to_bf16(x1);
          } else {
            const int g = (wcol0 - a.Nq - a.Nkv) >> 7;
            bf16_t* Vc = (bf16_t*)a.kv.v;
            Vc[a.kv.v_off(bseq, pos, g, pi)] = f32_to_bf16(x0);
            Vc[a.kv.v_off(bseq, pos, g, pi + 64)] = f32_to_bf16(x1);
          }
        }
      }
    }
  }
  if constexpr (EPI == EPI_RESID) {
    if (a.lens_add && blockIdx.x == 0 && tid < a.n_seq) a.lens_add[tid] += a.lens_inc;
  }
}

template <int BM, int BN, int EPI>
static void launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * (a.N / BN);
  const size_t lds = (size_t)2 * (BM + BN) * gm::LDS_ST * sizeof(bf16_t);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_mfma<BM, BN, EPI>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)lds);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, EPI>), dim3(tiles), dim3(256), lds, s, a);
}

template <int EPI>
static void launch_epi(const GemmArgs& a, hipStream_t s) {
  // Pick the largest tile that still gives about one wave of blocks per CU.
  const long t256 = (long)((a.M + 255) / 256) * (a.N / 256);
  const bool n256 = (a.N % 256) == 0;
  if (n256 && t256 >= 240) return launch_cfg<256, 256, EPI>(a, s);
  if (n256 && (long)((a.M + 127) / 128) * (a.N / 256) >= 200) return launch_cfg<128, 256, EPI>(a, s);
  if (n256) return launch_cfg<128, 256, EPI>(a, s);
  return launch_cfg<128, 128, EPI>(a, s);
}

void launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return;
  switch (epi) {
    case EPI_F32: return launch_epi<EPI_F32>(a, s);
    case EPI_QKV: return launch_epi<EPI_QKV>(a, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s);
    default: return launch_epi<EPI_RESID>(a, s);
  }
}

}  // namespace lb

// bf16 MFMA GEMM for the prompt pass:  C[M, N] = A[M, K] * B[N, K]^T
// (A = activations, B = repacked nn.Linear weights, both K-contiguous), fp32
// accumulation on v_mfma_f32_32x32x16_bf16, with the block's element-wise work
// fused into the epilogue so no fp32 intermediate reaches HBM:
//   EPI_F32    : plain fp32 store (split-K partials);
//   EPI_QKV    : RMSNorm row scale (gamma is folded into the weights), RoPE on
//                q and k, q to a [M, Nq] buffer, k and v appended to the pages;
//   EPI_SWIGLU : RMSNorm row scale, silu(w1 n) * (w3 n) on interleaved columns;
//   EPI_RESID  : residual add (wo and w2), optionally with the sums of squares
//                of the stored rows per 128 columns: the statistic of the next
//                RMSNorm, which the W1/W3 GEMM reduces into its row scales.
//
// Main path (DEPTH 0; every bf16 prefill GEMM whose N is a multiple of 256):
// a 256 x 256 (or 128 x 256) block tile, four wavefronts, each owning a
// (BM / 2) x 128 tile so that one wavefront always holds whole 128-wide heads
// (the RoPE partner columns i and i + 64 sit in the same lane).  A and B stream
// global -> LDS with direct loads (global_load_lds_dwordx4, no register
// staging) into a four-stage ring of 32-wide K steps; the LDS image is laid out
// in 16-row x 32-column blocks of 1 KB (the tiled weight format), so every
// direct load of a wavefront fills one contiguous kilobyte and fragment reads
// have no bank conflicts.  One load or fragment read is slotted after each
// MFMA, with one barrier per K step.  Blocks are renumbered XCD-major and
// walked in GROUP_M-row bands so that co-resident blocks of one XCD share A and
// B tiles in that XCD's L2.
// Other paths (DEPTH 1/2, register-staged 64-wide K steps through two padded
// LDS buffers): split-K partials, N not a multiple of 256, and row-major fp16
// B operands (4-bit weights dequantized for shapes the tiled layout misses).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kernels.hpp"

namespace lb {

namespace gm {
constexpr int BK = 64;
constexpr int LDS_ST = BK + 8;  // bf16 per LDS row
constexpr int GROUP_M = 8;
}  // namespace gm

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E), so that
// accumulator registers are always indexed by constants (a runtime index would
// push the accumulator array to scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ inline bf16x8 u4_as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// F16: the MFMA runs on fp16 operands (4-bit weights dequantized to fp16).
// Register-staged tiles: B fp16 row-major, A (bf16) converted to fp16 on its
// way into LDS.  Direct-to-LDS tiles: A already fp16 in memory, B fp16 in the
// tiled layout.
__device__ inline uint4 bf16x8_to_f16x8(uint4 v) {
  uint32_t in[4] = {v.x, v.y, v.z, v.w}, out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)bf16_to_f32((bf16_t)(in[j] & 0xffffu));
    const _Float16 hi = (_Float16)bf16_to_f32((bf16_t)(in[j] >> 16));
    uint16_t l, h;
    __builtin_memcpy(&l, &lo, 2);
    __builtin_memcpy(&h, &hi, 2);
    out[j] = (uint32_t)l | ((uint32_t)h << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

__device__ inline f16x8 u4_as_f16x8(uint4 v) {
  f16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// NW wavefronts per block (4 or 8), DEPTH K steps of global loads in flight
// (1 or 2 register sets).  DEPTH 0 (bf16 tiled B, 256 x 256, 4 wavefronts):
// global -> LDS direct loads (global_load_lds_dwordx4) into a four-stage ring of
// 32-wide K steps, no register staging; see the main loop below.
// Q4 (DEPTH 0, F16): B is 4-bit group-affine weights dequantized inside the
// kernel: each step's codes and group scale/bias pairs come into the ring stage
// with the A tile (direct loads), and every thread turns its row's 32 codes
// into fp16 s * q + b in the stage's B tile one step before the MFMAs read it.
template <int BM, int BN, int NW, int DEPTH, int EPI, bool F16, bool Q4 = false>
__global__ __launch_bounds__(NW * 64, 1) void k_gemm_mfma(GemmArgs a) {
  using namespace gm;
  constexpr int NT = NW * 64;
  constexpr int WN = BN / 128;
  constexpr int WM = NW / WN;
  constexpr int WTM = BM / WM;
  constexpr int MI = WTM / 32;
  constexpr int A_CH = BM * 8 / NT;  // 16-byte chunks per thread per K step
  constexpr int B_CH = BN * 8 / NT;
  static_assert(MI >= 1 && A_CH >= 1 && B_CH >= 1, "tile / wave split");
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  // buffer b: A tile at lds + b * (BM + BN) * LDS_ST, B tile right after it
  auto As = [&](int b) { return lds + b * (BM + BN) * LDS_ST; };
  auto Bs = [&](int b) { return lds + b * (BM + BN) * LDS_ST + BM * LDS_ST; };

  const int M = a.M, N = a.N;
  const int n_lo = a.n_lo, n_hi = a.n_hi > 0 ? a.n_hi : N;   // this launch's columns
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (n_hi - n_lo) / BN;
  // XCD-major renumbering, then grouped ordering; K slice = slowest index
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int ntile = tiles_m * tiles_n;
  const int ksi = bid / ntile;
  bid -= ksi * ntile;
  const int K = a.K;                          // row stride of A and B
  const int Kslice = a.K / (a.ksplit > 0 ? a.ksplit : 1);
  // B: fp16 row-major [N][K] (dequantized 4-bit weights) or bf16 in the tiled
  // layout (chunk-major): the 32-column block holding column k of 16-row group
  // g sits at tblk(k) + g * kTileElems, and a 64-wide K step that starts on a
  // multiple of 64 stays inside one chunk (2 KB of each group)
  const int ngr = N >> 4;
  auto tblk = [&](int k) { return (size_t)(k >> 8) * ngr * kTileElems + ((k >> 5) & 7) * 512; };
  const int kslice0 = ksi * Kslice;
  const bf16_t* Ag = a.A + (size_t)kslice0;
  constexpr bool DIRECT = DEPTH == 0 || DEPTH == 3 || DEPTH == 4;
  constexpr bool BROW = F16 && !DIRECT;   // B row-major (else tiled)
  const bf16_t* Bg = a.B + (BROW ? (size_t)kslice0 : 0);
  const int per_group = GROUP_M * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (bid % per_group) % gsz;
  const int tn = (bid % per_group) / gsz;
  const int m0 = tm * BM, n0 = n_lo + tn * BN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hg = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  // Two register sets of prefetched K steps: the global loads of step kt+2 are
  // issued while step kt is multiplied, so each load has two MFMA phases to land.
  uint4 ra0[A_CH], rb0[B_CH], ra1[A_CH], rb1[B_CH];
  // Tile bases are uniform (scalar registers); per-lane offsets are 32-bit
  // element offsets (operands are < 2^31 elements), so each load needs one VGPR
  // of address instead of two.
  const bf16_t* Atile = Ag + (size_t)m0 * K;
  const bf16_t* Btile = Bg + (BROW ? (size_t)n0 * K : (size_t)(n0 >> 4) * kTileElems);
  uint32_t aoff[A_CH], boff[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + NT * i, r = c >> 3, kc = c & 7;
    aoff[i] = (uint32_t)(min(r, M - 1 - m0) * K + kc * 8);
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + NT * i;
    if constexpr (BROW) {
      boff[i] = (uint32_t)((c >> 3) * K + (c & 7) * 8);
    } else {
      // piece c of a K step: group c / 128, 1 KB block (c / 64) % 2, lane c % 64
      boff[i] = (uint32_t)((c >> 7) * kTileElems + ((c >> 6) & 1) * 512 + (c & 63) * 8);
    }
  }
  auto gload = [&](int kt, uint4(&ra)[A_CH], uint4(&rb)[B_CH]) {
    const bf16_t* at = Atile + kt * BK;
    const bf16_t* bt = Btile + (BROW ? (size_t)kt * BK : tblk(kslice0 + kt * BK));
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = ld16(at + aoff[i]);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = ld16(bt + boff[i]);
  };
  auto lstore = [&](int buf, const uint4(&ra)[A_CH], const uint4(&rb)[B_CH]) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + NT * i;
      st16(As(buf) + (c >> 3) * LDS_ST + (c & 7) * 8, F16 ? bf16x8_to_f16x8(ra[i]) : ra[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + NT * i;
      if constexpr (BROW)
        st16(Bs(buf) + (c >> 3) * LDS_ST + (c & 7) * 8, rb[i]);
      else  // row 16 * group + lane % 16, columns 32 * block + 8 * (lane / 16)
        st16(Bs(buf) + ((c >> 7) * 16 + (c & 15)) * LDS_ST + ((c >> 6) & 1) * 32 + ((c >> 4) & 3) * 8, rb[i]);
    }
  };

  f32x16 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  // One K step from LDS buffer `buf`: fragments of sub-step kk+1 are read while
  // the MFMAs of sub-step kk run (two fragment register sets), and the
  // scheduler is asked to interleave one LDS read between MFMAs.
  auto compute = [&](int buf) {
    const bf16_t* as = As(buf) + (wm * WTM + l32) * LDS_ST + hg * 8;
    const bf16_t* bs = Bs(buf) + (wn * 128 + l32) * LDS_ST + hg * 8;
    // 4 wavefronts (one per SIMD): fragments double-buffered so the next
    // sub-step's LDS reads overlap this sub-step's MFMAs.  8 wavefronts: one
    // fragment set (registers go to the second prefetch set instead); the other
    // wavefront on the SIMD covers the LDS latency.
    constexpr int FS = NW == 4 ? 2 : 1;
    uint4 fa[FS][MI], fb[FS][4];
    auto lfrag = [&](int kk, uint4(&a_)[MI], uint4(&b_)[4]) {
#pragma unroll
      for (int i = 0; i < MI; ++i) a_[i] = ld16(as + i * 32 * LDS_ST + kk * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) b_[j] = ld16(bs + j * 32 * LDS_ST + kk * 16);
    };
    auto mfmas = [&](const uint4(&a_)[MI], const uint4(&b_)[4]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(u4_as_f16x8(a_[i]), u4_as_f16x8(b_[j]), acc[i][j],
                                                               0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u4_as_bf16x8(a_[i]), u4_as_bf16x8(b_[j]),
                                                                acc[i][j], 0, 0, 0);
        }
    };
    if constexpr (FS == 2) {
      lfrag(0, fa[0], fb[0]);
      static_for<0, BK / 16>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        constexpr int cur = kk & 1;
        if constexpr (kk + 1 < BK / 16) lfrag(kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
        // fence: the reads above are issued before, and stay before, these MFMAs
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fa[cur], fb[cur]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        lfrag(kk, fa[0], fb[0]);
        mfmas(fa[0], fb[0]);
      }
    }
  };

  // LDS buffer b is rewritten two steps after it was read; the barrier of the
  // step in between guarantees every wavefront has finished reading it.
  if constexpr (DEPTH == 0 || DEPTH == 3 || DEPTH == 4) {   // (BM 128 or 256 with DEPTH 0)
    // Direct-to-LDS ring (DEPTH 0: 32-wide K steps in 4 stages; DEPTH 3:
    // 64-wide K steps in 2 stages).  A stage holds the A and B tiles of one K
    // step as 16-row x 32-column blocks of 1 KB in the tiled weight format
    // (piece 16*j + r = row r of the group, columns 8j .. 8j+7), block (kb, g)
    // at (kb * 16 + g) KB: every direct load instruction of a wavefront fills
    // one contiguous kilobyte (lane l -> piece l), and every 16-lane phase of a
    // fragment read touches 256 contiguous bytes (no bank conflicts).  Each
    // wavefront loads 4 row groups of A and of B per 32 columns of the step.
    //
    // Schedule of step kt, sub-steps kk of 16 (fragments of kk = 0 already in
    // registers): read the fragments of kk+1, then the MFMAs of kk; before the
    // MFMAs of the last sub-step: wait for this wavefront's loads of step kt+1,
    // barrier (all loads of kt+1 landed, every wavefront done reading stage
    // kt), refill stage kt with step kt+STG, read the kk = 0 fragments of step
    // kt+1.  The matrix cores stay busy across the barrier.
    constexpr int BKS = DEPTH == 3 ? 64 : 32;          // K step
    constexpr int STG = DEPTH == 0 ? 4 : DEPTH == 3 ? 2 : 5;   // stages
    constexpr int NKB = BKS / 32;                      // 32-column blocks per step
    constexpr int NKK = BKS / 16;                      // MFMA sub-steps per step
    // direct loads per wavefront per step: A and B groups, or (Q4) A groups,
    // this wavefront's 64 rows of codes and a copy of the 256 rows' scale/bias pairs
    constexpr int LPS = Q4 ? BM / 64 + 2 : (BM / 64 + 4) * NKB;
    static_assert((!F16 || DEPTH == 0) && NW == 4 && BN == 256 && (BM == 256 || (BM == 128 && DEPTH == 0)),
                  "direct-LDS configuration");
    static_assert(!Q4 || (F16 && DEPTH == 0), "4-bit B: fp16 MFMA on the four-stage ring");
    constexpr int AG = BM / 64, BG = 4;                // A and B row groups each wavefront loads
    constexpr int SA = BM * BKS, SB = BN * BKS;        // bf16 per stage
    // (Q4) per stage after the B tile: codes, 16 bytes per row; NW copies of the
    // pairs, 4 bytes per row (in 2-byte units)
    constexpr int SC = Q4 ? BN * 8 : 0, SS = Q4 ? NW * BN * 2 : 0;
    constexpr int STS = SA + SB + SC + SS;             // 2-byte units per stage
    const int KT = Kslice / BKS;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int r16 = lane & 15, j4 = lane >> 4;
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(char*)lds);
    // Per-lane byte offsets (32-bit: the host keeps A below 4 GB) from the
    // slice bases: A rows of this lane's pieces (clamped: rows past M load row
    // M-1, whose results are never stored), B pieces of this lane's groups.
    uint32_t voa[AG], vob[BG];
#pragma unroll
    for (int i = 0; i < AG; ++i) voa[i] = (uint32_t)(min(m0 + 16 * (wv * AG + i) + r16, M - 1) * K + 8 * j4) * 2;
#pragma unroll
    for (int i = 0; i < BG; ++i) vob[i] = (uint32_t)(((wv * BG + i) * kTileElems + lane * 8) * 2);
    const char* abase = (const char*)Ag;
    const char* bbase = (const char*)Btile;
    // The loads of step t come from two wave-uniform global bases (A and B of
    // that step) and land in stage t % STG.  Past the last step the global
    // bases stay at the last step (the data then lands in a stage no later
    // step reads), so every step issues the same loads: the wait counts below
    // are constants and no branch sits between the MFMAs.
    struct StepAddr {
      const char* ga;
      const char* gb;
      uint32_t la;
    };
    auto step_addr = [&](int t) {
      const int tc = min(t, KT - 1);
      return StepAddr{abase + (size_t)(tc * BKS) * 2, Q4 ? nullptr : bbase + tblk(kslice0 + tc * BKS) * 2,
                      lds_base + (uint32_t)((t % STG) * STS) * 2};
    };
    // direct load number idx (0 .. LPS-1) of a step: 32-column block
    // idx / (AG + BG); inside a block, A and B groups alternate while both
    // last (A on even numbers), then the remaining B groups.  (A 32-wide K step
    // starting on a multiple of 64 keeps the next 32 columns in the same
    // 256-column chunk: B 1 KB further, A 64 bytes.)
    // (Q4) codes: lane l of wavefront w brings row n0 + 64 w + l, the 32 codes
    // of the step (16 bytes); pairs: the group's [N] row of transposed pairs,
    // rows n0 .. n0+255 (1 KB, 4 rows per lane)
    const int kw = K / 8;                                    // code words per row
    const uint32_t voc = Q4 ? (uint32_t)((n0 + 64 * wv + lane) * kw) * 4 : 0u;
    const char* cbase = Q4 ? (const char*)a.q4w : nullptr;
    const char* pbase = Q4 ? (const char*)(a.q4sb + n0) : nullptr;
    auto issue_at = [&](const StepAddr& sa, int idx) {
      if constexpr (Q4) {
        // (a step past the last one repeats the last step's loads: sa.ga)
        const int kc = (int)((sa.ga - abase) / 2) + kslice0;   // first column of the step
        if (idx < AG)
          lds_dma16(voa[idx], sa.ga, sa.la + (wv * AG + idx) * 1024);
        else if (idx == AG)
          lds_dma16(voc, cbase + (size_t)(kc / 8) * 4, sa.la + (SA + SB) * 2 + wv * 1024);
        else
          lds_dma16((uint32_t)lane * 16, pbase + (size_t)(kc / 64) * a.N * 4, sa.la + (SA + SB + SC) * 2 + wv * 1024);
        return;
      }
      const int kb = idx / (AG + BG), q = idx % (AG + BG);
      const bool is_a = q < 2 * AG && (q & 1) == 0;
      const int i = q < 2 * AG ? q >> 1 : q - AG;
      if (is_a)
        lds_dma16(voa[i], sa.ga + kb * 64, sa.la + (kb * (BM / 16) + wv * AG + i) * 1024);
      else
        lds_dma16(vob[i], sa.gb + kb * 1024, sa.la + SA * 2 + (kb * 16 + wv * BG + i) * 1024);
    };
    // lane's piece inside a pair of groups: fragment rows 32t + l%32, k = 8*(l/32)
    const int fpiece = (16 * (lane >> 5) + r16) * 8 + ((lane >> 4) & 1) * 512;
    // Fragment reads go in the order A0, B0, B1, B2, B3, A1 .. A(MI-1), the
    // order the MFMAs of a sub-step first need them (MFMA q takes A q/4, B q%4).
    // Read number r (0 .. MI+3): A0 at 0, B j at 1 + j, A i at 4 + i.
    auto lfrag_one = [&](int st, int kk, int r, uint4(&a_)[MI], uint4(&b_)[4]) {
      const bf16_t* la = lds + st * STS + fpiece + (kk & 1) * 256;
      const bool is_a = r == 0 || r > 4;
      const int i = r == 0 ? 0 : r - 4, j = r - 1;
      if (is_a) a_[i] = ld16(la + (kk >> 1) * (BM / 16) * 512 + (wm * (WTM / 16) + 2 * i) * 512);
      else b_[j] = ld16(la + SA + (kk >> 1) * 16 * 512 + (wn * 8 + 2 * j) * 512);
    };
    constexpr int NF = MI + 4;                 // fragment reads per sub-step
    constexpr int NM = MI * 4;                 // MFMAs per sub-step
    static_assert(NM >= NF, "interleave slots");
    // Before MFMA q of a sub-step whose slots issue the next sub-step's reads:
    // its two fragments (read during the previous sub-step) must have landed,
    // while the reads after them and the min(q, NF) reads this sub-step has
    // issued so far may still be in flight (LDS reads complete in order).
    // (Q4: the B tile built in slot NF adds 6 LDS operations after it.)
    auto frag_wait = [](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int ra = q / 4 == 0 ? 0 : 4 + q / 4, rb = 1 + q % 4;
      constexpr int need = ra > rb ? ra : rb;
      constexpr int later = (NF - 1 - need) + (q < NF ? q : NF) + (Q4 && q > NF ? 6 : 0);
      static_assert(later >= 0 && later < 16, "lgkm count");
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (later << 8) | (3 << 14));
    };
    // The MFMAs of one sub-step, with one other instruction slotted in after
    // each: while an MFMA runs the wavefront issues the next load, so the
    // matrix core is never left waiting on an issue.  STAGGER: each MFMA waits
    // only for its own fragments (else the caller waited for all of them).
    auto mfmas_with = [&](const uint4(&a_)[MI], const uint4(&b_)[4], auto&& slot, auto stagger) {
      static_for<0, NM>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (decltype(stagger)::value) frag_wait(qc);
        if constexpr (F16)
          acc[q / 4][q % 4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(u4_as_f16x8(a_[q / 4]), u4_as_f16x8(b_[q % 4]),
                                                                     acc[q / 4][q % 4], 0, 0, 0);
        else
          acc[q / 4][q % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u4_as_bf16x8(a_[q / 4]),
                                                                      u4_as_bf16x8(b_[q % 4]), acc[q / 4][q % 4], 0, 0, 0);
        slot(q);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // (Q4) B tile of step t from its codes and pairs in stage t % STG: thread
    // tid owns row tid, whose fp16 s * q + b for columns 8j .. 8j+7 form piece
    // 16 j + tid % 16 of the 1 KB block of row group tid / 16 (the layout of
    // the direct-loaded tiles).  Only this wavefront's own loads are read, so
    // its vmcnt wait suffices (no barrier).
    auto dequant_b = [&](int t) {
      if constexpr (Q4) {
        const int sti = t % STG;
        const bf16_t* sb0 = lds + sti * STS + SA + SB;
        const uint4 cw = ld16(sb0 + tid * 8);
        const uint32_t pr = *reinterpret_cast<const uint32_t*>(sb0 + SC + wv * 512 + tid * 2);
        // Packed fp16: the codes of columns 2e and 2e + 1 become the fp16
        // pair (1024 + q0, 1024 + q1) by placing each code in the low
        // mantissa bits of 1024.0 (bit pattern 0x6400); subtracting 1024 is
        // exact, and one fused multiply-add per pair gives s q + b rounded
        // once to fp16 (s and b, bf16 values, are exact in fp16 inside its
        // normal range).  About 2.4 instructions per code.
        const _Float16 s16 = (_Float16)bf16_to_f32((bf16_t)(pr & 0xffffu));
        const _Float16 b16 = (_Float16)bf16_to_f32((bf16_t)(pr >> 16));
        const f16x2 sv = {s16, s16}, bv = {b16, b16}, k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
        bf16_t* dst = lds + sti * STS + SA + (tid >> 4) * 512 + (tid & 15) * 8;
        const uint32_t w4[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // even-column codes in the bytes of lo, odd-column codes in those of hi
          const uint32_t lo = w4[j] & 0x0f0f0f0fu, hi = (w4[j] >> 4) & 0x0f0f0f0fu;
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // byte e of lo -> byte 0, byte e of hi -> byte 2, zero bytes 1 and 3
            const uint32_t sel = (uint32_t)e | (0x0cu << 8) | ((uint32_t)(4 + e) << 16) | (0x0cu << 24);
            const uint32_t x = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
            const f16x2 q = __builtin_bit_cast(f16x2, x) - k1024;
            o[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, sv, bv));
          }
          st16(dst + j * 128, make_uint4(o[0], o[1], o[2], o[3]));
        }
      }
    };
    uint4 fa[2][MI], fb[2][4];
#pragma unroll
    for (int t = 0; t < STG; ++t) {
      const StepAddr sa = step_addr(t);
#pragma unroll
      for (int idx = 0; idx < LPS; ++idx) issue_at(sa, idx);
    }
    // step 0 landed: the other STG - 1 steps may still be in flight; (Q4)
    // step 0's B tile, then every wavefront's writes complete before the barrier
    wait_vmcnt<(STG - 1) * LPS>();
    if constexpr (Q4) {
      dequant_b(0);
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    }
    asm volatile("s_barrier" ::: "memory");
    // nothing but LDS reads may be pending on the lgkm counter inside the loop
    // (a scalar load in flight would force every fragment wait to lgkmcnt(0))
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    for (int q = 0; q < NF; ++q) lfrag_one(0, 0, q, fa[0], fb[0]);
    // A sub-step before the last of step kt: its fragments were read during
    // the previous sub-step, and each MFMA waits for its own; its slots read the
    // next sub-step's.
    // (Q4) The first sub-step of step kt also builds the B tile of step kt+1
    // (its stage was freed by the barrier of step kt+1-STG; the barrier of step
    // kt's last sub-step publishes it): wait for that step's own loads (those of
    // the STG-2 later steps may still be in flight), then dequantize in the
    // slots after the fragment reads.
    // SPREAD: a step's direct loads are not issued together right after the
    // barrier, where the four wavefronts it releases would all hand theirs to
    // the address unit at once (and an MFMA stuck behind a load that cannot
    // issue leaves the matrix core idle): LPS1 of them go out in the last
    // sub-step, the rest on every other slot of the next step's first
    // sub-step from SLOT0 (measured on 256-row tiles: 2 after the barrier and 6
    // spread beat 4 + 4, 0 + 8 and all 8 together).  The barrier's wait still
    // finds the loads of the two steps after the one it waits for issued, so
    // its count is unchanged; (Q4) the first sub-step's wait for the next step
    // finds the step after that issued and only LPS1 loads of the one after.
    constexpr bool SPREAD = NKK == 2 && ((MI == 4 && NM == 2 * NF) || MI == 2);
    constexpr int LPS1 = SPREAD ? 2 : LPS;
    constexpr int SLOT0 = MI == 4 ? 5 : 1;
    auto sub_first = [&](int kt, auto kc, auto with_loads) {
      constexpr int kk = decltype(kc)::value;
      constexpr int cur = kk & 1;
      const int st = kt % STG;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (Q4 && kk == 0) wait_vmcnt<SPREAD ? (STG - 3) * LPS + LPS1 : (STG - 2) * LPS>();
      // (SPREAD: the rest of step kt-1+STG's loads)
      [[maybe_unused]] StepAddr sa{};
      if constexpr (SPREAD && decltype(with_loads)::value) sa = step_addr(kt - 1 + STG);
      mfmas_with(fa[cur], fb[cur], [&](int slot) {
        if (slot < NF) lfrag_one(st, kk + 1, slot, fa[cur ^ 1], fb[cur ^ 1]);
        if constexpr (SPREAD && kk == 0 && decltype(with_loads)::value) {
          if (slot >= SLOT0 && ((slot - SLOT0) & 1) == 0 && LPS1 + (slot - SLOT0) / 2 < LPS)
            issue_at(sa, LPS1 + (slot - SLOT0) / 2);
        }
        if constexpr (Q4 && kk == 0) {
          if (slot == NF) dequant_b(kt + 1);
        }
      }, std::true_type{});
    };
    // The last sub-step of step kt: every read of stage st completes before the
    // barrier that lets the other wavefronts refill it, and step kt+1 has
    // landed (steps kt+2 .. kt+STG-1 may still be in flight; after the last
    // step this waits for nothing and reads an unused stage, kept unconditional
    // so the reads stay in one straight line).  Its slots read step kt+1's first
    // fragments, then issue the direct loads of step kt+STG into stage st.
    auto sub_last = [&](int kt) {
      constexpr int cur = (NKK - 1) & 1;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
      wait_vmcnt<(STG - 2) * LPS>();
      asm volatile("s_barrier" ::: "memory");
      const int nxt = (kt + 1) % STG;
      const StepAddr sa = step_addr(kt + STG);
      __builtin_amdgcn_sched_barrier(0);
      mfmas_with(fa[cur], fb[cur], [&](int slot) {
        if constexpr (SPREAD && MI == 4) {
          // reads on the even slots, the two loads on slots 1 and 9
          if ((slot & 1) == 0) lfrag_one(nxt, 0, slot / 2, fa[cur ^ 1], fb[cur ^ 1]);
          else if (slot == 1 || slot == 9) issue_at(sa, slot / 8);
        } else {
          if (slot < NF) lfrag_one(nxt, 0, slot, fa[cur ^ 1], fb[cur ^ 1]);
          else if (slot - NF < LPS1) issue_at(sa, slot - NF);
        }
      }, std::false_type{});
      if constexpr (!SPREAD) {
#pragma unroll
        for (int idx = NM - NF; idx < LPS; ++idx) issue_at(sa, idx);
      }
      static_assert(!SPREAD || (MI == 4 ? LPS1 == 2 : LPS1 <= NM - NF), "loads after the barrier");
    };
    // The loop body runs from one step's last sub-step into the next step's
    // leading ones, so the staggered waits sit in straight-line code (at a loop
    // head the compiler would merge them into a full wait).
    static_for<0, NKK - 1>([&](auto kc) { sub_first(0, kc, std::false_type{}); });
    for (int kt = 0; kt + 1 < KT; ++kt) {
      sub_last(kt);
      static_for<0, NKK - 1>([&](auto kc) { sub_first(kt + 1, kc, std::true_type{}); });
    }
    sub_last(KT - 1);
    // the loads issued past the last step land in LDS the epilogue reuses
    wait_vmcnt<0>();
  } else if constexpr (DEPTH == 2) {
    const int KT = Kslice / BK;
    gload(0, ra0, rb0);
    if (KT > 1) gload(1, ra1, rb1);
    for (int kt = 0; kt < KT; kt += 2) {
      lstore(0, ra0, rb0);
      __syncthreads();
      if (kt + 2 < KT) gload(kt + 2, ra0, rb0);
      compute(0);
      if (kt + 1 < KT) {
        lstore(1, ra1, rb1);
        __syncthreads();
        if (kt + 3 < KT) gload(kt + 3, ra1, rb1);
        compute(1);
      }
    }
  } else {
    const int KT = Kslice / BK;
    gload(0, ra0, rb0);
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      lstore(buf, ra0, rb0);
      __syncthreads();
      if (kt + 1 < KT) gload(kt + 1, ra0, rb0);
      compute(buf);
    }
  }

  // ---------------- epilogue: lane holds column l32 of each 32x32 subtile,
  // rows 8*(r/4) + 4*hg + r%4 for register r.  Results go through a per-wave
  // LDS staging area, 32 rows at a time, so that global stores (and the
  // residual loads) are 16-byte pieces of contiguous rows.
  const int wcol0 = n0 + wn * 128;  // first column of this wavefront (head aligned)
  __syncthreads();                  // main-loop LDS is free
  // [0, 4 KB): per-row data (EPI_QKV, EPI_SWIGLU); then 17 KB per wavefront
  char* stage = reinterpret_cast<char*>(lds) + 4096 + wave * 17408;
  auto wave_sync = [&]() {
    // LDS accesses of one wavefront complete in order once waited for
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  // RMSNorm row scales of the block's rows into s_rs[BM] (the caller
  // synchronizes): from inv_rms, or reduced from the producer's partial sums of
  // squares, every partial of a row requested at once and summed in order
  auto row_scales = [&](float* s_rs) {
    for (int r = tid; r < BM; r += NT) {
      const int row = m0 + r, rr = min(row, M - 1);
      float v;
      if (a.inv_rms) {
        v = a.inv_rms[rr];
      } else {
        const RowStat& st = a.rstat;
        float p[kGemmMaxRowPartials];
#pragma unroll
        for (int j = 0; j < kGemmMaxRowPartials; ++j) p[j] = st.ss[(size_t)min(j, st.nb - 1) * st.M + rr];
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < kGemmMaxRowPartials; ++j)
          if (j < st.nb) t += p[j];
        v = 1.0f / sqrtf(t / (float)st.n + st.eps);
      }
      s_rs[r] = row < M ? v : 0.f;
    }
  };
  if constexpr (EPI == EPI_QKV) {
    // Per-row data once per block: position, RMSNorm row scale and the element
    // offset of the row's page (bytes [0, 4 BM), [4 BM, 8 BM), [8 BM, 16 BM)).
    int* s_pos = reinterpret_cast<int*>(lds);
    float* s_rs = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + 4 * BM);
    long long* s_page = reinterpret_cast<long long*>(lds + 4 * BM);  // byte 8 BM: 8-byte aligned
    row_scales(s_rs);
    for (int r = tid; r < BM; r += NT) {
      const int row = m0 + r;
      if (row < M) {
        const int bseq = a.kv.seq_of_row(row, a.L);
        const int pos = a.kv.lens[bseq] + (row - a.kv.first_row(bseq, a.L));
        s_pos[r] = pos;
        s_page[r] = (long long)a.kv.page_base(bseq, pos);
      }
    }
    __syncthreads();
    const bool is_q = wcol0 < a.Nq;
    const bool is_k = !is_q && wcol0 < a.Nq + a.Nkv;
    const int ps = a.kv.ps;
    const int g = is_q ? 0 : (is_k ? (wcol0 - a.Nq) >> 7 : (wcol0 - a.Nq - a.Nkv) >> 7);
    bf16_t* sq = reinterpret_cast<bf16_t*>(stage);   // Q/K: [32 rows][136]; V: [128 dims][40]
    constexpr int QST = 136, VTS = 40;
    static_for<0, MI>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rb = wm * WTM + i * 32;   // block-local first row of this subtile
      // all of this subtile's row scales and rotation factors are requested
      // before any is used (one batch of loads in flight, not 32 round trips)
      float rsv[16];
      float2 csv[16][2];
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int lr = 8 * (r >> 2) + 4 * hg + (r & 3);
        const int row = m0 + rb + lr;
        const int pos = row < M ? s_pos[rb + lr] : 0;
        rsv[r] = s_rs[rb + lr];
        static_for<0, 2>([&](auto jc) {
          constexpr int jp = decltype(jc)::value;
          csv[r][jp] = (is_q || is_k) ? a.rope[(size_t)pos * 64 + jp * 32 + l32] : make_float2(1.f, 0.f);
        });
      });
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int lr = 8 * (r >> 2) + 4 * hg + (r & 3);   // row inside the subtile
        const float rs = rsv[r];
        static_for<0, 2>([&](auto jc) {
          constexpr int jp = decltype(jc)::value;
          const int pi = jp * 32 + l32;  // pair index: columns pi and pi + 64 of the head
          float x0 = acc[i][jp][r] * rs, x1 = acc[i][jp + 2][r] * rs;
          if (is_q || is_k) {
            const float2 cs = csv[r][jp];
            const float y0 = x0 * cs.x - x1 * cs.y;
            const float y1 = x1 * cs.x + x0 * cs.y;
            x0 = y0;
            x1 = y1;
          }
          const int ca = (is_q || is_k) && a.traditional ? 2 * pi : pi;
          const int cb = (is_q || is_k) && a.traditional ? 2 * pi + 1 : pi + 64;
          if (is_q || is_k) {
            sq[lr * QST + ca] = f32_to_bf16(x0);
            sq[lr * QST + cb] = f32_to_bf16(x1);
          } else {
            sq[ca * VTS + lr] = f32_to_bf16(x0);
            sq[cb * VTS + lr] = f32_to_bf16(x1);
          }
        });
      });
      wave_sync();
      if (is_q || is_k) {
        // 32 rows x 16 pieces of 8 columns
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = lane + 64 * t, lr = c >> 4, pc = c & 15;
          const int row = m0 + rb + lr;
          if (row < M) {
            const uint4 v = ld16(sq + lr * QST + 8 * pc);
            if (is_q) {
              st16(a.q_out + (size_t)row * a.Nq + wcol0 + 8 * pc, v);
            } else {
              bf16_t* kb = (bf16_t*)a.kv.k + s_page[rb + lr] + (size_t)g * ps * 128;
              st16(kb + kv_tiled_k(s_pos[rb + lr] % ps, 8 * pc), v);
            }
          }
        }
      } else {
        // 128 dims x 4 pieces of 8 tokens; a piece whose 8 rows are 8 consecutive
        // 8-aligned positions of one sequence and page is one 16-byte store
        bf16_t* Vc = (bf16_t*)a.kv.v;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = lane + 64 * t, dd = c >> 2, p8 = c & 3;
          const int lr0 = 8 * p8, row0 = m0 + rb + lr0;
          if (row0 >= M) continue;
          const int p0 = s_pos[rb + lr0];
          const bool vec = row0 + 7 < M && (p0 & 7) == 0 && s_pos[rb + lr0 + 7] == p0 + 7 &&
                           s_page[rb + lr0 + 7] == s_page[rb + lr0];
          if (vec) {
            st16(Vc + s_page[rb + lr0] + (size_t)g * 128 * ps + kv_tiled_v(p0 % ps, dd), ld16(sq + dd * VTS + lr0));
          } else {
            for (int e = 0; e < 8 && row0 + e < M; ++e)
              Vc[s_page[rb + lr0 + e] + (size_t)g * 128 * ps + kv_tiled_v(s_pos[rb + lr0 + e] % ps, dd)] =
                  sq[dd * VTS + lr0 + e];
          }
        }
      }
      wave_sync();
    });
  } else if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hg + (r & 3);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a.C[(size_t)ksi * M * N + (size_t)row * N + wcol0 + j * 32 + l32] = acc[i][j][r];
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    float* sf = reinterpret_cast<float*>(stage);   // [32 rows][132] fp32
    constexpr int FST = 132;
    // the residual pieces of subtile i (piece t: row (lane + 64 t) / 16, 8
    // columns at 8 ((lane + 64 t) % 16); rows past M read row M - 1, unused).
    // Subtile i + 1's pieces are requested before subtile i's stores: loads and
    // stores share one counter, so waiting for them then never waits for the
    // stores' completion.
    uint4 rres[2][8];
    auto load_resid = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rb = wm * WTM + i * 32;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = lane + 64 * t, lr = c >> 4, pc = c & 15;
        const int row = min(m0 + rb + lr, M - 1);
        rres[i & 1][t] = ld16(a.resid + (size_t)row * N + wcol0 + 8 * pc);
      }
    };
    load_resid(std::integral_constant<int, 0>{});
    static_for<0, MI>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rb = wm * WTM + i * 32;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int lr = 8 * (r >> 2) + 4 * hg + (r & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) sf[lr * FST + j * 32 + l32] = acc[i][j][r];
      });
      wave_sync();
      if constexpr (i + 1 < MI) load_resid(std::integral_constant<int, i + 1>{});
      // 32 rows x 16 pieces of 8 columns: out = resid + acc, rounded once
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = lane + 64 * t, lr = c >> 4, pc = c & 15;
        const int row = m0 + rb + lr;
        float ssq = 0.f;
        if (row < M) {
          const size_t idx = (size_t)row * N + wcol0 + 8 * pc;
          const float4 f0 = *reinterpret_cast<const float4*>(sf + lr * FST + 8 * pc);
          const float4 f1 = *reinterpret_cast<const float4*>(sf + lr * FST + 8 * pc + 4);
          const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
          const uint4 rv = rres[i & 1][t];
          const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
          uint32_t ow[4], bw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float r0 = bf16_to_f32((bf16_t)(rw[e] & 0xffffu)), r1 = bf16_to_f32((bf16_t)(rw[e] >> 16));
            ow[e] = pack_bf16x2(r0 + f[2 * e], r1 + f[2 * e + 1]);
            bw[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
          }
          st16(a.out + idx, make_uint4(ow[0], ow[1], ow[2], ow[3]));
          if (a.branch) st16(a.branch + idx, make_uint4(bw[0], bw[1], bw[2], bw[3]));
          if (a.ss_out) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float o0 = __builtin_bit_cast(float, ow[e] << 16);
              const float o1 = __builtin_bit_cast(float, ow[e] & 0xffff0000u);
              ssq += o0 * o0 + o1 * o1;
            }
          }
        }
        if (a.ss_out) {
          // the row's 16 pieces sit in 16 consecutive lanes: sum them, in a
          // fixed order, and the first lane writes this 128-column block's partial
          float v = ssq;
          v += __shfl_xor(v, 1, 64);
          v += __shfl_xor(v, 2, 64);
          v += __shfl_xor(v, 4, 64);
          v += __shfl_xor(v, 8, 64);
          if (pc == 0 && row < M) a.ss_out[(size_t)(wcol0 >> 7) * M + row] = v;
        }
      }
      wave_sync();
    });
  } else if constexpr (EPI == EPI_SWIGLU) {
    bf16_t* sg = reinterpret_cast<bf16_t*>(stage);   // [32 rows][72] bf16: this wave's 64 g columns
    constexpr int GST = 72;
    const int F = N >> 1;
    // interleave blocks of 32: columns wcol0 + 64*jp .. +31 are w1 rows, the
    // next 32 the matching w3 rows; this wave's g columns start at wcol0 / 2
    const int gcol0 = wcol0 >> 1;
    float* s_rs = reinterpret_cast<float*>(lds);   // [BM] (below the staging areas)
    row_scales(s_rs);
    __syncthreads();
    static_for<0, MI>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rb = wm * WTM + i * 32;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int lr = 8 * (r >> 2) + 4 * hg + (r & 3);
        const float rs = s_rs[rb + lr];
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const float gt = acc[i][2 * jp][r] * rs, up = acc[i][2 * jp + 1][r] * rs;
          sg[lr * GST + jp * 32 + l32] = f32_to_bf16(silu_f(gt) * up);
        }
      });
      wave_sync();
      // 32 rows x 8 pieces of 8 g columns
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = lane + 64 * t, lr = c >> 3, pc = c & 7;
        const int row = m0 + rb + lr;
        if (row < M) st16(a.g_out + (size_t)row * F + gcol0 + 8 * pc, ld16(sg + lr * GST + 8 * pc));
      }
      wave_sync();
    });
  }
  if constexpr (EPI == EPI_RESID) {
    if (a.lens_add && blockIdx.x == 0 && tid < a.n_seq)
      a.lens_add[tid] += a.lens_cu ? a.lens_cu[tid + 1] - a.lens_cu[tid] : a.lens_inc;
  }
}

template <int BM, int BN, int NW, int DEPTH, int EPI, bool F16, bool Q4 = false>
static void launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int ncols = (a.n_hi > 0 ? a.n_hi : a.N) - a.n_lo;
  const int tiles = ((a.M + BM - 1) / BM) * (ncols / BN) * (EPI == EPI_F32 && a.ksplit > 1 ? a.ksplit : 1);
  const size_t lds = Q4 ? (size_t)4 * ((BM + BN) * 32 + BN * 8 + NW * BN * 2) * sizeof(bf16_t)
                     : DEPTH == 4 ? (size_t)(BM + BN) * 160 * sizeof(bf16_t)
                     : DEPTH == 0 || DEPTH == 3 ? std::max<size_t>((size_t)(BM + BN) * 128 * sizeof(bf16_t), 4096 + 4 * 17408)
                                : (size_t)2 * (BM + BN) * gm::LDS_ST * sizeof(bf16_t);
  if (plan_log_on())
    plan_log("gemm M %d N %d K %d cols [%d, %d): %dx%d tiles, %d waves, %s, split-K %d, epilogue %d%s, %d blocks",
             a.M, a.N, a.K, a.n_lo, a.n_hi > 0 ? a.n_hi : a.N, BM, BN, NW,
             DEPTH == 0 ? "direct-to-LDS 4-stage ring" : "register-staged", a.ksplit > 0 ? a.ksplit : 1, EPI,
             Q4 ? ", 4-bit B dequantized in LDS" : F16 ? ", fp16" : "", tiles);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_mfma<BM, BN, NW, DEPTH, EPI, F16, Q4>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  hipExtLaunchKernelGGL((k_gemm_mfma<BM, BN, NW, DEPTH, EPI, F16, Q4>), dim3(tiles), dim3(NW * 64), lds, s,
                        g_clock.start, g_clock.stop, 0, a);
  g_clock = LaunchClock{};
}

// Rounds of 256 blocks, 128-row tiles counted at 0.6 of a 256-row round (half
// the work each, 20% dearer: measured).  Returns the 256-column tile columns
// to run as 256-row tiles before the rest run as 128-row tiles (0: one shape),
// the split that ends soonest when the 256-row grid leaves a partial round;
// `cost` is its time in rounds.
static int gemm_two_shapes(int M, int N, double& cost) {
  const long tm2 = (M + 255) / 256, tm1 = (M + 127) / 128, tn = N / 256;
  auto rounds = [](long t) { return (double)((t + 255) / 256); };
  const double c256 = rounds(tm2 * tn), c128 = 0.6 * rounds(tm1 * tn);
  cost = std::min(c256, c128);
  int best = 0;
  // the first launch: the tile columns that fill r whole rounds
  for (long r = 1; r * 256 < tm2 * tn; ++r) {
    const long nb = r * 256 / tm2;
    if (nb <= 0 || nb >= tn) continue;
    const double c = rounds(nb * tm2) + 0.6 * rounds((tn - nb) * tm1);
    if (c < cost - 1e-9) {
      cost = c;
      best = (int)nb;
    }
  }
  return best;
}

// Tile choice: the direct-to-LDS ring where the shape allows, 128-row tiles
// when their rounds of 256 blocks finish sooner than those of 256-row tiles,
// and both (two launches over disjoint columns) when the 256-row grid's last
// round would run part empty and the split ends sooner; register-staged tiles
// otherwise.
template <int EPI, bool F16>
static void launch_epi(const GemmArgs& a, hipStream_t s) {
  const bool n256 = (a.N % 256) == 0;
  if constexpr (F16) {
    if (a.q4w) {
      // 4-bit B dequantized in the kernel (gemm_q4_direct_ok shapes), fp16 A.
      // 256-row tiles unless the rounds of 256 blocks of 128-row tiles end
      // sooner (a 128-row round counted at 0.6 of a 256-row one, as measured
      // for bf16; the B tile's dequantization favours the taller tile further)
      const long t256 = (long)((a.M + 255) / 256) * (a.N / 256), t128 = (long)((a.M + 127) / 128) * (a.N / 256);
      const bool use128 = ((t128 + 255) / 256) * 0.6 < (double)((t256 + 255) / 256);
      if ((EPI == EPI_F32 && a.ksplit > 1) || !use128) return launch_cfg<256, 256, 4, 0, EPI, true, true>(a, s);
      return launch_cfg<128, 256, 4, 0, EPI, true, true>(a, s);
    }
    if (a.a_f16) {
      // fp16 A and tiled fp16 B (gemm_f16_direct_ok): direct-to-LDS tiles,
      // the tile height chosen as for bf16
      const long t256 = (long)((a.M + 255) / 256) * (a.N / 256), t128 = (long)((a.M + 127) / 128) * (a.N / 256);
      const bool use128 = ((t128 + 255) / 256) * 0.6 < (double)((t256 + 255) / 256);
      if ((EPI == EPI_F32 && a.ksplit > 1) || (t256 >= 240 && !use128)) return launch_cfg<256, 256, 4, 0, EPI, true>(a, s);
      return launch_cfg<128, 256, 4, 0, EPI, true>(a, s);
    }
  }
  if constexpr (!F16) {
    // direct-to-LDS tiles address A with 32-bit per-lane byte offsets
    const bool a32 = (size_t)a.M * a.K * sizeof(bf16_t) < ((size_t)1 << 32);
    const bool big = a32 && n256 && (EPI == EPI_F32 && a.ksplit > 1 || ((a.M + 255) / 256) * (a.N / 256) >= 240);
    // 128-row tiles when their rounds of 256 blocks finish sooner (half the
    // work each, counted 20% dearer: measured) than those of 256-row tiles
    const long t256 = (long)((a.M + 255) / 256) * (a.N / 256), t128 = (long)((a.M + 127) / 128) * (a.N / 256);
    const bool use128 = ((t128 + 255) / 256) * 0.6 < (double)((t256 + 255) / 256);
    if (big && !(EPI == EPI_F32 && a.ksplit > 1) && a.n_hi == 0) {
      double cost;
      const int nb = gemm_two_shapes(a.M, a.N, cost);
      if (nb > 0) {
        // (a launch clock brackets both launches; block 0 of the first alone
        // advances the lengths)
        const LaunchClock clk = g_clock;
        GemmArgs a1 = a, a2 = a;
        a1.n_hi = nb * 256;
        a2.n_lo = nb * 256;
        a2.lens_add = nullptr;
        g_clock = LaunchClock{clk.start, nullptr};
        launch_cfg<256, 256, 4, 0, EPI, F16>(a1, s);
        g_clock = LaunchClock{nullptr, clk.stop};
        launch_cfg<128, 256, 4, 0, EPI, F16>(a2, s);
        return;
      }
    }
    if (big && use128 && !(EPI == EPI_F32 && a.ksplit > 1)) return launch_cfg<128, 256, 4, 0, EPI, F16>(a, s);
    if (!big && a32 && n256 && t128 >= 240 && !(EPI == EPI_F32 && a.ksplit > 1))
      return launch_cfg<128, 256, 4, 0, EPI, F16>(a, s);
    if (big) return launch_cfg<256, 256, 4, 0, EPI, F16>(a, s);
  }
  if (EPI == EPI_F32 && a.ksplit > 1) return launch_cfg<256, 256, 8, 2, EPI, F16>(a, s);
  // register-staged: the largest tile that still gives about one wave of blocks per CU
  const long t256 = (long)((a.M + 255) / 256) * (a.N / 256);
  if (n256 && t256 >= 240) return launch_cfg<256, 256, 8, 2, EPI, F16>(a, s);
  if (n256) return launch_cfg<128, 256, 4, 2, EPI, F16>(a, s);
  return launch_cfg<128, 128, 4, 2, EPI, F16>(a, s);
}

template <bool F16>
static void launch_any(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_epi<EPI_F32, F16>(a, s);
    case EPI_QKV: return launch_epi<EPI_QKV, F16>(a, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU, F16>(a, s);
    default: return launch_epi<EPI_RESID, F16>(a, s);
  }
}

bool gemm_f16_direct_ok(int M, int N, int K) {
  return N % 256 == 0 && (size_t)M * K * sizeof(bf16_t) < ((size_t)1 << 32);
}

bool gemm_q4_direct_ok(int M, int N, int K) {
  return gemm_f16_direct_ok(M, N, K) && K % 64 == 0 && (size_t)N * K / 2 < ((size_t)1 << 32);
}

int gemm_split_k(int M, int N, int K, bool b_f16) {
  if (N % 256) return 1;
  const long t256 = (long)((M + 255) / 256) * (N / 256), t128 = (long)((M + 127) / 128) * (N / 256);
  // up to K = 8192, unsplit 128x256 direct-to-LDS tiles beat a 2-way split
  // once they fill the chip: the split's fp32 partials cost a round trip
  // of 2*M*N*4 bytes per slice (measured on 2048x4096x4096 and x11008)
  if (!b_f16 && t256 < 240 && t128 >= 240 && K <= 8192 && (size_t)M * K * sizeof(bf16_t) < ((size_t)1 << 32)) return 1;
  int ks = 1;
  // double while the grid is short of about 200 tiles and each slice keeps
  // at least 512 of K in whole 64-wide steps
  while (ks < kMaxSplitK && ks * t256 < 200 && K % (128 * ks) == 0 && K / (2 * ks) >= 512) ks *= 2;
  return ks;
}

int gemm_split_k_q4(int M, int N, int K) {
  if (N % 256) return 1;
  const long t256 = (long)((M + 255) / 256) * (N / 256);
  if (t256 >= 200) return 1;
  // The most slices that keep the grid within one round of 256 blocks, each
  // slice whole 64-column groups and at least 512 columns: the per-step
  // dequantization is paid once per block whatever its row count, so filling
  // the chip with slices of 256-row tiles beats fewer, longer blocks.
  int best = 1;
  for (int ks = 2; ks <= kMaxSplitKQ4; ++ks)
    if (ks * t256 <= 256 && K % (64 * ks) == 0 && K / ks >= 512) best = ks;
  return best;
}

void launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return;
  if (a.b_f16) launch_any<true>(epi, a, s);
  else launch_any<false>(epi, a, s);
}

}  // namespace lb

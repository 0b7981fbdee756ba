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

// s_waitcnt with only the vector-memory counter constrained (vmcnt <= n)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at LDS byte address lds_addr + 16 l (lds_addr wave-uniform, passed in M0).
// Written as inline asm so that the compiler, which cannot tell the stages of
// the ring apart, does not make every LDS read wait for every load in flight;
// the kernel waits on the vector-memory counter itself (wait_vmcnt) before the
// barrier that publishes a stage.  The instruction has no register result: its
// address registers are read at issue.  M0 is set in the same statement.
// Address = sbase (wave-uniform, scalar registers) + voff (per lane, 32-bit).
__device__ __forceinline__ void lds_dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

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
template <int BM, int BN, int NW, int DEPTH, int EPI, bool F16>
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
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
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
  const int m0 = tm * BM, n0 = tn * BN;

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
    constexpr int LPS = (BM / 64 + 4) * NKB;           // direct loads per wavefront per step
    static_assert((!F16 || DEPTH == 0) && NW == 4 && BN == 256 && (BM == 256 || (BM == 128 && DEPTH == 0)),
                  "direct-LDS configuration");
    constexpr int AG = BM / 64, BG = 4;                // A and B row groups each wavefront loads
    constexpr int SA = BM * BKS, SB = BN * BKS;        // bf16 per stage
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
    // direct load number idx (0 .. LPS-1) of step kt: 32-column block
    // idx / (AG + BG); inside a block, A and B groups alternate while both
    // last (A on even numbers), then the remaining B groups
    auto issue_one = [&](int kt, int idx) {
      const uint32_t la = lds_base + (uint32_t)((kt % STG) * (SA + SB)) * 2;
      const int kb = idx / (AG + BG), q = idx % (AG + BG);
      const bool is_a = q < 2 * AG && (q & 1) == 0;
      const int i = q < 2 * AG ? q >> 1 : q - AG;
      if (is_a)
        lds_dma16(voa[i], abase + (size_t)(kt * BKS + kb * 32) * 2, la + (kb * (BM / 16) + wv * AG + i) * 1024);
      else
        lds_dma16(vob[i], bbase + tblk(kslice0 + kt * BKS + kb * 32) * 2, la + SA * 2 + (kb * 16 + wv * BG + i) * 1024);
    };
    // lane's piece inside a pair of groups: fragment rows 32t + l%32, k = 8*(l/32)
    const int fpiece = (16 * (lane >> 5) + r16) * 8 + ((lane >> 4) & 1) * 512;
    // fragment read number q (0 .. MI+3): A tile q, or B tile q - MI
    auto lfrag_one = [&](int st, int kk, int q, uint4(&a_)[MI], uint4(&b_)[4]) {
      const bf16_t* la = lds + st * (SA + SB) + fpiece + (kk & 1) * 256;
      if (q < MI) a_[q] = ld16(la + (kk >> 1) * (BM / 16) * 512 + (wm * (WTM / 16) + 2 * q) * 512);
      else b_[q - MI] = ld16(la + SA + (kk >> 1) * 16 * 512 + (wn * 8 + 2 * (q - MI)) * 512);
    };
    // wait until this wavefront's loads of step t have landed, given the steps
    // issued up to step `last`
    auto wait_step = [&](int t, int last) {
      const int later = max(0, min(STG - 1, last - t));
      if constexpr (STG > 4) {
        if (later >= 4) return wait_vmcnt<4 * LPS>();
      }
      if constexpr (STG > 3) {
        if (later >= 3) return wait_vmcnt<3 * LPS>();
      }
      if constexpr (STG > 2) {
        if (later >= 2) return wait_vmcnt<2 * LPS>();
      }
      if (later >= 1) return wait_vmcnt<LPS>();
      wait_vmcnt<0>();
    };
    constexpr int NF = MI + 4;                 // fragment reads per sub-step
    constexpr int NM = MI * 4;                 // MFMAs per sub-step
    static_assert(NM >= NF, "interleave slots");
    // The MFMAs of one sub-step, with one other instruction slotted in after
    // each: while an MFMA runs the wavefront issues the next load, so the
    // matrix core is never left waiting on an issue.
    auto mfmas_with = [&](const uint4(&a_)[MI], const uint4(&b_)[4], auto&& slot) {
      static_for<0, NM>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
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
    uint4 fa[2][MI], fb[2][4];
#pragma unroll
    for (int t = 0; t < STG; ++t)
      if (t < KT) {
#pragma unroll
        for (int idx = 0; idx < LPS; ++idx) issue_one(t, idx);
      }
    int last = min(STG, KT) - 1;
    wait_step(0, last);
    asm volatile("s_barrier" ::: "memory");
    // nothing but LDS reads may be pending on the lgkm counter inside the loop
    // (a scalar load in flight would force every fragment wait to lgkmcnt(0))
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    for (int q = 0; q < NF; ++q) lfrag_one(0, 0, q, fa[0], fb[0]);
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt % STG;
      static_for<0, NKK>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        constexpr int cur = kk & 1;
        // this sub-step's fragments were read during the previous one
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kk + 1 < NKK) {
          mfmas_with(fa[cur], fb[cur], [&](int slot) {
            if (slot < NF) lfrag_one(st, kk + 1, slot, fa[cur ^ 1], fb[cur ^ 1]);
          });
        } else {
          // (after the last step this waits for nothing and reads an unused
          // stage; kept unconditional so the reads stay in one straight line)
          wait_step(kt + 1, last);
          // this stage's fragment reads are complete (waited above); barrier:
          // every wavefront is done with stage st, and step kt+1 has landed
          asm volatile("s_barrier" ::: "memory");
          const bool refill = kt + STG < KT;
          const int nxt = (kt + 1) % STG;
          __builtin_amdgcn_sched_barrier(0);
          // slots: fragment reads of step kt+1 first (needed soonest), then the
          // direct loads of step kt+STG into stage st
          mfmas_with(fa[cur], fb[cur], [&](int slot) {
            if (slot < NF) lfrag_one(nxt, 0, slot, fa[cur ^ 1], fb[cur ^ 1]);
            else if (refill && slot - NF < LPS) issue_one(kt + STG, slot - NF);
          });
          if (refill) {
#pragma unroll
            for (int idx = NM - NF; idx < LPS; ++idx) issue_one(kt + STG, idx);
            last = kt + STG;
          }
        }
      });
    }
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
  // [0, 4 KB): per-row cache metadata (EPI_QKV); then 17 KB per wavefront
  char* stage = reinterpret_cast<char*>(lds) + 4096 + wave * 17408;
  auto wave_sync = [&]() {
    // LDS accesses of one wavefront complete in order once waited for
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (EPI == EPI_QKV) {
    // Per-row cache metadata once per block: position, and the element offset
    // of the row's page.
    int* s_pos = reinterpret_cast<int*>(lds);
    long long* s_page = reinterpret_cast<long long*>(lds + 4 * BM);  // 8-byte aligned
    for (int r = tid; r < BM; r += NT) {
      const int row = m0 + r;
      if (row < M) {
        const int bseq = row / a.L;
        const int pos = a.kv.lens[bseq] + (row - bseq * a.L);
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
        rsv[r] = row < M ? a.inv_rms[row] : 0.f;
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
      // 32 rows x 16 pieces of 8 columns: out = resid + acc, rounded once
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = lane + 64 * t, lr = c >> 4, pc = c & 15;
        const int row = m0 + rb + lr;
        if (row < M) {
          const size_t idx = (size_t)row * N + wcol0 + 8 * pc;
          const float4 f0 = *reinterpret_cast<const float4*>(sf + lr * FST + 8 * pc);
          const float4 f1 = *reinterpret_cast<const float4*>(sf + lr * FST + 8 * pc + 4);
          const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
          const uint4 rv = ld16(a.resid + idx);
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
    static_for<0, MI>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rb = wm * WTM + i * 32;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int lr = 8 * (r >> 2) + 4 * hg + (r & 3);
        const int row = m0 + rb + lr;
        const float rs = row < M ? a.inv_rms[row] : 0.f;
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
    if (a.lens_add && blockIdx.x == 0 && tid < a.n_seq) a.lens_add[tid] += a.lens_inc;
  }
}

template <int BM, int BN, int NW, int DEPTH, int EPI, bool F16>
static void launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * (a.N / BN) * (EPI == EPI_F32 && a.ksplit > 1 ? a.ksplit : 1);
  const size_t lds = DEPTH == 4 ? (size_t)(BM + BN) * 160 * sizeof(bf16_t)
                     : DEPTH == 0 || DEPTH == 3 ? std::max<size_t>((size_t)(BM + BN) * 128 * sizeof(bf16_t), 4096 + 4 * 17408)
                                : (size_t)2 * (BM + BN) * gm::LDS_ST * sizeof(bf16_t);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_mfma<BM, BN, NW, DEPTH, EPI, F16>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  hipExtLaunchKernelGGL((k_gemm_mfma<BM, BN, NW, DEPTH, EPI, F16>), dim3(tiles), dim3(NW * 64), lds, s,
                        g_clock.start, g_clock.stop, 0, a);
  g_clock = LaunchClock{};
}

// Tile choice; LLAMA_BLOCK_GEMM_TILE = "256x256d" (direct-to-LDS), "256x256w8",
// "256x256w4", "128x256w4" or "128x128w4" forces one (for measurements).
static int forced_tile() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("LLAMA_BLOCK_GEMM_TILE");
    v = 0;
    if (e) {
      if (!strcmp(e, "256x256w8")) v = 1;
      else if (!strcmp(e, "256x256w4")) v = 2;
      else if (!strcmp(e, "128x256w4")) v = 3;
      else if (!strcmp(e, "128x128w4")) v = 4;
      else if (!strcmp(e, "256x256d")) v = 5;
      else if (!strcmp(e, "256x256d64")) v = 6;
      else if (!strcmp(e, "256x256d5")) v = 7;
      else if (!strcmp(e, "128x256d")) v = 8;
    }
  }
  return v;
}

template <int EPI, bool F16>
static void launch_epi(const GemmArgs& a, hipStream_t s) {
  const bool n256 = (a.N % 256) == 0;
  const int f = forced_tile();
  if constexpr (F16) {
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
    if (f == 8 && a32 && n256) return launch_cfg<128, 256, 4, 0, EPI, F16>(a, s);
    if (f == 0 && big && use128 && !(EPI == EPI_F32 && a.ksplit > 1)) return launch_cfg<128, 256, 4, 0, EPI, F16>(a, s);
    if (f == 0 && !big && a32 && n256 && t128 >= 240 && !(EPI == EPI_F32 && a.ksplit > 1))
      return launch_cfg<128, 256, 4, 0, EPI, F16>(a, s);
    if (f == 6 && big) return launch_cfg<256, 256, 4, 3, EPI, F16>(a, s);
    if (f == 7 && big) return launch_cfg<256, 256, 4, 4, EPI, F16>(a, s);
    if ((f == 0 || f == 5) && big) return launch_cfg<256, 256, 4, 0, EPI, F16>(a, s);
  }
  if (EPI == EPI_F32 && a.ksplit > 1) return launch_cfg<256, 256, 8, 2, EPI, F16>(a, s);
  if (f == 1 && n256) return launch_cfg<256, 256, 8, 2, EPI, F16>(a, s);
  if (f == 2 && n256) return launch_cfg<256, 256, 4, 1, EPI, F16>(a, s);
  if (f == 3 && n256) return launch_cfg<128, 256, 4, 2, EPI, F16>(a, s);
  if (f == 4) return launch_cfg<128, 128, 4, 2, EPI, F16>(a, s);
  // default: the largest tile that still gives about one wave of blocks per CU
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

void launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return;
  if (a.b_f16) launch_any<true>(epi, a, s);
  else launch_any<false>(epi, a, s);
}

}  // namespace lb

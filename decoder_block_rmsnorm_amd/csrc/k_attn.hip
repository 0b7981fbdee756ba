// Causal grouped-query attention over the paged KV cache:
//   o[h] = softmax_j( q[h] . k[g][j] / sqrt(d) ) v[g][j],  j <= position,
//   g = h / (H / G)
// (LLaMAAttention of page 二 with its expand-then-reshape kv sharing; the causal
// rule of "5. 因果掩码" and the KV cache of "2. 注意力机制", MLX page).
//
//  * k_attn_simt         : one wavefront per (token, head), lanes over head_dim,
//                          online softmax over keys (fp32 path).
//  * k_attn_prefill_bf16 : flash-style prefill: 128 queries of one head per
//                          block, 64-key K / V tiles copied from the tiled pages
//                          into LDS by direct loads, S^T = K Q^T and O^T = V^T P^T
//                          on 32x32x16 bf16 MFMA, fp32 online softmax, the next
//                          tile's S interleaved with this tile's exponentials
//                          (the tiling idea credited to FlashAttention in
//                          "Transformer 块的内部结构" of the reading-notes page).
//  * k_attn_decode_bf16  : split-K decode: each wavefront streams a 256-key
//                          chunk of one (sequence, kv head) straight from the
//                          pages with 128-bit loads, serving up to 16 query heads
//                          of the group with 16x16x32 MFMA (more query heads: one
//                          wavefront per 16 of them); k_attn_merge combines
//                          the chunks with a log-sum-exp merge in a fixed order.
#include <type_traits>

#include "kernels.hpp"

namespace lb {

// ===========================================================================
// generic (fp32 path)
// ===========================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_attn_simt(const T* q, KVView kv, int M, int L, int H, int G, int d,
                                                   T* out) {
  int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (wid >= M * H) return;
  int h = wid % H;
  int m = wid / H;
  int b = kv.seq_of_row(m, L), l = m - kv.first_row(b, L);
  int g = h / (H / G);
  int pos = kv.lens[b] + l;
  const T* qr = q + (size_t)m * H * d + (size_t)h * d;
  const float scale = 1.0f / sqrtf((float)d);
  float q0 = lane < d ? Elt<T>::load(qr, lane) * scale : 0.f;
  float q1 = lane + 64 < d ? Elt<T>::load(qr, lane + 64) * scale : 0.f;
  const T* K = (const T*)kv.k;
  const T* V = (const T*)kv.v;
  float mx = -INFINITY, den = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = kv.window > 0 ? max(0, pos - kv.window + 1) : 0; j <= pos; ++j) {
    float part = 0.f;
    if (lane < d) part += q0 * Elt<T>::load(K, kv.k_off(b, j, g, lane));
    if (lane + 64 < d) part += q1 * Elt<T>::load(K, kv.k_off(b, j, g, lane + 64));
    float sc = warp_sum(part);
    float mn = fmaxf(mx, sc);
    float alpha = __expf(mx - mn);
    float p = __expf(sc - mn);
    den = den * alpha + p;
    float v0 = lane < d ? Elt<T>::load(V, kv.v_off(b, j, g, lane)) : 0.f;
    float v1 = lane + 64 < d ? Elt<T>::load(V, kv.v_off(b, j, g, lane + 64)) : 0.f;
    o0 = o0 * alpha + p * v0;
    o1 = o1 * alpha + p * v1;
    mx = mn;
  }
  T* orow = out + (size_t)m * H * d + (size_t)h * d;
  if (lane < d) Elt<T>::store(orow, lane, o0 / den);
  if (lane + 64 < d) Elt<T>::store(orow, lane + 64, o1 / den);
}

template <typename T>
void launch_attn_simt(const T* q, KVView kv, int M, int L, int H, int G, int d, T* out, hipStream_t s) {
  int waves = M * H;
  if (waves <= 0) return;
  hipLaunchKernelGGL(k_attn_simt<T>, dim3((waves + 3) / 4), dim3(256), 0, s, q, kv, M, L, H, G, d, out);
}

template void launch_attn_simt<float>(const float*, KVView, int, int, int, int, int, float*, hipStream_t);
template void launch_attn_simt<bf16_t>(const bf16_t*, KVView, int, int, int, int, int, bf16_t*, hipStream_t);

// ===========================================================================
// bf16 flash prefill, head_dim 128
// ===========================================================================
// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E), so that
// register arrays are indexed by constants.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for_fa(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for_fa<B + 1, E>(f);
  }
}

namespace fa {
constexpr int D = 128;
constexpr int BK = 64;         // keys per tile
constexpr int TB = BK * D * 2; // bytes of one K (or V) tile: one 64-slot block of a page
}  // namespace fa

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// One block per (head, sequence, query tile of 128), heavy (late) query tiles
// first; with `flip`, the second half of the grid's tiles light first, so that
// blocks z and z + n_qt / 2 of a head together take n_qt + 1 key tiles.
//
// A key tile is one 64-slot block of a page, 16 KB of K and 16 KB of V in the
// cache's tiled layout, copied into LDS as it is by direct loads (each
// wavefront instruction moves one contiguous kilobyte; no register staging).
// Two K and two V tiles are resident: during step t the block holds K(t+1)
// and V(t) while the loads of K(t+2) and V(t+1) land in the other halves.
// The operands are read from those images directly.  S^T = K Q^T uses A-row r
// of a 32-key half for key (r & 3) + 8 ((r >> 2) & 3) + 4 (r >> 4), so that the
// 16 lanes of each read phase take 16 consecutive 16-byte pieces of one
// kilobyte (no bank conflicts), and lane group hg of a query column then holds
// the aligned key octets 8 hg + 0..7 and 16 + 8 hg + 0..7 of the half: one
// 16-byte V^T operand each, also conflict-free.
// Each wavefront runs its steps software-pipelined: the S MFMAs of tile t+1 are
// issued one at a time between the softmax instructions of tile t (the matrix
// core works while the vector ALU exponentiates), then O^T += V^T P^T for t.
template <int NWV>
__global__ __launch_bounds__(NWV * 64, 2) void k_attn_prefill_bf16(const bf16_t* __restrict__ q, KVView kv, int B,
                                                             int L, int H, int G, int n_qt, int flip,
                                                             bf16_t* __restrict__ out) {
  using namespace fa;
  // K tiles at bytes 0 and TB, V tiles at 2 TB and 3 TB
  __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * BK * D];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / (H / G);
  // (a ragged call: this sequence's own count of new tokens and first row)
  const int row0 = kv.first_row(b, L);
  L = kv.rows_of(b, L);
  const int zh = n_qt >> 1, z = blockIdx.z;
  const int qt = flip && z >= zh ? z - zh : n_qt - 1 - z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hg = lane >> 5;
  const int S = kv.lens[b];               // tokens cached before this call
  constexpr int BQ = 32 * NWV;            // queries per block (32 per wavefront)
  const int q_first = qt * BQ;            // first query index (within the new tokens)
  if (q_first >= L) return;               // (a shorter sequence of a ragged call: no queries here)
  const int wq0 = q_first + wv * 32;      // this wave's first query
  const int nq_valid = L - q_first;       // queries of this block that exist
  const int kmax_block = S + min(q_first + BQ, L);   // keys [0, kmax_block)
  const int n_tiles = (kmax_block + BK - 1) / BK;
  // sliding window: the block's earliest query sees keys from S + q_first - W + 1
  const int W = kv.window;
  const int t_first = W > 0 ? max(0, S + q_first - W + 1) / BK : 0;
  const int my_q = wq0 + l32;             // query handled by this lane (as an S^T column)
  const int my_pos = S + my_q;
  const int wave_kmax = S + min(wq0 + 32, L);        // keys this wave needs: [0, wave_kmax)

  // Q^T fragments (B operand): lane holds Q[q = l32][d = 16*kc + 8*hg .. +7]
  bf16x8 qf[8];
  {
    const bool ok = my_q < L;
    const bf16_t* qrow = q + ((size_t)(row0 + (ok ? my_q : 0)) * H + h) * D;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 v = ok ? ld16(qrow + 16 * kc + 8 * hg) : make_uint4(0, 0, 0, 0);
      qf[kc] = as_bf16x8(v);
    }
  }

  // page-table entry of key tile t (clamped to the table row: entries past the
  // block's last tile are read and not used)
  const int32_t* trow = kv.table + (size_t)b * kv.pps;
  auto page_of = [&](int t) __attribute__((always_inline)) { return trow[min(t * BK / kv.ps, kv.pps - 1)]; };
  // byte offset of this head's 64-slot block of tile t in the K (or V) pool
  auto tile_off = [&](int t, int page) __attribute__((always_inline)) {
    return ((size_t)page * kv.G + g) * kv.ps * (D * 2) + (size_t)(((t * BK) % kv.ps) >> 6) * TB;
  };
  const char* Kg = (const char*)kv.k;
  const char* Vg = (const char*)kv.v;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(char*)smem);
  const uint32_t vlane = (uint32_t)lane * 16;
  // wavefront wv copies kilobytes 4 wv .. 4 wv + 3 of a tile
  auto copy_tile = [&](const char* pool, size_t off, uint32_t lds_byte) __attribute__((always_inline)) {
    constexpr int PER = TB / NWV;         // bytes of a tile each wavefront copies
    const char* src = pool + off + wv * PER;
    const uint32_t dst = lds0 + lds_byte + wv * PER;
#pragma unroll
    for (int i = 0; i < PER / 1024; ++i) lds_dma16(vlane, src + i * 1024, dst + i * 1024);
  };
  const char* sm = (const char*)smem;
  // fragment byte offsets inside a tile image (see the layout note above)
  const uint32_t klane = (l32 >> 4) * 4096 + hg * 256 + (l32 & 15) * 16;
  const uint32_t vl = (l32 >> 4) * 2048 + hg * 256 + (l32 & 15) * 16;
  auto kfrag = [&](int t, int st2, int kc) __attribute__((always_inline)) {
    return as_bf16x8(ld16(sm + (t & 1) * TB + klane + st2 * 8192 + (kc >> 1) * 1024 + (kc & 1) * 512));
  };
  auto vfrag = [&](int t, int ds, int c) __attribute__((always_inline)) {
    return ld16(sm + 2 * TB + (t & 1) * TB + vl + ds * 4096 + (c >> 1) * 1024 + (c & 1) * 512);
  };

  f32x16 o_acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o_acc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // does this wavefront take key tile t (causal end, its queries, the window)
  auto need = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * BK;
    return key0 < wave_kmax && nq_valid > wv * 32 && (W == 0 || key0 + BK > S + wq0 - W + 1);
  };
  // some key of tile t may exceed some query position, or (window) lie
  // before one query's window
  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * BK;
    return key0 + BK - 1 > S + wq0 || (W > 0 && key0 < S + wq0 + 32 - W);
  };
  // key offset (minus 8 hg) of score i of half st2 in the tile
  auto kofs = [](int st2, int i) { return 32 * st2 + (i & 3) + 16 * ((i >> 2) & 1) + 4 * (i >> 3); };

  auto qk = [&](int t, f32x16(&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2) {
      s[st2] = (f32x16){};
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) s[st2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(t, st2, kc), qf[kc], s[st2], 0, 0, 0);
    }
  };
  // scores -> row max; raise the exponent base (and rescale o, l) only when a
  // query's tile maximum exceeds it by more than 2^8, decided per wavefront:
  // p <= 256 stays exact in fp32 and safe in bf16, and o / l does not depend
  // on the base.  Returns the base to use (0 while a row is fully masked).
  auto rebase = [&](f32x16(&s)[2]) __attribute__((always_inline)) {
    float tmax = -INFINITY;
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[st2][i]);
    tmax = fmaxf(tmax, xor_lane<32>(tmax, lane));
    const bool raise = tmax * sl2 > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? tmax * sl2 : m_run;
      // (a fully masked row so far keeps m = -inf, so alpha = 0 scales nothing)
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) o_acc[ds] *= alpha;
      m_run = m_new;
    }
    return m_run == -INFINITY ? 0.f : m_run;
  };
  // O^T += V^T P^T for tile t; chunk c of 16 keys takes the lane's octet of
  // half c / 2: scores 0-3, 8-11 (c even) or 4-7, 12-15 (c odd).  On the last
  // tile, V of slots at or past kmax_block (stale or never written) is zeroed
  // in the operand, so that a 0 weight never meets a NaN.
  auto pv = [&](int t, const f32x16(&s)[2]) __attribute__((always_inline)) {
    const int nvalid = kmax_block - t * BK;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int st2 = c >> 1, r0 = 4 * (c & 1);
      uint4 pw;
      pw.x = pack_bf16x2(s[st2][r0 + 0], s[st2][r0 + 1]);
      pw.y = pack_bf16x2(s[st2][r0 + 2], s[st2][r0 + 3]);
      pw.z = pack_bf16x2(s[st2][r0 + 8], s[st2][r0 + 9]);
      pw.w = pack_bf16x2(s[st2][r0 + 10], s[st2][r0 + 11]);
      const bf16x8 pb = as_bf16x8(pw);   // P^T: keys 16 c + 8 hg + 0..7 of query l32
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        uint4 v = vfrag(t, ds, c);
        if (nvalid < BK) {
          const int nok = nvalid - 16 * c - 8 * hg;
          if (nok < 8) {
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= nok) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
        o_acc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v), pb, o_acc[ds], 0, 0, 0);
      }
    }
  };
  // softmax and P.V of tile t (any tile: causal / window mask as needed)
  auto softmax_pv = [&](int t, f32x16(&s)[2]) __attribute__((always_inline)) {
    if (need_mask(t)) {
      // keep key offsets ko (minus 8 hg) with lo < ko <= rel: one unsigned
      // compare per score
      const int rel = my_pos - t * BK - 8 * hg;
      const int lo = W > 0 ? rel - W : -1;
      const unsigned n_keep = rel > lo ? (unsigned)(rel - lo) : 0u;
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[st2][i] = (unsigned)(kofs(st2, i) - lo - 1) < n_keep ? s[st2][i] : -INFINITY;
    }
    const float m_use = rebase(s);
    float psum = 0.f;
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st2][i], sl2, -m_use));
        s[st2][i] = p;
        psum += p;
      }
    psum += xor_lane<32>(psum, lane);
    l_run += psum;
    pv(t, s);
  };
  // an unmasked tile t whose successor this wavefront also takes: the 16 S
  // MFMAs of tile t + 1 go out one per group of two exponentials of tile t
  // (the fences keep that order), each fragment read four MFMAs ahead
  auto fused = [&](int t, f32x16(&sc)[2], f32x16(&sn)[2]) __attribute__((always_inline)) {
    constexpr int AHEAD = 4;
    bf16x8 kf[AHEAD];
    // MFMA j: half j & 1, d chunk j >> 1 (the two halves' chains alternate)
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) kf[j] = kfrag(t + 1, j & 1, j >> 1);
    const float m_use = rebase(sc);
    sn[0] = (f32x16){};
    sn[1] = (f32x16){};
    float psum = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // (raised issue priority while this wavefront feeds the matrix core: the
    // SIMD's other wavefront, often in its vector-only softmax, yields to it)
    __builtin_amdgcn_s_setprio(1);
    static_for_fa<0, 16>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % AHEAD], qf[j >> 1], sn[j & 1], 0, 0, 0);
      if constexpr (j + AHEAD < 16) kf[j % AHEAD] = kfrag(t + 1, (j + AHEAD) & 1, (j + AHEAD) >> 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 2 * j + u;            // score i % 16 of half i / 16
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i >> 4][i & 15], sl2, -m_use));
        sc[i >> 4][i & 15] = p;
        psum += p;
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    psum += xor_lane<32>(psum, lane);
    l_run += psum;
    pv(t, sc);
    __builtin_amdgcn_s_setprio(0);
  };

  // prologue: K(t0), V(t0), K(t0+1) resident, S(t0) computed
  const int t0 = t_first;
  if (t0 >= n_tiles) return;
  int pg1 = page_of(t0 + 1), pg2 = page_of(t0 + 2);
  {
    const int p0 = page_of(t0);
    copy_tile(Kg, tile_off(t0, p0), (t0 & 1) * TB);
    copy_tile(Vg, tile_off(t0, p0), 2 * TB + (t0 & 1) * TB);
    if (t0 + 1 < n_tiles) copy_tile(Kg, tile_off(t0 + 1, pg1), ((t0 + 1) & 1) * TB);
    wait_vmcnt<0>();
    lds_barrier();
  }
  f32x16 sA[2], sB[2];
  if (need(t0)) qk(t0, sA);
  // step t: S(t) in sc; K(t+1) and V(t) resident after the barrier.  FUSED:
  // a tile in the wavefront's unmasked interior (it also takes tile t+1)
  auto step = [&](int t, f32x16(&sc)[2], f32x16(&sn)[2], auto fused_c) __attribute__((always_inline)) {
    // this wavefront's loads of the previous step have landed; after the
    // barrier every wavefront's have, and every wavefront is done with step
    // t - 1 (its reads of K(t) and V(t-1), whose buffers are refilled now)
    wait_vmcnt<0>();
    lds_barrier();
    const int pg3 = page_of(t + 3);   // requested a step before its use
    if (t + 2 < n_tiles) copy_tile(Kg, tile_off(t + 2, pg2), (t & 1) * TB);
    if (t + 1 < n_tiles) copy_tile(Vg, tile_off(t + 1, pg1), 2 * TB + ((t + 1) & 1) * TB);
    pg1 = pg2;
    pg2 = pg3;
    if constexpr (decltype(fused_c)::value) {
      fused(t, sc, sn);
    } else {
      if (t + 1 < n_tiles && need(t + 1)) qk(t + 1, sn);
      if (need(t)) softmax_pv(t, sc);
    }
  };
  // The steps up to n_tiles in three runs (bounds wave-uniform): tiles before
  // the unmasked interior, the interior [lo, hi), the rest.  Every wavefront
  // takes every step (one barrier each); each run alternates the two score
  // sets, and a run of odd length hands S over with one copy.
  int lo = t0, hi = t0;
  if (nq_valid > wv * 32) {
    const int te = (wave_kmax + BK - 1) / BK;                 // tiles [.., te) needed
    // window: tiles whose keys all lie inside every query's window
    if (W > 0) lo = max(lo, (S + wq0 + 32 - W + BK - 1) / BK);
    // causal: tiles wholly below the wave's first query, and a successor taken
    const int diag = S + wq0 - (BK - 1) >= 0 ? (S + wq0 - (BK - 1)) / BK + 1 : 0;
    hi = min(te - 1, diag);
    if (hi < lo) hi = lo;
  }
  int t = t0;
  auto run = [&](int t_end, auto fused_c) __attribute__((always_inline)) {
    for (; t + 1 < t_end; t += 2) {
      step(t, sA, sB, fused_c);
      step(t + 1, sB, sA, fused_c);
    }
    if (t < t_end) {
      step(t, sA, sB, fused_c);
      sA[0] = sB[0];
      sA[1] = sB[1];
      ++t;
    }
  };
  run(lo, std::false_type{});
  run(hi, std::true_type{});
  run(n_tiles, std::false_type{});

  // write O[q][d] = O^T / l : lane holds q = l32, d = 32*ds + 8*(i/4) + 4*hg + i%4
  if (my_q < L) {
    const float inv = 1.0f / l_run;
    bf16_t* orow = out + ((size_t)(row0 + my_q) * H + h) * D;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        int dd = 32 * ds + 8 * r4 + 4 * hg;
        uint2 w;
        w.x = pack_bf16x2(o_acc[ds][4 * r4 + 0] * inv, o_acc[ds][4 * r4 + 1] * inv);
        w.y = pack_bf16x2(o_acc[ds][4 * r4 + 2] * inv, o_acc[ds][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dd) = w;
      }
  }
}

void launch_attn_prefill_bf16(const bf16_t* q, KVView kv, int B, int L, int H, int G, bf16_t* out, hipStream_t s) {
  if (B <= 0 || L <= 0) return;
  constexpr int NWV = 4;                    // wavefronts (32 queries each) per block
  constexpr int BQ = 32 * NWV;
  const int n_qt = (L + BQ - 1) / BQ;
  // A grid of one round of blocks (two per compute unit) puts its second half
  // light first: block i and block i + half then take complementary query
  // tiles (measured: 3-4% faster at 32 heads x 16 tiles); heavy-first order
  // otherwise, which dynamic dispatch balances over several rounds.  (Two
  // tiles per block, complementary ones, measured no faster.)
  const long blocks = (long)H * B * n_qt;
  const int flip = blocks <= 256 * (8 / NWV) ? 1 : 0;
  plan_log("attention prefill: %d heads (%d kv) x %d sequences x %d query tiles of %d, %s order", H, G, B, n_qt,
           BQ, flip ? "half-flipped" : "heavy-first");
  dim3 grid(H, B, n_qt);
  hipLaunchKernelGGL(k_attn_prefill_bf16<NWV>, grid, dim3(NWV * 64), 0, s, q, kv, B, L, H, G, n_qt, flip, out);
}

// ===========================================================================
// bf16 split-K decode, head_dim 128
// ===========================================================================
// One wavefront = one (sequence b, kv head g, key chunk c of split_len keys).
// Query columns: up to 16 query heads of kv head g (a virtual group), padded to 16.
// S^T (16 keys x 16 q) = K (16 x 32 d) Q^T via 16x16x32 MFMA, 4 d-chunks;
// O^T (16 d x 16 q) += V^T (16 d x 32 keys) P^T, 8 d-subtiles.
// Partials: part_o [B][H][n_splits][128], part_ml [B][H][n_splits][2] (max, sum).
// Keys are processed 64 per step (a step never crosses a page: pages are a
// multiple of 64 slots).  The four 16-key S tiles load their K rows in an order
// that leaves every lane holding 8 consecutive keys of one 32-key half for its
// query column: tile st = 2*half + t, A-row r loads key 32*half + 8*(r/4) +
// 4*t + r%4, so accumulator element i of lane group hg is key 32*half + 8*hg +
// 4*t + i.  Those 8 probabilities are then directly the B operand of the P.V
// MFMA, and the matching V^T operand is one 16-byte load of 8 consecutive
// slots of a transposed V page row.
// BM (few sequences and kv heads, a short cache): one block of 8 wavefronts per
// (b, g), wavefront c taking keys [c * split_len, (c + 1) * split_len); the 8
// partials are merged through LDS in the same block, so no second kernel.
// two wavefronts per SIMD: the register budget of one 64-key step (K, V, P, O)
template <bool BM>
__global__ __launch_bounds__(BM ? 512 : 256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_decode_bf16(
    const bf16_t* __restrict__ q, KVView kv, int B, int H, int G, int n_splits, int split_len,
    float* __restrict__ part_o, float* __restrict__ part_ml, bf16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, hg = lane >> 4;
  // wave-uniform indices in scalar registers: the lens and block-table reads are
  // scalar loads, counted apart from the vector loads in flight
  // a kv head's n_rep query heads go in virtual groups of at most 16 (the MFMA
  // rows), each read against the same keys: nv per kv head, VG in all
  const int n_rep = H / G, nv = (n_rep + 15) >> 4, VG = G * nv;
  int c, vg, b;
  if constexpr (BM) {
    c = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    vg = __builtin_amdgcn_readfirstlane(blockIdx.x % VG);
    b = __builtin_amdgcn_readfirstlane(blockIdx.x / VG);
  } else {
    const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const int total = B * VG * n_splits;
    if (wid >= total) return;
    c = wid % n_splits;
    vg = (wid / n_splits) % VG;
    b = wid / (n_splits * VG);
  }
  const int g = vg / nv, h0 = (vg % nv) * 16, nr = min(16, n_rep - h0);
  const bool qvalid = l16 < nr;
  const int hq = g * n_rep + h0 + (qvalid ? l16 : 0);
  // BM without a window: the page-table entries of the wavefront's first
  // kBMPages steps (its range starts at c * split_len) are requested together
  // with the length and the query, so the first K/V loads wait for one
  // round trip, not two; entries past the last key are read (clamped to the
  // table row) and not used
  constexpr int kBMPages = 4;
  const int32_t* trow = kv.table + (size_t)b * kv.pps;
  int pg[kBMPages];
  if constexpr (BM) {
#pragma unroll
    for (int j = 0; j < kBMPages; ++j) pg[j] = trow[min((c * split_len + 64 * j) / kv.ps, kv.pps - 1)];
  }
  const int pos = kv.lens[b];               // the new token's position; keys 0..pos
  // Q^T fragments: lane holds Q[q = l16][d = 32*kc + 8*hg .. +7]
  bf16x8 qf[4];
  {
    const bf16_t* qrow = q + ((size_t)b * H + hq) * 128;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[kc] = as_bf16x8(qvalid ? ld16(qrow + 32 * kc + 8 * hg) : make_uint4(0, 0, 0, 0));
  }
  // (one wait for all of them here, before anything depends on the length)
  if constexpr (BM) asm volatile("" ::"s"(pg[0]), "s"(pg[1]), "s"(pg[2]), "s"(pg[3]), "s"(pos));
  const int nkeys = pos + 1;
  const int k_lo = kv.window > 0 ? max(0, nkeys - kv.window) : 0;   // sliding window: keys k_lo..pos
  // splits tile the keys from the window's start (rounded down to a 64-key step)
  const int k_begin = (k_lo & ~63) + c * split_len;
  const int k_end = min(nkeys, k_begin + split_len);

  const bf16_t* Kp = (const bf16_t*)kv.k;
  const bf16_t* Vp = (const bf16_t*)kv.v;
  const float sl2 = 1.4426950408889634f / sqrtf(128.f);
  f32x4 o_acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o_acc[i] = (f32x4){};
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = k_begin; k0 < k_end; k0 += 64) {
    const int j = (k0 - k_begin) >> 6;
    int page;
    if (BM && kv.window <= 0 && j < kBMPages)
      page = j == 0 ? pg[0] : j == 1 ? pg[1] : j == 2 ? pg[2] : pg[3];
    else
      page = trow[k0 / kv.ps];
    const size_t base = (size_t)page * kv.G * kv.ps * 128;
    // this head's K and V blocks, 64-slot sub-block of k0 (tiled layout)
    const size_t sub = base + (size_t)g * kv.ps * 128 + (size_t)((k0 % kv.ps) >> 6) * (64 * 128);
    const bf16_t* kpage = Kp + sub + lane * 8;
    const bf16_t* vpage = Vp + sub + lane * 8;
    uint4 kr[4][4], vr[8][2];
    // each load: one contiguous KB holding this tile's operand fragment
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) kr[st][kc] = ld16(kpage + (st * 4 + kc) * 512);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) vr[ds][hf] = ld16(vpage + (ds * 2 + hf) * 512);
    f32x4 s_acc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      s_acc[st] = (f32x4){};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        s_acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[st][kc]), qf[kc], s_acc[st], 0, 0, 0);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 32 * (st >> 1) + 8 * hg + 4 * (st & 1) + i;
        const float v = key < k_end && key >= k_lo ? s_acc[st][i] : -INFINITY;
        s_acc[st][i] = v;
        tmax = fmaxf(tmax, v);
      }
    // (lane-row swaps, not LDS permutes: nothing else in the loop waits on the
    // LDS / scalar counter)
    tmax = fmaxf(tmax, xor_lane<16>(tmax, lane));
    tmax = fmaxf(tmax, xor_lane<32>(tmax, lane));
    // running max in log2 units: p = 2^(s * log2(e)/sqrt(d) - m), one fma + v_exp_f32
    const float m_new = fmaxf(m_run, tmax * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[st][i], sl2, -m_new));
        s_acc[st][i] = p;
        psum += p;
      }
    psum += xor_lane<16>(psum, lane);
    psum += xor_lane<32>(psum, lane);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    bf16x8 pb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint4 pw;
      pw.x = pack_bf16x2(s_acc[2 * hf][0], s_acc[2 * hf][1]);
      pw.y = pack_bf16x2(s_acc[2 * hf][2], s_acc[2 * hf][3]);
      pw.z = pack_bf16x2(s_acc[2 * hf + 1][0], s_acc[2 * hf + 1][1]);
      pw.w = pack_bf16x2(s_acc[2 * hf + 1][2], s_acc[2 * hf + 1][3]);
      pb[hf] = as_bf16x8(pw);
    }
    if (k0 + 64 > k_end) {
      // slots past the last key: zero the values (a stale NaN times weight 0
      // would poison the sum)
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          uint32_t w[4] = {vr[ds][hf].x, vr[ds][hf].y, vr[ds][hf].z, vr[ds][hf].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + 32 * hf + 8 * hg + e >= k_end) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          vr[ds][hf] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      o_acc[ds] *= alpha;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        o_acc[ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[ds][hf]), pb[hf], o_acc[ds], 0, 0, 0);
    }
  }
  // lane: O^T[d = 16*ds + 4*hg + i][q = l16]
  if constexpr (BM) {
    // rows padded to 132 floats: the 16 query columns' writes spread over banks
    __shared__ float so[8][16][132];
    __shared__ float2 sml[8][16];
    if (qvalid) {
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        *reinterpret_cast<float4*>(&so[c][l16][16 * ds + 4 * hg]) =
            make_float4(o_acc[ds][0], o_acc[ds][1], o_acc[ds][2], o_acc[ds][3]);
      if (hg == 0) sml[c][l16] = make_float2(m_run, l_run);
    }
    __syncthreads();
    // wavefront w merges query heads w, w + 8, ... of the virtual group: o =
    // sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c in split order
    for (int r = c; r < nr; r += 8) {
      float M = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, sml[j][r].x);
      float o0 = 0.f, o1 = 0.f, den = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float mj = sml[j][r].x;
        const float w = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj - M);
        den += w * sml[j][r].y;
        o0 += w * so[j][r][lane];
        o1 += w * so[j][r][lane + 64];
      }
      bf16_t* orow = out + ((size_t)b * H + g * n_rep + h0 + r) * 128;
      orow[lane] = f32_to_bf16(o0 / den);
      orow[lane + 64] = f32_to_bf16(o1 / den);
    }
    return;
  }
  if (qvalid) {
    const size_t pi = (((size_t)b * H + hq) * n_splits + c);
    float* po = part_o + pi * 128;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds)
      *reinterpret_cast<float4*>(po + 16 * ds + 4 * hg) =
          make_float4(o_acc[ds][0], o_acc[ds][1], o_acc[ds][2], o_acc[ds][3]);
    if (hg == 0) {
      part_ml[pi * 2 + 0] = m_run;
      part_ml[pi * 2 + 1] = l_run;
    }
  }
}

// One wavefront per (b, h): o = sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c,
// summed in chunk order.  Lane c computes the weight of chunk c (64 chunks at a
// time, shared by shuffles); each lane owns two of the 128 output columns.
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int BH, int n_splits,
                                                    bf16_t* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wid = blockIdx.x * (blockDim.x >> 6) + wave;
  if (wid >= BH) return;
  const float* ml = part_ml + (size_t)wid * n_splits * 2;
  const float* po = part_o + (size_t)wid * n_splits * 128;
  float o0 = 0.f, o1 = 0.f, den = 0.f;
  float M = -INFINITY;
  for (int c = lane; c < n_splits; c += 64) M = fmaxf(M, ml[2 * c]);
  M = warp_max(M);
  for (int c0 = 0; c0 < n_splits; c0 += 64) {
    const int c = c0 + lane;
    float w = 0.f, dl = 0.f;
    if (c < n_splits) {
      const float mc = ml[2 * c];
      w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
      dl = w * ml[2 * c + 1];
    }
    den += dl;
    const int nc = min(64, n_splits - c0);
    int j = 0;
    for (; j + 4 <= nc; j += 4) {
      float a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = po[(size_t)(c0 + j + u) * 128 + lane];
        bb[u] = po[(size_t)(c0 + j + u) * 128 + lane + 64];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = __shfl(w, j + u, 64);
        o0 += wu * a[u];
        o1 += wu * bb[u];
      }
    }
    for (; j < nc; ++j) {
      const float wu = __shfl(w, j, 64);
      o0 += wu * po[(size_t)(c0 + j) * 128 + lane];
      o1 += wu * po[(size_t)(c0 + j) * 128 + lane + 64];
    }
  }
  den = warp_sum(den);
  bf16_t* orow = out + (size_t)wid * 128;
  orow[lane] = f32_to_bf16(o0 / den);
  orow[lane + 64] = f32_to_bf16(o1 / den);
}

void launch_attn_decode_bf16(const bf16_t* q, KVView kv, int B, int H, int G, int n_splits, int split_len,
                             float* part_o, float* part_ml, bf16_t* out, hipStream_t s) {
  if (B <= 0) return;
  // the keys the splits cover (at least every cached key)
  const long keys = (long)n_splits * split_len;
  const int VG = G * ((H / G + 15) / 16);   // virtual groups of at most 16 query heads
  if (B * VG <= 128 && keys <= 2048) {
    // few (b, g) pairs and a short cache: one block each, eight key ranges of
    // whole 64-key steps, merged in the block
    const int sl8 = (int)(((keys + 7) / 8 + 63) / 64 * 64);
    plan_log("attention decode: %d sequences x %d head groups, one block each, 8 ranges of %d keys merged in LDS", B,
             VG, sl8);
    hipExtLaunchKernelGGL(k_attn_decode_bf16<true>, dim3(B * VG), dim3(512), 0, s, g_clock.start, g_clock.stop, 0, q,
                          kv, B, H, G, 8, sl8, part_o, part_ml, out);
    g_clock = LaunchClock{};
    return;
  }
  // (a grid of fewer wavefronts than a round of the chip goes one wavefront
  // per block, so the dispatcher spreads it over all compute units)
  const int waves = B * VG * n_splits, wpb = waves < 1024 ? 1 : 4;
  plan_log("attention decode: %d sequences x %d head groups x %d splits of %d keys, %d wavefronts per block, merge "
           "kernel", B, VG, n_splits, split_len, wpb);
  hipExtLaunchKernelGGL(k_attn_decode_bf16<false>, dim3((waves + wpb - 1) / wpb), dim3(64 * wpb), 0, s, g_clock.start,
                        nullptr, 0, q, kv, B, H, G, n_splits, split_len, part_o, part_ml, nullptr);
  const int bh = B * H, mpb = bh < 1024 ? 1 : 4;
  hipExtLaunchKernelGGL(k_attn_merge, dim3((bh + mpb - 1) / mpb), dim3(64 * mpb), 0, s, nullptr, g_clock.stop, 0,
                        part_o, part_ml, bh, n_splits, out);
  g_clock = LaunchClock{};
}

}  // namespace lb

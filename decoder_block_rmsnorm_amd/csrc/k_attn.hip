// Causal grouped-query attention over the paged KV cache:
//   o[h] = softmax_j( q[h] . k[g][j] / sqrt(d) ) v[g][j],  j <= position,
//   g = h / (H / G)
// (LLaMAAttention of page 二 with its expand-then-reshape kv sharing; the causal
// rule of "5. 因果掩码" and the KV cache of "2. 注意力机制", MLX page).
//
//  * k_attn_simt         : one wavefront per (token, head), lanes over head_dim,
//                          online softmax over keys (fp32 path).
//  * k_attn_prefill_bf16 : flash-style prefill: 128 queries of one head per
//                          block, 64-key K / V^T tiles staged in LDS, S^T = K Q^T
//                          and O^T = V^T P^T on 32x32x16 bf16 MFMA, fp32 online
//                          softmax (the tiling idea credited to FlashAttention in
//                          "Transformer 块的内部结构" of the reading-notes page).
//  * k_attn_decode_bf16  : split-K decode: each wavefront streams a 256-key
//                          chunk of one (sequence, kv head) straight from the
//                          pages with 128-bit loads, serving up to 16 query heads
//                          of the group with 16x16x32 MFMA (more query heads: one
//                          wavefront per 16 of them); k_attn_merge combines
//                          the chunks with a log-sum-exp merge in a fixed order.
#include "kernels.hpp"

namespace lb {

// ===========================================================================
// generic (fp32 path)
// ===========================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_attn_simt(const T* q, KVView kv, int B, int L, int H, int G, int d,
                                                   T* out) {
  int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (wid >= B * L * H) return;
  int h = wid % H;
  int m = wid / H;
  int b = m / L, l = m % L;
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
void launch_attn_simt(const T* q, KVView kv, int B, int L, int H, int G, int d, T* out, hipStream_t s) {
  int waves = B * L * H;
  if (waves <= 0) return;
  hipLaunchKernelGGL(k_attn_simt<T>, dim3((waves + 3) / 4), dim3(256), 0, s, q, kv, B, L, H, G, d, out);
}

template void launch_attn_simt<float>(const float*, KVView, int, int, int, int, int, float*, hipStream_t);
template void launch_attn_simt<bf16_t>(const bf16_t*, KVView, int, int, int, int, int, bf16_t*, hipStream_t);

// ===========================================================================
// bf16 flash prefill, head_dim 128
// ===========================================================================
namespace fa {
constexpr int D = 128;
constexpr int BQ = 128;        // queries per block (4 waves x 32)
constexpr int BK = 64;         // keys per tile
constexpr int KST = D + 8;     // LDS row stride (bf16) of the K tile  [key][d]
constexpr int VST = BK + 8;    // LDS row stride (bf16) of the V^T tile [d][key]
constexpr int K_ELEMS = BK * KST;
constexpr int V_ELEMS = D * VST;
}  // namespace fa

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}


// Causal work per query tile grows with its index, so when the grid is large
// enough a block takes the pair (z, n_qt - 1 - z): every block then does the
// same amount of work.
__global__ __launch_bounds__(256, 2) void k_attn_prefill_bf16(const bf16_t* __restrict__ q, KVView kv, int B,
                                                             int L, int H, int G, int n_qt, int paired,
                                                             bf16_t* __restrict__ out) {
  using namespace fa;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (K_ELEMS + V_ELEMS)];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / (H / G);
  for (int pass = 0; pass < 2; ++pass) {
  // unpaired: one tile per block, heavy (late) query tiles first
  const int qt = !paired ? n_qt - 1 - (int)blockIdx.z : pass == 0 ? n_qt - 1 - (int)blockIdx.z : (int)blockIdx.z;
  if (pass == 1 && (!paired || qt >= n_qt - 1 - (int)blockIdx.z)) break;   // (middle tile of an odd count: done)
  __syncthreads();   // LDS of the previous pass is free
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hg = lane >> 5;
  const int S = kv.lens[b];               // tokens cached before this call
  const int q_first = qt * BQ;            // first query index (within the new tokens)
  const int wq0 = q_first + wave * 32;    // this wave's first query
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
    const bf16_t* qrow = q + ((size_t)(b * L + (ok ? my_q : 0)) * H + h) * D;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 v = ok ? ld16(qrow + 16 * kc + 8 * hg) : make_uint4(0, 0, 0, 0);
      qf[kc] = as_bf16x8(v);
    }
  }

  const bf16_t* Kp = (const bf16_t*)kv.k;
  const bf16_t* Vp = (const bf16_t*)kv.v;
  // tile loader: K tile 64 keys x 128 d (16 chunks of 16 B per key row); V^T tile
  // 128 d rows x 64 keys (8 chunks per row).  1024 chunks each, 4 per thread.
  // Slots at or past kmax_block hold no key of this call (stale or never
  // written); they are zeroed so that a 0 softmax weight never meets a NaN.
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
    int key0 = t * BK;
    size_t base = kv.page_base(b, key0);
    int slot0 = key0 % kv.ps;
    int nvalid = kmax_block - key0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      int kr = c >> 4, kc = c & 15;
      const size_t blk = base + (size_t)g * kv.ps * D;   // this head's K (and V) block of the page
      kreg[i] = kr < nvalid ? ld16(Kp + blk + kv_tiled_k(slot0 + kr, kc * 8)) : make_uint4(0, 0, 0, 0);
      int vr = c >> 3, vc = c & 7;
      uint4 v = ld16(Vp + blk + kv_tiled_v(slot0 + vc * 8, vr));
      int nok = nvalid - vc * 8;
      if (nok < 8) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nok) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      vreg[i] = v;
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* ks = smem + buf * (K_ELEMS + V_ELEMS);
    bf16_t* vs = ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      int kr = c >> 4, kc = c & 15;
      st16(ks + kr * KST + kc * 8, kreg[i]);
      int vr = c >> 3, vc = c & 7;
      st16(vs + vr * VST + vc * 8, vreg[i]);
    }
  };

  f32x16 o_acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o_acc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  if (t_first < n_tiles) load_tile(t_first);
  for (int t = t_first; t < n_tiles; ++t) {
    const int buf = (t - t_first) & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);
    const int key0 = t * BK;
    // (W > 0: tiles wholly before the window of this wave's first query skip)
    if (key0 < wave_kmax && nq_valid > wave * 32 && (W == 0 || key0 + BK > S + wq0 - W + 1)) {
      const bf16_t* ks = smem + buf * (K_ELEMS + V_ELEMS);
      const bf16_t* vs = ks + K_ELEMS;
      // S^T = K Q^T : 2 key subtiles of 32.  A-row r = 8a + 4h + m of subtile st
      // holds key 32 st + 16 (a / 2) + 8 h + 4 (a % 2) + m, so that afterwards
      // lane group hg holds keys 16 c + 8 hg + 0..7 of each 16-key chunk c: the
      // P.V operands are then 8 consecutive keys (one 16-byte V^T read).
      const int krow = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
      f32x16 s_acc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s_acc[st] = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) {
          bf16x8 a = as_bf16x8(ld16(ks + (st * 32 + krow) * KST + kc * 16 + hg * 8));
          s_acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s_acc[st], 0, 0, 0);
        }
      }
      // scale, causal mask, online softmax (query = column l32; rows = keys)
      // (scores stay unscaled; the running max m is kept in log2 units, so
      // p = 2^(s * log2(e)/sqrt(d) - m) is one fma and one v_exp_f32)
      // some key may exceed some query position, or (window) lie before one
      // query's window
      const bool need_mask = key0 + BK - 1 > S + wq0 || (W > 0 && key0 < S + wq0 + 32 - W);
      float tmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = s_acc[st][i];
          if (need_mask) {
            int key = key0 + st * 32 + 16 * (i >> 3) + 8 * hg + (i & 7);
            if (key > my_pos || (W > 0 && key <= my_pos - W)) v = -INFINITY;
          }
          s_acc[st][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax * sl2);
      // a fully masked row so far keeps m = -inf; use 0 as the exponent base then
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[st][i], sl2, -m_use));
          s_acc[st][i] = p;
          psum += p;
        }
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) o_acc[ds] *= alpha;
      // O^T += V^T P^T : 4 key chunks of 16 (B operand straight from S^T registers)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int st = c >> 1, r0 = 8 * (c & 1);
        uint4 pw;
        pw.x = pack_bf16x2(s_acc[st][r0 + 0], s_acc[st][r0 + 1]);
        pw.y = pack_bf16x2(s_acc[st][r0 + 2], s_acc[st][r0 + 3]);
        pw.z = pack_bf16x2(s_acc[st][r0 + 4], s_acc[st][r0 + 5]);
        pw.w = pack_bf16x2(s_acc[st][r0 + 6], s_acc[st][r0 + 7]);
        bf16x8 pb = as_bf16x8(pw);   // P^T: keys 16 c + 8 hg + 0..7 of query l32
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          bf16x8 a = as_bf16x8(ld16(vs + (ds * 32 + l32) * VST + 16 * c + 8 * hg));
          o_acc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o_acc[ds], 0, 0, 0);
        }
      }
    }
  }
  // write O[q][d] = O^T / l : lane holds q = l32, d = 32*ds + 8*(i/4) + 4*hg + i%4
  if (my_q < L) {
    const float inv = 1.0f / l_run;
    bf16_t* orow = out + ((size_t)(b * L + my_q) * H + h) * D;
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
  }  // pass
}

void launch_attn_prefill_bf16(const bf16_t* q, KVView kv, int B, int L, int H, int G, bf16_t* out, hipStream_t s) {
  if (B <= 0 || L <= 0) return;
  const int n_qt = (L + fa::BQ - 1) / fa::BQ;
  // (measured: no faster than one tile per block at the configurations here,
  // so pairing is off)
  const int paired = 0;
  dim3 grid(H, B, paired ? (n_qt + 1) / 2 : n_qt);
  hipLaunchKernelGGL(k_attn_prefill_bf16, grid, dim3(256), 0, s, q, kv, B, L, H, G, n_qt, paired, out);
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
    const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int total = B * VG * n_splits;
    if (wid >= total) return;
    c = wid % n_splits;
    vg = (wid / n_splits) % VG;
    b = wid / (n_splits * VG);
  }
  const int g = vg / nv, h0 = (vg % nv) * 16, nr = min(16, n_rep - h0);
  const int pos = kv.lens[b];               // the new token's position; keys 0..pos
  const int nkeys = pos + 1;
  const int k_lo = kv.window > 0 ? max(0, nkeys - kv.window) : 0;   // sliding window: keys k_lo..pos
  // splits tile the keys from the window's start (rounded down to a 64-key step)
  const int k_begin = (k_lo & ~63) + c * split_len;
  const int k_end = min(nkeys, k_begin + split_len);
  const bool qvalid = l16 < nr;
  const int hq = g * n_rep + h0 + (qvalid ? l16 : 0);

  // Q^T fragments: lane holds Q[q = l16][d = 32*kc + 8*hg .. +7]
  bf16x8 qf[4];
  {
    const bf16_t* qrow = q + ((size_t)b * H + hq) * 128;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[kc] = as_bf16x8(qvalid ? ld16(qrow + 32 * kc + 8 * hg) : make_uint4(0, 0, 0, 0));
  }
  const bf16_t* Kp = (const bf16_t*)kv.k;
  const bf16_t* Vp = (const bf16_t*)kv.v;
  const float sl2 = 1.4426950408889634f / sqrtf(128.f);
  f32x4 o_acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o_acc[i] = (f32x4){};
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = k_begin; k0 < k_end; k0 += 64) {
    const size_t base = kv.page_base(b, k0);
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
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
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
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
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
  const int wid = blockIdx.x * 4 + wave;
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
    hipExtLaunchKernelGGL(k_attn_decode_bf16<true>, dim3(B * VG), dim3(512), 0, s, g_clock.start, g_clock.stop, 0, q,
                          kv, B, H, G, 8, sl8, part_o, part_ml, out);
    g_clock = LaunchClock{};
    return;
  }
  int waves = B * VG * n_splits;
  hipExtLaunchKernelGGL(k_attn_decode_bf16<false>, dim3((waves + 3) / 4), dim3(256), 0, s, g_clock.start, nullptr, 0, q, kv, B, H, G, n_splits,
                     split_len, part_o, part_ml, nullptr);
  int bh = B * H;
  hipExtLaunchKernelGGL(k_attn_merge, dim3((bh + 3) / 4), dim3(256), 0, s, nullptr, g_clock.stop, 0, part_o, part_ml,
                        bh, n_splits, out);
  g_clock = LaunchClock{};
}

}  // namespace lb

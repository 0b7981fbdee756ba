// Shared device/host definitions for the gfx950 decoder-block kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef __HIP_DEVICE_COMPILE__
#include <cstdio>
#endif

namespace lb {

typedef uint16_t bf16_t;  // raw bfloat16 storage

// MFMA operand / accumulator vector types (gfx950 builtins take __bf16 / _Float16 vectors).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__host__ __device__ inline float bf16_to_f32(bf16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

// float -> bf16, round to nearest even (one v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ inline bf16_t f32_to_bf16(float f) {
  const __bf16 h = (__bf16)f;
  bf16_t r;
  __builtin_memcpy(&r, &h, 2);
  return r;
}
// two floats -> packed bf16 pair (a in the low half), one instruction
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
  const bf16x2v v = {(__bf16)a, (__bf16)b};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// Element type traits: the fp32 and bf16 paths share templates through these.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __host__ inline float load(const float* p, size_t i) { return p[i]; }
  static __device__ __host__ inline void store(float* p, size_t i, float v) { p[i] = v; }
  static __device__ __host__ inline float to_f(float v) { return v; }
  static __device__ __host__ inline float from_f(float v) { return v; }
  // round a float to what storage keeps
  static __device__ __host__ inline float round(float v) { return v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __host__ inline float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ inline void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  static __device__ __host__ inline float to_f(bf16_t v) { return bf16_to_f32(v); }
  static __device__ inline bf16_t from_f(float v) { return f32_to_bf16(v); }
  static __device__ inline float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Paged KV cache view of one layer, passed by value to kernels.  A page holds
// ps slots for each of the G kv heads: per head a K block and a V block of
// ps * d elements each.
//   fp32 (row-major):  K block [ps][d], V block [d][ps] (transposed).
//   bf16, d = 128 (tiled): each block is ps/64 sub-blocks of 64 slots in the
//   operand order of the decode attention's 16x16x32 MFMAs, so that every
//   wavefront-wide 16-byte load there is one contiguous kilobyte:
//     K: fragment (st, kc) = 1 KB at ((st * 4 + kc) * 64 + lane) * 8, lane =
//        16 * (d % 32 / 8) + r, holding key 32 (st / 2) + 8 (r / 4) + 4 (st % 2)
//        + r % 4 and dims 32 kc + 8 (lane / 16) .. + 7;
//     V: fragment (ds, hf) = 1 KB at ((ds * 2 + hf) * 64 + lane) * 8, lane =
//        16 * (key % 32 / 8) + d % 16, holding dim 16 ds + d % 16 and keys
//        32 hf + 8 (lane / 16) .. + 7.
//   Within a 16-byte piece, 8 consecutive dims (K) or 8 consecutive keys (V).
__host__ __device__ inline int kv_tiled_k(int slot, int e) {
  const int k = slot & 63;
  const int st = 2 * (k >> 5) + ((k >> 2) & 1), r = 4 * ((k >> 3) & 3) + (k & 3);
  return (slot >> 6) * (64 * 128) + ((st * 4 + (e >> 5)) * 64 + ((e >> 3) & 3) * 16 + r) * 8 + (e & 7);
}
__host__ __device__ inline int kv_tiled_v(int slot, int e) {
  const int k = slot & 63;
  return (slot >> 6) * (64 * 128) + (((e >> 4) * 2 + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (e & 15)) * 8 + (k & 7);
}
struct KVView {
  void* k;              // this layer's K pool base
  void* v;              // this layer's V pool base
  const int32_t* table; // [max_batch][pps]
  int32_t* lens;        // this layer's lens [max_batch]
  int32_t G, d, ps, pps;
  int32_t tiled;        // bf16 / d = 128 operand-order layout (see above)
  int32_t window;       // sliding window: keys pos - window + 1 .. pos (0 = all keys up to pos)
  // The rows of a prefill call: a ragged call (sequences bringing different
  // numbers of new tokens) gives cu[b] = first row of sequence b, for b <=
  // n_seq (cu[n_seq] = rows of the call); otherwise cu is null and every
  // sequence has L rows.
  const int32_t* cu;
  int32_t n_seq;
  __device__ inline int first_row(int b, int L) const { return cu ? cu[b] : b * L; }
  __device__ inline int rows_of(int b, int L) const { return cu ? cu[b + 1] - cu[b] : L; }
  // the sequence row r belongs to (for a ragged call: the b with cu[b] <= r < cu[b + 1])
  __device__ inline int seq_of_row(int r, int L) const {
    if (!cu) return r / L;
    int lo = 0, hi = n_seq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= r) lo = mid;
      else hi = mid;
    }
    return lo;
  }
  __device__ __host__ inline size_t page_base(int b, int pos) const {
    int page = table[(size_t)b * pps + pos / ps];
    return (size_t)page * G * ps * d;
  }
  // element offsets
  __device__ inline size_t k_off(int b, int pos, int g, int e) const {
    if (tiled) return page_base(b, pos) + (size_t)g * ps * d + kv_tiled_k(pos % ps, e);
    return page_base(b, pos) + ((size_t)g * ps + (pos % ps)) * d + e;
  }
  __device__ inline size_t v_off(int b, int pos, int g, int e) const {
    if (tiled) return page_base(b, pos) + (size_t)g * ps * d + kv_tiled_v(pos % ps, e);
    return page_base(b, pos) + ((size_t)g * d + e) * ps + (pos % ps);
  }
};

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

// Workgroup barrier for LDS communication: waits for this wave's LDS accesses,
// not for its global loads in flight.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// the value of lane l ^ M (M a power of two below 64): quad permutes and row
// rotates (DPP) within 16 lanes, lane-row swaps across 16 and 32
template <int M>
__device__ inline float xor_lane(float v, int lane) {
  const int b = __builtin_bit_cast(int, v);
  if constexpr (M == 1) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, b, 0x114, 0xF, 0xF, false);  // row_shr:4 (lane - 4)
    const int dn = __builtin_amdgcn_update_dpp(0, b, 0x104, 0xF, 0xF, false);  // row_shl:4 (lane + 4)
    return __builtin_bit_cast(float, (lane & 4) ? up : dn);
  } else if constexpr (M == 8) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else {
    // swap(v, v): the first result holds the partner's value in the odd
    // 16-/32-lane rows, the second in the even ones
    const auto p = M == 16 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                           : __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (int)((lane & M) ? p[0] : p[1]));
  }
}

__device__ inline float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(z) = z / (1 + e^-z), the quotient by the hardware reciprocal (1 ulp;
// every caller rounds the product to bf16 or sums it in fp32): z -> -inf gives
// -0, z -> +inf gives z
__device__ inline float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// 16-byte vector load/store helpers.
// Tiled layout of the bf16 dense weights [N][K] (N a multiple of 16): 16-row
// groups by 256-column chunks, each (group, chunk) tile 8 KB contiguous, stored
// chunk-major: tile (g, c) at (c * ngroups + g) * 8 KB, so that all the groups'
// tiles of one chunk form one contiguous region (a grid streaming the matrix
// chunk by chunk sweeps memory in address order).  Inside a tile, the
// 32-column block kb is 1 KB holding 64 pieces of 16 bytes: piece 16*j + r =
// row r of the group, columns 32*kb + 8*j .. 8*j + 7.  One wavefront-wide
// 16-byte load of a block (lane = piece) is then one contiguous kilobyte and
// lands as the B operand of v_mfma_f32_16x16x32_bf16 (lane l holds
// B[k = 8*(l/16) + e][n = l%16]).  K is padded to a multiple of 256 (kTileK).
constexpr int kTileK = 256;
constexpr int kTileElems = kTileK * 16;  // bf16 per (group, chunk) tile
__host__ __device__ inline int tiled_chunks(int K) { return (K + kTileK - 1) / kTileK; }
__host__ __device__ inline size_t tiled_off(int n, int k, int ngroups) {
  return ((((size_t)(k >> 8) * ngroups + (n >> 4)) * 8 + ((k >> 5) & 7)) * 64 + (((k >> 3) & 3) * 16 + (n & 15))) * 8 +
         (k & 7);
}

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace lb

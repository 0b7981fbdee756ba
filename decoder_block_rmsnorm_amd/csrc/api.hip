// C ABI of the decoder block: host-side validation, weight repacking, scratch
// layout and the launch sequences of prefill and decode.  See llama_block.h for
// the contract of every entry point.
#include <cmath>
#include <cstdarg>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "llama_block.h"

using namespace lb;

namespace lb {
thread_local LaunchClock g_clock;
}  // namespace lb

// ---------------------------------------------------------------- errors
static thread_local std::string g_err;

static llama_status fail(llama_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

static llama_status hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return LLAMA_OK;
}

#define HIP_TRY(call, what)                                                                  \
  do {                                                                                       \
    hipError_t _e = (call);                                                                  \
    if (_e != hipSuccess) return fail(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(_e)); \
  } while (0)

extern "C" const char* llama_last_error(void) { return g_err.c_str(); }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline size_t esize(int dt) { return dt == LLAMA_F32 ? 4 : 2; }

// ---------------------------------------------------------------- config
struct Dims {
  int D, H, G, d, F, Nq, Nkv, Nqkv, IB, n_rep;
  bool bf16, q4;
};

static llama_status check_config(const llama_block_config* c, Dims* o) {
  if (!c) return fail(LLAMA_ERR_INVALID_ARG, "config is NULL");
  if (c->dim <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->ffn_dim <= 0 || c->max_seq <= 0)
    return fail(LLAMA_ERR_INVALID_ARG, "dim, n_heads, n_kv_heads, ffn_dim and max_seq must be positive");
  if (c->n_heads % c->n_kv_heads)
    return fail(LLAMA_ERR_INVALID_ARG, "n_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_heads, c->n_kv_heads);
  if (c->sliding_window < 0) return fail(LLAMA_ERR_INVALID_ARG, "sliding_window must be >= 0");
  if (c->dim % c->n_heads) return fail(LLAMA_ERR_INVALID_ARG, "dim (%d) must be a multiple of n_heads (%d)", c->dim, c->n_heads);
  if (!(c->norm_eps > 0.f) || !std::isfinite(c->norm_eps)) return fail(LLAMA_ERR_INVALID_ARG, "norm_eps must be > 0");
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return fail(LLAMA_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (c->rope_traditional != 0 && c->rope_traditional != 1)
    return fail(LLAMA_ERR_INVALID_ARG, "rope_traditional must be 0 or 1");
  if (c->act_dtype != LLAMA_F32 && c->act_dtype != LLAMA_BF16) return fail(LLAMA_ERR_INVALID_ARG, "unknown act_dtype");
  if (c->weight_format != LLAMA_W_DENSE && c->weight_format != LLAMA_W_Q4)
    return fail(LLAMA_ERR_INVALID_ARG, "unknown weight_format");
  Dims d{};
  d.D = c->dim;
  d.H = c->n_heads;
  d.G = c->n_kv_heads;
  d.d = c->dim / c->n_heads;
  d.F = c->ffn_dim;
  d.Nq = d.H * d.d;
  d.Nkv = d.G * d.d;
  d.Nqkv = d.Nq + 2 * d.Nkv;
  d.n_rep = d.H / d.G;
  d.bf16 = c->act_dtype == LLAMA_BF16;
  d.q4 = c->weight_format == LLAMA_W_Q4;
  if (d.d % 2) return fail(LLAMA_ERR_INVALID_ARG, "head_dim (%d) must be even for RoPE pairs", d.d);
  if (d.bf16) {
    if (d.d != 128) return fail(LLAMA_ERR_UNSUPPORTED, "bf16 path supports head_dim 128 only (got %d)", d.d);
    if (d.D % 64 || d.F % 64) return fail(LLAMA_ERR_UNSUPPORTED, "bf16 path needs dim and ffn_dim multiples of 64");
    d.IB = 32;
  } else {
    if (d.d > 128) return fail(LLAMA_ERR_UNSUPPORTED, "fp32 path supports head_dim <= 128 (got %d)", d.d);
    if (d.F % 16) return fail(LLAMA_ERR_UNSUPPORTED, "fp32 path needs ffn_dim multiple of 16");
    d.IB = (d.F % 32) ? 16 : 32;
  }
  if (d.q4) {
    if (!d.bf16) return fail(LLAMA_ERR_UNSUPPORTED, "4-bit weights need bf16 activations");
    if (c->group_size != 64) return fail(LLAMA_ERR_UNSUPPORTED, "4-bit weights support group_size 64 only");
  }
  if (o) *o = d;
  return LLAMA_OK;
}

// ---------------------------------------------------------------- weights
struct Lin {            // a repacked linear inside the block's device memory
  void* w = nullptr;    // dense E[N, K] or q4 uint32 [N, K/8]
  bf16_t* s = nullptr;  // q4 scales [N, K/64]
  bf16_t* b = nullptr;  // q4 biases
  uint32_t* pairs = nullptr;  // q4 (scale, bias) pairs [K/64][N] for the prompt-pass GEMM
  int N = 0, K = 0;
};

struct llama_block {
  llama_block_config cfg;
  Dims dm;
  float2* rope;     // [max_seq][d/2]
  float* gamma1;    // fp32 [D]
  float* gamma2;
  Lin qkv, o, w13, w2;
  int diag = 0;     // store the feed-forward branch for LLAMA_DIAG_FFN
  // profiling: events [max_calls][kMaxMarks], calls recorded so far
  std::vector<hipEvent_t> ev;
  int prof_max = 0, prof_calls = 0, prof_marks = 0;
  uint32_t prof_mask = 0;  // phases timed (bit p = phase p); all when 0
  ~llama_block() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

static const int kMaxMarks = 12;

// Records an event before the first kernel and after each phase of one call.
// Phase boundary b (before phase b, after phase b-1) gets an event only when
// one of those two phases is timed.
//
// clocked >= 0: the single timed phase is timed by events attached to its own
// kernel launches (g_clock) instead of marker packets.
struct Marker {
  hipEvent_t* ev = nullptr;
  uint32_t mask = 0;
  int i = 0;
  int clocked = -1;
  void operator()(hipStream_t s) {
    if (!ev || i >= kMaxMarks) return;
    if (clocked >= 0) {
      g_clock = i == clocked ? LaunchClock{ev[i], ev[i + 1]} : LaunchClock{};
      ++i;
      return;
    }
    const bool need = mask == 0 || ((mask >> i) & 1u) || (i > 0 && ((mask >> (i - 1)) & 1u));
    if (need) (void)hipEventRecord(ev[i], s);
    ++i;
  }
};

struct WLayout {
  size_t rope, g1, g2, total;
  size_t lin[4][4];  // per linear: w, s, b, pairs offsets
};

static void lin_shapes(const Dims& d, int NK[4][2]) {
  NK[0][0] = d.Nqkv; NK[0][1] = d.D;
  NK[1][0] = d.D;    NK[1][1] = d.Nq;
  NK[2][0] = 2 * d.F; NK[2][1] = d.D;
  NK[3][0] = d.D;    NK[3][1] = d.F;
}

static WLayout weight_layout(const llama_block_config& c, const Dims& d) {
  WLayout L{};
  size_t off = 0;
  L.rope = off; off = align256(off + (size_t)c.max_seq * (d.d / 2) * sizeof(float2));
  L.g1 = off; off = align256(off + (size_t)d.D * 4);
  L.g2 = off; off = align256(off + (size_t)d.D * 4);
  int NK[4][2];
  lin_shapes(d, NK);
  for (int i = 0; i < 4; ++i) {
    size_t N = NK[i][0], K = NK[i][1];
    L.lin[i][0] = off;
    if (d.q4) {
      off = align256(off + N * K / 2);
      L.lin[i][1] = off; off = align256(off + N * (K / 64) * 2);
      L.lin[i][2] = off; off = align256(off + N * (K / 64) * 2);
      L.lin[i][3] = off; off = align256(off + N * (K / 64) * 4);
    } else if (d.bf16) {
      // tiled layout: K padded to whole 256-column chunks
      off = align256(off + N * (size_t)tiled_chunks((int)K) * kTileK * 2);
      L.lin[i][1] = L.lin[i][2] = 0;
    } else {
      off = align256(off + N * K * esize(c.act_dtype));
      L.lin[i][1] = L.lin[i][2] = 0;
    }
  }
  L.total = off;
  return L;
}

extern "C" size_t llama_block_weight_bytes(const llama_block_config* cfg) {
  Dims d;
  if (check_config(cfg, &d) != LLAMA_OK) return 0;
  return weight_layout(*cfg, d).total;
}

static bool lin_ok(const llama_linear& l, bool q4) {
  if (!l.w) return false;
  if (q4 && (!l.scales || !l.biases)) return false;
  return true;
}

// Copy one source linear into the repacked buffer with a row map (and, dense
// only, a column scale).
static void repack_linear(const Dims& d, int dt, const Lin& dst, const llama_linear& src, int rows, int K,
                          const void* gamma, int row0, int ib, int ib_stride, int perm_d, hipStream_t s) {
  if (d.q4) {
    launch_repack_bytes((uint8_t*)dst.w, (const uint8_t*)src.w, rows, K / 2, row0, ib, ib_stride, perm_d, s);
    launch_repack_bytes((uint8_t*)dst.s, (const uint8_t*)src.scales, rows, (K / 64) * 2, row0, ib, ib_stride, perm_d, s);
    launch_repack_bytes((uint8_t*)dst.b, (const uint8_t*)src.biases, rows, (K / 64) * 2, row0, ib, ib_stride, perm_d, s);
  } else if (dt == LLAMA_F32) {
    launch_repack_rows<float>((float*)dst.w, (const float*)src.w, rows, K, (const float*)gamma, row0, ib, ib_stride,
                              perm_d, 0, s);
  } else {
    launch_repack_rows<bf16_t>((bf16_t*)dst.w, (const bf16_t*)src.w, rows, K, (const bf16_t*)gamma, row0, ib,
                               ib_stride, perm_d, dst.N / 16, s);
  }
}

extern "C" llama_status llama_block_create(const llama_block_config* cfg, const llama_block_weights* w, void* dev_mem,
                                           size_t dev_bytes, void* stream, llama_block** out) {
  Dims d;
  llama_status st = check_config(cfg, &d);
  if (st != LLAMA_OK) return st;
  if (!w || !out || !dev_mem) return fail(LLAMA_ERR_INVALID_ARG, "weights, dev_mem and out must be non-NULL");
  if (!w->attention_norm || !w->ffn_norm) return fail(LLAMA_ERR_INVALID_ARG, "norm weights must be non-NULL");
  const llama_linear* ls[7] = {&w->wq, &w->wk, &w->wv, &w->wo, &w->w1, &w->w2, &w->w3};
  for (int i = 0; i < 7; ++i)
    if (!lin_ok(*ls[i], d.q4)) return fail(LLAMA_ERR_INVALID_ARG, "linear weight %d is incomplete", i);
  if (((uintptr_t)dev_mem) & 255) return fail(LLAMA_ERR_INVALID_ARG, "dev_mem must be 256-byte aligned");
  WLayout L = weight_layout(*cfg, d);
  if (dev_bytes < L.total)
    return fail(LLAMA_ERR_CAPACITY, "block memory too small: %zu < %zu bytes", dev_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)dev_mem;

  llama_block* b = new llama_block();
  b->cfg = *cfg;
  b->dm = d;
  b->rope = (float2*)(base + L.rope);
  b->gamma1 = (float*)(base + L.g1);
  b->gamma2 = (float*)(base + L.g2);
  Lin* lins[4] = {&b->qkv, &b->o, &b->w13, &b->w2};
  int NK[4][2];
  lin_shapes(d, NK);
  for (int i = 0; i < 4; ++i) {
    lins[i]->w = base + L.lin[i][0];
    lins[i]->s = d.q4 ? (bf16_t*)(base + L.lin[i][1]) : nullptr;
    lins[i]->b = d.q4 ? (bf16_t*)(base + L.lin[i][2]) : nullptr;
    lins[i]->pairs = d.q4 ? (uint32_t*)(base + L.lin[i][3]) : nullptr;
    lins[i]->N = NK[i][0];
    lins[i]->K = NK[i][1];
  }

  // RoPE table: angle = p * theta^(-2i/d), built in float64 (LLaMARoPE of page 二).
  const int half = d.d / 2;
  std::vector<float2> tab((size_t)cfg->max_seq * half);
  for (int i = 0; i < half; ++i) {
    const double w = std::pow((double)cfg->rope_theta, -2.0 * i / d.d);
    for (int p = 0; p < cfg->max_seq; ++p) {
      const double a = (double)p * w;
      tab[(size_t)p * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
  }
  hipError_t e = hipMemcpyAsync(b->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    const int dt = cfg->act_dtype;
    if (dt == LLAMA_F32) {
      launch_to_f32<float>((const float*)w->attention_norm, b->gamma1, d.D, s);
      launch_to_f32<float>((const float*)w->ffn_norm, b->gamma2, d.D, s);
    } else {
      launch_to_f32<bf16_t>((const bf16_t*)w->attention_norm, b->gamma1, d.D, s);
      launch_to_f32<bf16_t>((const bf16_t*)w->ffn_norm, b->gamma2, d.D, s);
    }
    // dense weights take the norm weight of the RMSNorm in front of them:
    // (x * r * gamma) W^T = r * (x (W diag(gamma))^T)
    const void* g1 = d.q4 ? nullptr : w->attention_norm;
    const void* g2 = d.q4 ? nullptr : w->ffn_norm;
    const int pd = cfg->rope_traditional ? d.d : 0;
    const int big = 1 << 30;
    repack_linear(d, dt, b->qkv, w->wq, d.Nq, d.D, g1, 0, big, 0, pd, s);
    repack_linear(d, dt, b->qkv, w->wk, d.Nkv, d.D, g1, d.Nq, big, 0, pd, s);
    repack_linear(d, dt, b->qkv, w->wv, d.Nkv, d.D, g1, d.Nq + d.Nkv, big, 0, 0, s);
    repack_linear(d, dt, b->o, w->wo, d.D, d.Nq, nullptr, 0, big, 0, 0, s);
    repack_linear(d, dt, b->w13, w->w1, d.F, d.D, g2, 0, d.IB, 2 * d.IB, 0, s);
    repack_linear(d, dt, b->w13, w->w3, d.F, d.D, g2, d.IB, d.IB, 2 * d.IB, 0, s);
    repack_linear(d, dt, b->w2, w->w2, d.D, d.F, nullptr, 0, big, 0, 0, s);
    if (d.q4)
      for (int i = 0; i < 4; ++i) launch_q4_pairs(lins[i]->s, lins[i]->b, lins[i]->N, lins[i]->K / 64, lins[i]->pairs, s);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete b;
    return fail(LLAMA_ERR_HIP, "block create: %s", hipGetErrorString(e));
  }
  *out = b;
  return LLAMA_OK;
}

extern "C" void llama_block_destroy(llama_block* b) { delete b; }

// ---------------------------------------------------------------- cache
struct llama_kvcache {
  llama_kvcache_config cfg;
  int pps, n_pages;
  size_t page_elems, layer_bytes;
  char* k_pool;
  char* v_pool;
  int32_t* table;
  int32_t* lens;
  std::vector<int32_t> lens_host;   // [n_layers][max_batch]
  std::vector<int32_t> table_host;
};

struct CLayout {
  size_t k, v, table, lens, total;
  int pps, n_pages;
  size_t page_elems, layer_bytes;
};

static llama_status check_cache_config(const llama_kvcache_config* c) {
  if (!c) return fail(LLAMA_ERR_INVALID_ARG, "cache config is NULL");
  if (c->n_layers <= 0 || c->max_batch <= 0 || c->max_seq <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->page_size <= 0)
    return fail(LLAMA_ERR_INVALID_ARG, "cache dimensions must be positive");
  if (c->page_size % 64) return fail(LLAMA_ERR_UNSUPPORTED, "page_size must be a multiple of 64");
  if (c->dtype != LLAMA_F32 && c->dtype != LLAMA_BF16) return fail(LLAMA_ERR_INVALID_ARG, "unknown cache dtype");
  if (c->max_batch > 256) return fail(LLAMA_ERR_UNSUPPORTED, "max_batch above 256");
  return LLAMA_OK;
}

static CLayout cache_layout(const llama_kvcache_config& c) {
  CLayout L{};
  L.pps = (c.max_seq + c.page_size - 1) / c.page_size;
  L.n_pages = c.max_batch * L.pps;
  L.page_elems = (size_t)c.n_kv_heads * c.page_size * c.head_dim;
  L.layer_bytes = (size_t)L.n_pages * L.page_elems * esize(c.dtype);
  size_t off = 0;
  L.k = off; off = align256(off + L.layer_bytes * c.n_layers);
  L.v = off; off = align256(off + L.layer_bytes * c.n_layers);
  L.table = off; off = align256(off + (size_t)L.n_pages * 4);
  L.lens = off; off = align256(off + (size_t)c.n_layers * c.max_batch * 4);
  L.total = off;
  return L;
}

extern "C" size_t llama_kvcache_bytes(const llama_kvcache_config* c) {
  if (check_cache_config(c) != LLAMA_OK) return 0;
  return cache_layout(*c).total;
}

extern "C" llama_status llama_kvcache_alloc(const llama_kvcache_config* c, void* mem, size_t bytes, void* stream,
                                           llama_kvcache** out) {
  llama_status st = check_cache_config(c);
  if (st != LLAMA_OK) return st;
  if (!mem || !out) return fail(LLAMA_ERR_INVALID_ARG, "dev_mem and out must be non-NULL");
  if (((uintptr_t)mem) & 255) return fail(LLAMA_ERR_INVALID_ARG, "dev_mem must be 256-byte aligned");
  CLayout L = cache_layout(*c);
  if (bytes < L.total) return fail(LLAMA_ERR_CAPACITY, "cache memory too small: %zu < %zu bytes", bytes, L.total);
  llama_kvcache* kc = new llama_kvcache();
  kc->cfg = *c;
  kc->pps = L.pps;
  kc->n_pages = L.n_pages;
  kc->page_elems = L.page_elems;
  kc->layer_bytes = L.layer_bytes;
  kc->k_pool = (char*)mem + L.k;
  kc->v_pool = (char*)mem + L.v;
  kc->table = (int32_t*)((char*)mem + L.table);
  kc->lens = (int32_t*)((char*)mem + L.lens);
  kc->lens_host.assign((size_t)c->n_layers * c->max_batch, 0);
  kc->table_host.resize(L.n_pages);
  for (int i = 0; i < L.n_pages; ++i) kc->table_host[i] = i;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(kc->table, kc->table_host.data(), (size_t)L.n_pages * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    launch_fill_i32(kc->lens, c->n_layers * c->max_batch, 0, s);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete kc;
    return fail(LLAMA_ERR_HIP, "cache init: %s", hipGetErrorString(e));
  }
  *out = kc;
  return LLAMA_OK;
}

extern "C" void llama_kvcache_free(llama_kvcache* c) { delete c; }

extern "C" llama_status llama_kvcache_set_block_table(llama_kvcache* c, const int32_t* t, void* stream) {
  if (!c || !t) return fail(LLAMA_ERR_INVALID_ARG, "cache and table must be non-NULL");
  std::vector<char> seen(c->n_pages, 0);
  for (int i = 0; i < c->n_pages; ++i) {
    if (t[i] < 0 || t[i] >= c->n_pages || seen[t[i]])
      return fail(LLAMA_ERR_INVALID_ARG, "block table is not a permutation of 0..%d", c->n_pages - 1);
    seen[t[i]] = 1;
  }
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(s), "set_block_table");
  HIP_TRY(hipMemcpy(c->table, t, (size_t)c->n_pages * 4, hipMemcpyHostToDevice), "set_block_table");
  c->table_host.assign(t, t + c->n_pages);
  return LLAMA_OK;
}

extern "C" llama_status llama_kvcache_set_lens(llama_kvcache* c, int32_t layer, const int32_t* lens, int32_t batch,
                                               void* stream) {
  if (!c || !lens) return fail(LLAMA_ERR_INVALID_ARG, "cache and lens must be non-NULL");
  if (layer < -1 || layer >= c->cfg.n_layers) return fail(LLAMA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (batch <= 0 || batch > c->cfg.max_batch) return fail(LLAMA_ERR_INVALID_ARG, "batch %d out of range", batch);
  for (int b = 0; b < batch; ++b)
    if (lens[b] < 0 || lens[b] > c->cfg.max_seq) return fail(LLAMA_ERR_CAPACITY, "lens[%d] = %d exceeds max_seq", b, lens[b]);
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(s), "set_lens");
  int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->cfg.n_layers : layer + 1;
  for (int l = l0; l < l1; ++l) {
    HIP_TRY(hipMemcpy(c->lens + (size_t)l * c->cfg.max_batch, lens, (size_t)batch * 4, hipMemcpyHostToDevice), "set_lens");
    std::memcpy(&c->lens_host[(size_t)l * c->cfg.max_batch], lens, (size_t)batch * 4);
  }
  return LLAMA_OK;
}

extern "C" llama_status llama_kvcache_get_lens(const llama_kvcache* c, int32_t layer, int32_t* lens, int32_t batch) {
  if (!c || !lens) return fail(LLAMA_ERR_INVALID_ARG, "cache and lens must be non-NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(LLAMA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (batch <= 0 || batch > c->cfg.max_batch) return fail(LLAMA_ERR_INVALID_ARG, "batch %d out of range", batch);
  std::memcpy(lens, &c->lens_host[(size_t)layer * c->cfg.max_batch], (size_t)batch * 4);
  return LLAMA_OK;
}

static KVView kv_view(const llama_kvcache* c, int layer) {
  KVView v;
  v.k = c->k_pool + (size_t)layer * c->layer_bytes;
  v.v = c->v_pool + (size_t)layer * c->layer_bytes;
  v.table = c->table;
  v.lens = c->lens + (size_t)layer * c->cfg.max_batch;
  v.G = c->cfg.n_kv_heads;
  v.d = c->cfg.head_dim;
  v.ps = c->cfg.page_size;
  v.pps = c->pps;
  v.tiled = c->cfg.dtype == LLAMA_BF16 && c->cfg.head_dim == 128;
  v.window = 0;
  v.cu = nullptr;
  v.n_seq = 0;
  return v;
}

static llama_status kv_copy_check(const llama_kvcache* c, int layer, int seq, int pos0, int n, const void* k,
                                  const void* v) {
  if (!c || !k || !v) return fail(LLAMA_ERR_INVALID_ARG, "cache, k and v must be non-NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(LLAMA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (seq < 0 || seq >= c->cfg.max_batch) return fail(LLAMA_ERR_INVALID_ARG, "seq %d out of range", seq);
  if (pos0 < 0 || n < 0) return fail(LLAMA_ERR_INVALID_ARG, "pos0 and n must be >= 0");
  if ((long)pos0 + n > c->cfg.max_seq) return fail(LLAMA_ERR_CAPACITY, "positions beyond max_seq");
  return LLAMA_OK;
}

extern "C" llama_status llama_kvcache_write(llama_kvcache* c, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                                            const void* k, const void* v, void* stream) {
  llama_status st = kv_copy_check(c, layer, seq, pos0, n, k, v);
  if (st != LLAMA_OK) return st;
  KVView kv = kv_view(c, layer);
  if (c->cfg.dtype == LLAMA_F32)
    launch_kv_write<float>(kv, seq, pos0, n, (const float*)k, (const float*)v, (hipStream_t)stream);
  else
    launch_kv_write<bf16_t>(kv, seq, pos0, n, (const bf16_t*)k, (const bf16_t*)v, (hipStream_t)stream);
  return hip_check("kvcache_write");
}

extern "C" llama_status llama_kvcache_read(const llama_kvcache* c, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                                           void* k, void* v, void* stream) {
  llama_status st = kv_copy_check(c, layer, seq, pos0, n, k, v);
  if (st != LLAMA_OK) return st;
  KVView kv = kv_view(c, layer);
  if (c->cfg.dtype == LLAMA_F32)
    launch_kv_read<float>(kv, seq, pos0, n, (float*)k, (float*)v, (hipStream_t)stream);
  else
    launch_kv_read<bf16_t>(kv, seq, pos0, n, (bf16_t*)k, (bf16_t*)v, (hipStream_t)stream);
  return hip_check("kvcache_read");
}

// ---------------------------------------------------------------- scratch
static const int kSplitLen = 256;  // keys per decode-attention chunk (the least)
static const int kStackSplit = 64; // keys per chunk in the stack's single-sequence decode

// Keys per decode-attention split.  Each split of a sequence and kv head
// writes n_rep rows of fp32 partial output for the merge; with grouped heads
// (n_rep > 1) the splits are lengthened until the grid is about one resident
// round of wavefronts (256 CUs x 8), which keeps that traffic small
// (measured: 70B-shaped GQA decode at batch 64, splits of 1024 keys).
static int attn_split_len(const Dims& d, int B, int maxlen) {
  if (d.n_rep == 1) return kSplitLen;
  // (query heads ride 16 to a wavefront: n_rep > 16 gives several per chunk)
  const int ns = std::max(1, 2048 / (B * d.G * ((d.n_rep + 15) / 16)));
  const int sl = (maxlen + ns - 1) / ns;
  return std::max(kSplitLen, (sl + 63) / 64 * 64);
}

// K slices of a decode GEMV (any count; slices are runs of whole 256-wide
// chunks, at least four each).  The grid is sized to one pass of blocks over
// the chip: 256 blocks (one per CU) at M > 16, whose blocks hold 64 activation
// rows, 512 at M <= 16, twice that for a K of 64 chunks or more (measured on
// the 13B- and 70B-shaped projections at M = 16 and 64: a partly filled second
// round of blocks costs more than fewer, longer slices).
static int gemv_ks(int M, int N, int K) {
  const int tiles = N / gemv_cols(M, N);
  const int nchk = tiled_chunks(K);
  const int target = (M > 16 ? 256 : 512) * (nchk >= 64 ? 2 : 1);
  return std::max(1, std::min(target / tiles, nchk / 4));
}

// 4-bit decode of one sequence runs the single-row kernels with their
// epilogues fused (every K of the block at most 32768)
static bool q4_single(const Dims& d, int T, bool decode) {
  return d.q4 && decode && T == 1 && q4_fused_blocks(d.D, d.Nq) > 0 && q4_fused_blocks(d.Nqkv, d.D) > 0 &&
         q4_fused_blocks(2 * d.F, d.D) > 0 && q4_fused_blocks(d.D, d.F) > 0;
}

struct SLayout {
  size_t inv1, inv2, ssx, ssh, q, attn, h, g, ffn, part, ao, aml, xh, xsum, deq, a16, cu, total;
  int n_splits, split_len, ks_qkv, nb_h;
};

// T = rows of this call (batch * seq_len), B = batch, decode = one-token call.
// split_min: the shortest decode-attention key split the calls will use
static SLayout scratch_layout(const llama_block_config& c, const Dims& d, int T, int B, int max_seq, bool decode,
                              int split_min = kSplitLen) {
  SLayout L{};
  const size_t E = esize(c.act_dtype);
  size_t off = 0;
  L.inv1 = off; off = align256(off + (size_t)T * 4);
  L.inv2 = off; off = align256(off + (size_t)T * 4);
  // partial row statistics: of x per K slice of the decode QKV projection (in a
  // stack's prompt pass, per 128 columns from the writer of x), of h per
  // 256-column block of the residual epilogue kernel (per 128 columns in prefill)
  // (one partial per block of the single-row 4-bit wo kernel); sized alike for
  // prefill and decode so that the buffers after it sit at the same offsets
  L.ks_qkv = gemv_ks(T, d.Nqkv, d.D);
  const int nb_q4 = d.q4 ? q4_fused_blocks(d.D, d.Nq) : 0;
  L.nb_h = q4_single(d, T, decode) ? nb_q4 : (d.D + 255) / 256;
  L.ssx = off; off = align256(off + (size_t)std::max(L.ks_qkv, (d.D + 127) / 128) * T * 4);
  L.ssh = off; off = align256(off + (size_t)std::max(nb_q4, (d.D + 127) / 128) * T * 4);
  L.q = off; off = align256(off + (size_t)T * d.Nq * E);
  L.attn = off; off = align256(off + (size_t)T * d.Nq * E);
  L.h = off; off = align256(off + (size_t)T * d.D * E);
  L.g = off; off = align256(off + (size_t)T * d.F * E);
  L.ffn = off; off = align256(off + (size_t)T * d.D * E);
  size_t part = 0;
  const int maxN = std::max(std::max(d.Nqkv, 2 * d.F), d.D);
  if (!d.bf16) {
    part = (size_t)T * maxN * 4;
  } else if (decode && !d.q4) {
    int NK[4][2];
    lin_shapes(d, NK);
    for (int i = 0; i < 4; ++i)
      part = std::max(part, (size_t)gemv_ks(T, NK[i][0], NK[i][1]) * T * NK[i][0] * 4);
  } else if (decode && d.q4) {
    part = (size_t)T * maxN * 4;
  } else {
    // prefill: wo / w2 split along K when their tile grid is small; a split
    // needs fewer than 200 tiles of 256 x 256, which bounds the rows it covers
    const long rows_split = 256L * std::max(0L, (199L * 256 / d.D));
    part = (size_t)kMaxSplitK * std::min<long>(T, rows_split) * d.D * 4;
    // 4-bit weights: up to kMaxSplitKQ4 slices while slices x tiles stay
    // within one round of 256 blocks, so at most 256 tiles of 256 x 256 fp32
    if (d.q4) part = std::max(part, std::min((size_t)kMaxSplitKQ4 * T * d.D * 4, (size_t)256 * 256 * 256 * 4));
  }
  L.part = off; off = align256(off + part);
  L.n_splits = (max_seq + split_min - 1) / split_min;
  L.split_len = split_min;
  size_t ao = (d.bf16 && decode) ? (size_t)B * d.H * L.n_splits * 128 * 4 : 0;
  size_t aml = (d.bf16 && decode) ? (size_t)B * d.H * L.n_splits * 2 * 4 : 0;
  L.ao = off; off = align256(off + ao);
  L.aml = off; off = align256(off + aml);
  const int maxK = std::max(std::max(d.D, d.Nq), d.F);
  size_t xh = (d.q4 && decode) ? (size_t)T * maxK * 2 : 0;
  size_t xs = (d.q4 && decode) ? (size_t)T * (maxK / 32) * 2 * 4 : 0;
  L.xh = off; off = align256(off + xh);
  L.xsum = off; off = align256(off + xs);
  size_t deq = 0;
  if (d.q4 && !decode) {
    int NK[4][2];
    lin_shapes(d, NK);
    for (int i = 0; i < 4; ++i) deq = std::max(deq, (size_t)NK[i][0] * tiled_chunks(NK[i][1]) * kTileK * 2);
  }
  L.deq = off; off = align256(off + deq);
  // 4-bit prompt pass: fp16 copy of a GEMM's A
  L.a16 = off; off = align256(off + ((d.q4 && !decode) ? (size_t)T * maxK * 2 : 0));
  // a ragged prefill's first row of each sequence (B + 1 entries)
  L.cu = off; off = align256(off + (decode ? 0 : (size_t)(B + 1) * 4));
  L.total = off;
  return L;
}

extern "C" size_t llama_scratch_bytes(const llama_block_config* cfg, int32_t max_tokens, int32_t max_batch,
                                      int32_t max_seq) {
  Dims d;
  if (check_config(cfg, &d) != LLAMA_OK || max_tokens < 0 || max_batch < 0 || max_seq <= 0) return 0;
  size_t a = max_tokens > 0 ? scratch_layout(*cfg, d, max_tokens, std::max(1, max_batch), max_seq, false).total : 0;
  size_t b = max_batch > 0 ? scratch_layout(*cfg, d, max_batch, max_batch, max_seq, true).total : 0;
  return std::max(a, b);
}

extern "C" llama_status llama_block_diag(const llama_block* blk, void* scratch, int32_t which, int32_t tokens,
                                         void** ptr) {
  if (!blk || !scratch || !ptr) return fail(LLAMA_ERR_INVALID_ARG, "block, scratch and ptr must be non-NULL");
  if (tokens <= 0) return fail(LLAMA_ERR_INVALID_ARG, "tokens must be positive");
  SLayout L = scratch_layout(blk->cfg, blk->dm, tokens, 1, 1, false);
  if (which == LLAMA_DIAG_ATTN) *ptr = (char*)scratch + L.attn;
  else if (which == LLAMA_DIAG_H) *ptr = (char*)scratch + L.h;
  else if (which == LLAMA_DIAG_FFN) *ptr = (char*)scratch + L.ffn;
  else return fail(LLAMA_ERR_INVALID_ARG, "unknown diagnostic %d", which);
  return LLAMA_OK;
}

extern "C" llama_status llama_block_profile_start(llama_block* blk, int32_t max_calls, uint32_t phase_mask) {
  if (!blk || max_calls <= 0) return fail(LLAMA_ERR_INVALID_ARG, "block must be non-NULL and max_calls > 0");
  blk->prof_mask = phase_mask;
  const size_t need = (size_t)max_calls * kMaxMarks;
  while (blk->ev.size() < need) {
    hipEvent_t e;
    // timing-only events: no system-scope fence (no cache write-back between kernels)
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableSystemFence), "profile_start");
    blk->ev.push_back(e);
  }
  blk->prof_max = max_calls;
  blk->prof_calls = 0;
  blk->prof_marks = 0;
  return LLAMA_OK;
}

extern "C" llama_status llama_block_profile_read(llama_block* blk, float* ms, int32_t max_phases, int32_t* n_phases,
                                                 int32_t* n_calls) {
  if (!blk || !ms || !n_phases || !n_calls) return fail(LLAMA_ERR_INVALID_ARG, "NULL argument");
  const int np = std::max(0, std::min(blk->prof_marks - 1, (int)max_phases));
  for (int p = 0; p < np; ++p) ms[p] = 0.f;
  for (int c = 0; c < blk->prof_calls; ++c) {
    hipEvent_t* e = &blk->ev[(size_t)c * kMaxMarks];
    HIP_TRY(hipDeviceSynchronize(), "profile_read");
    for (int p = 0; p < np; ++p) {
      if (blk->prof_mask && !((blk->prof_mask >> p) & 1u)) continue;
      float t = 0.f;
      HIP_TRY(hipEventElapsedTime(&t, e[p], e[p + 1]), "profile_read");
      ms[p] += t;
    }
  }
  *n_phases = np;
  *n_calls = blk->prof_calls;
  blk->prof_max = blk->prof_calls = 0;
  return LLAMA_OK;
}

extern "C" llama_status llama_block_set_diag(llama_block* blk, int32_t enable) {
  if (!blk) return fail(LLAMA_ERR_INVALID_ARG, "block is NULL");
  blk->diag = enable ? 1 : 0;
  return LLAMA_OK;
}

// ---------------------------------------------------------------- block calls
// Ls (ragged prefill): new tokens of each sequence, each >= 0; else L each.
static llama_status check_call(const llama_block* blk, const llama_kvcache* c, int layer, const void* x, const void* y,
                               int batch, int L, const int32_t* Ls, void* scratch, size_t sbytes, bool decode,
                               int split_min, SLayout* lay) {
  if (!blk || !c) return fail(LLAMA_ERR_INVALID_ARG, "block and cache must be non-NULL");
  if (!x || !y || !scratch) return fail(LLAMA_ERR_INVALID_ARG, "x, y and scratch must be non-NULL");
  if (((uintptr_t)scratch) & 255) return fail(LLAMA_ERR_INVALID_ARG, "scratch must be 256-byte aligned");
  const Dims& d = blk->dm;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(LLAMA_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (batch <= 0 || batch > c->cfg.max_batch)
    return fail(LLAMA_ERR_INVALID_ARG, "batch %d outside 1..%d", batch, c->cfg.max_batch);
  long T = 0;
  if (Ls) {
    for (int b = 0; b < batch; ++b) {
      if (Ls[b] < 0) return fail(LLAMA_ERR_INVALID_ARG, "seq_lens[%d] = %d is negative", b, Ls[b]);
      T += Ls[b];
    }
    if (T <= 0) return fail(LLAMA_ERR_INVALID_ARG, "seq_lens are all 0: no tokens to prefill");
  } else {
    if (L <= 0) return fail(LLAMA_ERR_INVALID_ARG, "seq_len must be positive");
    T = (long)batch * L;
  }
  if (T > (1L << 30)) return fail(LLAMA_ERR_UNSUPPORTED, "%ld tokens in one call", T);
  if (c->cfg.n_kv_heads != d.G || c->cfg.head_dim != d.d || c->cfg.dtype != blk->cfg.act_dtype)
    return fail(LLAMA_ERR_INVALID_ARG, "cache (kv heads %d, head_dim %d, dtype %d) does not match the block",
                c->cfg.n_kv_heads, c->cfg.head_dim, c->cfg.dtype);
  if (decode && d.q4 && batch > 4) return fail(LLAMA_ERR_UNSUPPORTED, "4-bit decode supports batch <= 4");
  if (decode && d.bf16 && !d.q4 && batch > 64) return fail(LLAMA_ERR_UNSUPPORTED, "bf16 decode supports batch <= 64");
  const int cap = std::min(c->cfg.max_seq, blk->cfg.max_seq);
  int maxlen = 0;
  for (int b = 0; b < batch; ++b) {
    const int len = c->lens_host[(size_t)layer * c->cfg.max_batch + b], n = Ls ? Ls[b] : L;
    if ((long)len + n > cap)
      return fail(LLAMA_ERR_CAPACITY, "sequence %d: %d cached + %d new exceeds capacity %d", b, len, n, cap);
    maxlen = std::max(maxlen, len + n);
  }
  SLayout lo = scratch_layout(blk->cfg, d, (int)T, batch, c->cfg.max_seq, decode, split_min);
  if (sbytes < lo.total) return fail(LLAMA_ERR_CAPACITY, "scratch too small: %zu < %zu bytes", sbytes, lo.total);
  // (a sliding window: the splits cover the window, from its start rounded
  // down to a 64-key step)
  const int W = blk->cfg.sliding_window;
  const int span = W > 0 ? std::min(maxlen, W + 64) : maxlen;
  lo.split_len = attn_split_len(d, batch, span);
  lo.n_splits = (span + lo.split_len - 1) / lo.split_len;
  *lay = lo;
  return LLAMA_OK;
}

// M rows; L rows per sequence, or (ragged, kv.cu set) the most of any sequence
template <typename T>
static void fp32_path(const llama_block* blk, KVView kv, const void* x, void* y, int B, int L, int M, char* sc,
                      const SLayout& S, Marker& mk, hipStream_t s) {
  const Dims& d = blk->dm;
  float* inv1 = (float*)(sc + S.inv1);
  T* q = (T*)(sc + S.q);
  T* attn = (T*)(sc + S.attn);
  T* h = (T*)(sc + S.h);
  T* g = (T*)(sc + S.g);
  float* part = (float*)(sc + S.part);
  const float eps = blk->cfg.norm_eps;
  mk(s);
  launch_rms_inv<T>((const T*)x, M, d.D, eps, inv1, s);
  mk(s);
  launch_gemm_simt<T>((const T*)x, (const T*)blk->qkv.w, part, M, d.Nqkv, d.D, s);
  mk(s);
  RowStat st1;
  st1.inv = inv1;
  launch_epi_qkv<T>(part, 1, M, d.Nq, d.Nkv, st1, L, blk->rope, blk->cfg.rope_traditional, q, kv, s);
  mk(s);
  launch_attn_simt<T>(q, kv, M, L, d.H, d.G, d.d, attn, s);
  mk(s);
  launch_gemm_simt<T>(attn, (const T*)blk->o.w, part, M, d.D, d.Nq, s);
  mk(s);
  float* ssh = (float*)(sc + S.ssh);
  launch_epi_resid<T>(part, 1, M, d.D, (const T*)x, h, ssh, nullptr, 0, 0, nullptr, s);
  mk(s);
  launch_gemm_simt<T>(h, (const T*)blk->w13.w, part, M, 2 * d.F, d.D, s);
  mk(s);
  RowStat st2;
  st2.ss = ssh; st2.nb = S.nb_h; st2.M = M; st2.n = d.D; st2.eps = eps;
  launch_epi_swiglu<T>(part, 1, M, 2 * d.F, d.IB, st2, g, s);
  mk(s);
  launch_gemm_simt<T>(g, (const T*)blk->w2.w, part, M, d.D, d.F, s);
  mk(s);
  launch_epi_resid<T>(part, 1, M, d.D, h, (T*)y, nullptr, kv.lens, L, B, blk->diag ? (T*)(sc + S.ffn) : nullptr, s,
                      kv.cu);
  mk(s);
}

// A 4-bit block whose W2 product splits K (its residual then runs as a kernel
// of its own) and whose QKV product reads fp16 A: in a stack's prompt pass the
// W2 residual kernel can write the next block's fp16 A, y * gamma1 (next).
static bool q4_x16_chain(const Dims& d, int M) {
  return d.q4 && gemm_q4_direct_ok(M, d.D, d.F) && gemm_split_k_q4(M, d.D, d.F) > 1 &&
         gemm_q4_direct_ok(M, d.Nqkv, d.D);
}

// xstat bit 0: x's sums of squares per 128 columns are already in S.ssx (from
// the writer of x), so RMSNorm #1 needs no statistic pass; bit 1: the W2
// residual epilogue writes y's there for the next block; bit 2 (with
// next_g1, honoured when q4_x16_chain holds): it also writes fp16(y * next_g1)
// to the fp16 A buffer; bit 3: that buffer already holds fp16(x * gamma1)
static void bf16_prefill(const llama_block* blk, KVView kv, const void* x, void* y, int B, int L, int M, char* sc,
                         const SLayout& S, Marker& mk, hipStream_t s, int xstat, const float* next_g1) {
  const Dims& d = blk->dm;
  float* inv1 = (float*)(sc + S.inv1);
  float* inv2 = (float*)(sc + S.inv2);
  bf16_t* q = (bf16_t*)(sc + S.q);
  bf16_t* attn = (bf16_t*)(sc + S.attn);
  bf16_t* h = (bf16_t*)(sc + S.h);
  bf16_t* g = (bf16_t*)(sc + S.g);
  _Float16* deq = (_Float16*)(sc + S.deq);
  _Float16* a16 = (_Float16*)(sc + S.a16);
  const float eps = blk->cfg.norm_eps;
  // 4-bit weights run on fp16 MFMA.  Where the shape allows, the GEMM
  // dequantizes the codes itself and A is copied to fp16 with the norm weight
  // applied (x * gamma, one rounding); else the weights are dequantized (gamma
  // folded) to fp16 right before the GEMM, tiled for the direct-to-LDS tiles
  // when A can be copied to fp16 too.
  // a_ready: the fp16 copy of A (gamma applied) is already in a16
  auto operands = [&](GemmArgs& g, const bf16_t* A, const Lin& lin, const float* gamma, bool a_ready = false) {
    g.A = A;
    if (!d.q4) {
      g.B = (const bf16_t*)lin.w;
      return;
    }
    g.b_f16 = 1;
    if (gemm_q4_direct_ok(M, lin.N, lin.K)) {
      g.a_f16 = 1;
      g.q4w = (const uint32_t*)lin.w;
      g.q4sb = lin.pairs;
      g.B = nullptr;
      if (!a_ready) launch_bf16_to_f16(A, a16, (size_t)M * lin.K, s, gamma, lin.K);
      g.A = (const bf16_t*)a16;
      return;
    }
    g.a_f16 = gemm_f16_direct_ok(M, lin.N, lin.K);
    launch_q4_dequant((const uint32_t*)lin.w, lin.s, lin.b, lin.N, lin.K, 64, gamma, g.a_f16, deq, s);
    g.B = (const bf16_t*)deq;
    if (g.a_f16) {
      launch_bf16_to_f16(A, a16, (size_t)M * lin.K, s);
      g.A = (const bf16_t*)a16;
    }
  };
  // row statistics as partial sums of squares per 128 columns, at most
  // kGemmMaxRowPartials per row
  const bool stat128 = d.D % 128 == 0 && d.D / 128 <= kGemmMaxRowPartials;
  float* ssx = (float*)(sc + S.ssx);
  const bool x_in = stat128 && (xstat & 1);
  mk(s);
  if (!x_in) launch_rms_inv<bf16_t>((const bf16_t*)x, M, d.D, eps, inv1, s);
  mk(s);
  GemmArgs a{};
  operands(a, (const bf16_t*)x, blk->qkv, blk->gamma1, (xstat & 8) != 0 && q4_x16_chain(d, M));
  a.M = M; a.N = d.Nqkv; a.K = d.D;
  if (x_in) {
    a.rstat.ss = ssx; a.rstat.nb = d.D / 128; a.rstat.M = M; a.rstat.n = d.D; a.rstat.eps = eps;
  } else {
    a.inv_rms = inv1;
  }
  a.q_out = q; a.Nq = d.Nq; a.Nkv = d.Nkv; a.L = L;
  a.rope = blk->rope; a.traditional = blk->cfg.rope_traditional;
  a.kv = kv;
  launch_gemm_mfma(EPI_QKV, a, s);
  mk(s);
  launch_attn_prefill_bf16(q, kv, B, L, d.H, d.G, attn, s);
  mk(s);
  // wo and w2 (N = dim) give few output tiles at small T: there the K range is
  // split, every slice writes fp32 partials and the residual epilogue kernel
  // adds them (in slice order) to the residual.
  float* part = (float*)(sc + S.part);
  // ss_out (optional): the stored rows' sums of squares per 128 columns
  // out16 / gamma16 (optional): with a K split, the residual kernel also writes
  // fp16(out * gamma16) there; returns whether it did
  auto resid_gemm = [&](const bf16_t* A, const Lin& lin, const bf16_t* resid, bf16_t* out, int K, int32_t* lens_add,
                        int lens_inc, bf16_t* branch, float* ss_out, _Float16* out16 = nullptr,
                        const float* gamma16 = nullptr) {
    GemmArgs g{};
    operands(g, A, lin, nullptr);
    g.M = M; g.N = d.D; g.K = K;
    const int ks = g.q4w ? gemm_split_k_q4(M, d.D, K) : gemm_split_k(M, d.D, K, g.b_f16 && !g.a_f16);
    if (ks > 1) {
      g.C = part; g.ksplit = ks;
      launch_gemm_mfma(EPI_F32, g, s);
      launch_epi_resid<bf16_t>(part, ks, M, d.D, resid, out, ss_out, lens_add, lens_inc, B, branch, s, kv.cu, 1,
                               out16, gamma16);
      return out16 != nullptr;
    }
    g.resid = resid; g.out = out; g.lens_add = lens_add; g.lens_inc = lens_inc; g.n_seq = B; g.branch = branch;
    g.lens_cu = kv.cu; g.ss_out = ss_out;
    launch_gemm_mfma(EPI_RESID, g, s);
    return false;
  };
  // RMSNorm #2's statistic comes from the Wo epilogue (the rows' sums of
  // squares as stored), reduced by the W1/W3 GEMM into its row scales; a model
  // dim past 64 partials per row falls back to a statistic pass over h
  float* ssh = (float*)(sc + S.ssh);
  // (4-bit W1/W3 on the direct path: its fp16 A, h * gamma2, comes from the
  // Wo residual kernel when Wo splits K)
  const bool h16 = d.q4 && gemm_q4_direct_ok(M, 2 * d.F, d.D);
  const bool h16_done = resid_gemm(attn, blk->o, (const bf16_t*)x, h, d.Nq, nullptr, 0, nullptr,
                                   stat128 ? ssh : nullptr, h16 ? a16 : nullptr, blk->gamma2);
  if (!stat128) launch_rms_inv<bf16_t>(h, M, d.D, eps, inv2, s);
  mk(s);
  GemmArgs f{};
  operands(f, h, blk->w13, blk->gamma2, h16_done);
  f.M = M; f.N = 2 * d.F; f.K = d.D;
  f.g_out = g;
  if (stat128) {
    f.rstat.ss = ssh; f.rstat.nb = d.D / 128; f.rstat.M = M; f.rstat.n = d.D; f.rstat.eps = eps;
  } else {
    f.inv_rms = inv2;
  }
  launch_gemm_mfma(EPI_SWIGLU, f, s);
  mk(s);
  const bool x16 = (xstat & 4) && next_g1 && q4_x16_chain(d, M);
  resid_gemm(g, blk->w2, h, (bf16_t*)y, d.F, kv.lens, L, blk->diag ? (bf16_t*)(sc + S.ffn) : nullptr,
             stat128 && (xstat & 2) ? ssx : nullptr, x16 ? a16 : nullptr, next_g1);
  mk(s);
}

static void bf16_decode(const llama_block* blk, KVView kv, const void* x, void* y, int B, char* sc, const SLayout& S,
                        int n_splits, int split_len, Marker& mk, hipStream_t s) {
  const Dims& d = blk->dm;
  bf16_t* q = (bf16_t*)(sc + S.q);
  bf16_t* attn = (bf16_t*)(sc + S.attn);
  bf16_t* h = (bf16_t*)(sc + S.h);
  bf16_t* g = (bf16_t*)(sc + S.g);
  float* part = (float*)(sc + S.part);
  float* ao = (float*)(sc + S.ao);
  float* aml = (float*)(sc + S.aml);
  float* ssx = (float*)(sc + S.ssx);
  float* ssh = (float*)(sc + S.ssh);
  bf16_t* ffn = blk->diag ? (bf16_t*)(sc + S.ffn) : nullptr;
  const float eps = blk->cfg.norm_eps;
  RowStat none;
  RowStat sth;  // statistic of h from the wo residual epilogue
  sth.ss = ssh; sth.nb = S.nb_h; sth.M = B; sth.n = d.D; sth.eps = eps;
  mk(s);
  if (!d.q4) {
    // the QKV projection also emits sum(x^2) per K slice: attention_norm's statistic
    int ks = gemv_ks(B, d.Nqkv, d.D);
    launch_gemv_bf16((const bf16_t*)x, (const bf16_t*)blk->qkv.w, true, part, B, d.Nqkv, d.D, ks, ssx, s);
    mk(s);
    RowStat stx;
    stx.ss = ssx; stx.nb = ks; stx.M = B; stx.n = d.D; stx.eps = eps;
    launch_epi_qkv<bf16_t>(part, ks, B, d.Nq, d.Nkv, stx, 1, blk->rope, blk->cfg.rope_traditional, q, kv, s);
    mk(s);
    launch_attn_decode_bf16(q, kv, B, d.H, d.G, n_splits, split_len, ao, aml, attn, s);
    mk(s);
    ks = gemv_ks(B, d.D, d.Nq);
    launch_gemv_bf16(attn, (const bf16_t*)blk->o.w, true, part, B, d.D, d.Nq, ks, nullptr, s);
    mk(s);
    launch_epi_resid<bf16_t>(part, ks, B, d.D, (const bf16_t*)x, h, ssh, nullptr, 0, 0, nullptr, s);
    mk(s);
    // enough column tiles to fill the chip unsplit: SwiGLU in the GEMV itself
    ks = gemv_ks(B, 2 * d.F, d.D);
    if (ks == 1) {
      GemvSwiglu sw{};
      sw.stat = sth; sw.ib = d.IB; sw.g_out = g;
      launch_gemv_swiglu(h, (const bf16_t*)blk->w13.w, B, 2 * d.F, d.D, sw, s);
    } else {
      launch_gemv_bf16(h, (const bf16_t*)blk->w13.w, true, part, B, 2 * d.F, d.D, ks, nullptr, s);
      launch_epi_swiglu<bf16_t>(part, ks, B, 2 * d.F, d.IB, sth, g, s);
    }
    mk(s);
    ks = gemv_ks(B, d.D, d.F);
    launch_gemv_bf16(g, (const bf16_t*)blk->w2.w, true, part, B, d.D, d.F, ks, nullptr, s);
    mk(s);
    launch_epi_resid<bf16_t>(part, ks, B, d.D, h, (bf16_t*)y, nullptr, kv.lens, 1, B, ffn, s);
    mk(s);
  } else if (q4_single(d, B, true)) {
    // one sequence: each projection and what follows it in one kernel
    auto lin_q4 = [&](const Lin& lin, Q4Fused e, const bf16_t* X) {
      e.N = lin.N;
      e.K = lin.K;
      e.eps = eps;
      launch_q4_fused(X, (const uint32_t*)lin.w, lin.s, lin.b, e, s);
      mk(s);
    };
    Q4Fused e{};
    e.epi = Q4E_QKV; e.norm = 1; e.gamma = blk->gamma1;
    e.Nq = d.Nq; e.Nkv = d.Nkv; e.rope = blk->rope; e.traditional = blk->cfg.rope_traditional; e.q_out = q;
    e.kv = kv;
    lin_q4(blk->qkv, e, (const bf16_t*)x);
    launch_attn_decode_bf16(q, kv, B, d.H, d.G, n_splits, split_len, ao, aml, attn, s);
    mk(s);
    e = Q4Fused{};
    e.epi = Q4E_RESID; e.resid = (const bf16_t*)x; e.out = h; e.ss_out = ssh;
    lin_q4(blk->o, e, attn);
    e = Q4Fused{};
    e.epi = Q4E_SWIGLU; e.norm = 2; e.stat = sth; e.gamma = blk->gamma2; e.ib = d.IB; e.g_out = g;
    lin_q4(blk->w13, e, h);
    e = Q4Fused{};
    e.epi = Q4E_RESID; e.resid = h; e.out = (bf16_t*)y; e.lens_add = kv.lens; e.branch = ffn;
    lin_q4(blk->w2, e, g);
  } else {
    _Float16* xh = (_Float16*)(sc + S.xh);
    float* xs = (float*)(sc + S.xsum);
    auto gq = [&](const bf16_t* X, int norm, RowStat st, const float* gam, const Lin& lin) {
      launch_gemv_q4(X, norm, st, eps, gam, (const uint32_t*)lin.w, lin.s, lin.b, part, B, lin.N, lin.K, 64, xh, xs,
                     s);
    };
    gq((const bf16_t*)x, 1, none, blk->gamma1, blk->qkv);
    mk(s);
    launch_epi_qkv<bf16_t>(part, 1, B, d.Nq, d.Nkv, none, 1, blk->rope, blk->cfg.rope_traditional,
                           q, kv, s);
    mk(s);
    launch_attn_decode_bf16(q, kv, B, d.H, d.G, n_splits, split_len, ao, aml, attn, s);
    mk(s);
    gq(attn, 0, none, nullptr, blk->o);
    mk(s);
    launch_epi_resid<bf16_t>(part, 1, B, d.D, (const bf16_t*)x, h, ssh, nullptr, 0, 0, nullptr, s);
    mk(s);
    gq(h, 2, sth, blk->gamma2, blk->w13);
    mk(s);
    launch_epi_swiglu<bf16_t>(part, 1, B, 2 * d.F, d.IB, none, g, s);
    mk(s);
    gq(g, 0, none, nullptr, blk->w2);
    mk(s);
    launch_epi_resid<bf16_t>(part, 1, B, d.D, h, (bf16_t*)y, nullptr, kv.lens, 1, B, ffn, s);
    mk(s);
  }
}

// Enqueue one block call.  n_splits_override > 0 fixes the decode attention
// grid, with splits of kSplitLen keys (graph capture, where lengths grow
// between replays).
// Ls (prefill only, may be null): a ragged call's new tokens per sequence.
static llama_status enqueue(llama_block* blk, llama_kvcache* c, int layer, const void* x, void* y, int batch, int L,
                            void* scratch, size_t sbytes, bool decode, int n_splits_override, int split_len_override,
                            hipStream_t s, const int32_t* Ls = nullptr, int xstat = 0,
                            const float* next_g1 = nullptr) {
  SLayout S;
  llama_status st = check_call(blk, c, layer, x, y, batch, L, Ls, scratch, sbytes, decode,
                               n_splits_override > 0 ? split_len_override : kSplitLen, &S);
  if (st != LLAMA_OK) return st;
  if (plan_log_on())
    plan_log("block %s: layer %d, %d sequences, %s, %s weights%s; decode attention %d splits of %d keys",
             decode ? "decode" : "prefill", layer, batch,
             Ls ? "ragged new-token counts" : decode ? "one token each" : "equal new-token counts",
             blk->dm.q4 ? "4-bit" : blk->dm.bf16 ? "bf16" : "fp32", xstat ? ", x statistic from its writer" : "",
             S.n_splits, S.split_len);
  KVView kv = kv_view(c, layer);
  kv.window = blk->cfg.sliding_window;
  char* sc = (char*)scratch;
  int M = batch * L;
  if (Ls) {
    // the rows' sequence map goes to the device with the call (in a kernel's
    // arguments, so nothing on the host has to outlive the call)
    std::vector<int32_t> cu(batch + 1, 0);
    L = 0;
    for (int b = 0; b < batch; ++b) {
      cu[b + 1] = cu[b] + Ls[b];
      L = std::max(L, (int)Ls[b]);
    }
    M = cu[batch];
    kv.cu = (const int32_t*)(sc + S.cu);
    kv.n_seq = batch;
    launch_set_i32(cu.data(), batch + 1, (int32_t*)(sc + S.cu), s);
  }
  const Dims& d = blk->dm;
  Marker mk;
  if (blk->prof_calls < blk->prof_max) {
    mk.ev = &blk->ev[(size_t)(blk->prof_calls++) * kMaxMarks];
    mk.mask = blk->prof_mask;
    // phases whose kernels take launch-attached events: the w1/w3 GEMM of the
    // bf16 prefill (phase 4) and the decode attention (phase 2)
    const uint32_t clockable = !d.bf16 ? 0u : decode ? (1u << 2) : (1u << 4);
    if (mk.mask != 0 && (mk.mask & (mk.mask - 1)) == 0 && (mk.mask & clockable)) mk.clocked = __builtin_ctz(mk.mask);
  }
  if (!d.bf16) {
    fp32_path<float>(blk, kv, x, y, batch, L, M, sc, S, mk, s);
  } else if (!decode) {
    bf16_prefill(blk, kv, x, y, batch, L, M, sc, S, mk, s, xstat, next_g1);
  } else {
    if (n_splits_override > 0) bf16_decode(blk, kv, x, y, batch, sc, S, n_splits_override, split_len_override, mk, s);
    else bf16_decode(blk, kv, x, y, batch, sc, S, S.n_splits, S.split_len, mk, s);
  }
  if (mk.ev) blk->prof_marks = mk.i;
  g_clock = LaunchClock{};
  st = hip_check(decode ? "block decode" : "block prefill");
  if (st != LLAMA_OK) return st;
  for (int b = 0; b < batch; ++b) c->lens_host[(size_t)layer * c->cfg.max_batch + b] += Ls ? Ls[b] : L;
  return LLAMA_OK;
}

extern "C" llama_status llama_block_prefill(llama_block* blk, llama_kvcache* c, int32_t layer, const void* x, void* y,
                                            int32_t batch, int32_t seq_len, void* scratch, size_t sbytes, void* stream) {
  TraceRange trace_("llama_block_prefill");
  return enqueue(blk, c, layer, x, y, batch, seq_len, scratch, sbytes, false, 0, 0, (hipStream_t)stream);
}

extern "C" llama_status llama_block_prefill_ragged(llama_block* blk, llama_kvcache* c, int32_t layer, const void* x,
                                                   void* y, int32_t batch, const int32_t* seq_lens, void* scratch,
                                                   size_t sbytes, void* stream) {
  TraceRange trace_("llama_block_prefill_ragged");
  if (!seq_lens) return fail(LLAMA_ERR_INVALID_ARG, "seq_lens must be non-NULL");
  if (batch > kMaxSetI32 - 1) return fail(LLAMA_ERR_UNSUPPORTED, "ragged prefill of more than %d sequences", kMaxSetI32 - 1);
  return enqueue(blk, c, layer, x, y, batch, 1, scratch, sbytes, false, 0, 0, (hipStream_t)stream, seq_lens);
}

extern "C" llama_status llama_block_decode(llama_block* blk, llama_kvcache* c, int32_t layer, const void* x, void* y,
                                           int32_t batch, void* scratch, size_t sbytes, void* stream) {
  TraceRange trace_("llama_block_decode");
  return enqueue(blk, c, layer, x, y, batch, 1, scratch, sbytes, true, 0, 0, (hipStream_t)stream);
}

// ---------------------------------------------------------------- decode without allocation
// The transient values of llama_block_decode_noalloc live in this file-scope
// device array instead of a caller's scratch buffer.  Every device the library
// runs on holds its own copy from the code object's load until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory:
// host code uses only the address hipGetSymbolAddress returns for the current
// device (noalloc_scratch below).  Nothing in a decode reads scratch before the
// same call wrote it, so it needs no clearing between calls.
static constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static constexpr int kMaxDevices = 64;
static void* g_noalloc_ptr[kMaxDevices];
static std::mutex g_noalloc_mu;

// Device address of `scratch` on the current device, looked up once per device.
static llama_status noalloc_scratch(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "no-allocation decode: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LLAMA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "no-allocation decode: hipGetSymbolAddress");
    if (!p) return fail(LLAMA_ERR_HIP, "no-allocation decode: no device address for the scratch array");
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return LLAMA_OK;
}

extern "C" llama_status llama_block_decode_noalloc(llama_block* blk, llama_kvcache* c, int32_t layer, const void* x,
                                                   void* y, int32_t batch, void* stream) {
  TraceRange trace_("llama_block_decode_noalloc");
  if (!blk || !c) return fail(LLAMA_ERR_INVALID_ARG, "block and cache must be non-NULL");
  if (batch > 0) {
    const size_t need = scratch_layout(blk->cfg, blk->dm, batch, batch, c->cfg.max_seq, true).total;
    if (need > kNoAllocScratchBytes)
      return fail(LLAMA_ERR_CAPACITY,
                  "no-allocation decode: %d sequences against a %d-position cache need %zu bytes of scratch, "
                  "more than its fixed %zu bytes (use llama_block_decode with a scratch buffer)",
                  batch, c->cfg.max_seq, need, kNoAllocScratchBytes);
  }
  void* sc = nullptr;
  llama_status st = noalloc_scratch(&sc);
  if (st != LLAMA_OK) return st;
  return enqueue(blk, c, layer, x, y, batch, 1, sc, kNoAllocScratchBytes, true, 0, 0, (hipStream_t)stream);
}

// ---------------------------------------------------------------- stack ends
extern "C" llama_status llama_embed(const void* table, int32_t vocab, int32_t dim, int32_t dtype, const int32_t* ids,
                                    int32_t n, void* out, void* stream) {
  TraceRange trace_("llama_embed");
  if (!table || !ids || !out) return fail(LLAMA_ERR_INVALID_ARG, "table, ids and out must be non-NULL");
  if (vocab <= 0 || dim <= 0 || n < 0) return fail(LLAMA_ERR_INVALID_ARG, "vocab and dim must be positive, n >= 0");
  if (dtype == LLAMA_F32)
    launch_embed<float>((const float*)table, vocab, dim, ids, n, (float*)out, (hipStream_t)stream);
  else if (dtype == LLAMA_BF16)
    launch_embed<bf16_t>((const bf16_t*)table, vocab, dim, ids, n, (bf16_t*)out, (hipStream_t)stream);
  else
    return fail(LLAMA_ERR_INVALID_ARG, "unknown dtype");
  return hip_check("embed");
}

struct HLayout {
  size_t inv, gam, xn, logits, part, xh, xsum, total;
};
static HLayout head_layout(int B, int D, int V) {
  HLayout L{};
  size_t off = 0;
  L.inv = off; off = align256(off + (size_t)B * 4);
  L.gam = off; off = align256(off + (size_t)D * 4);
  L.xn = off; off = align256(off + (size_t)B * D * 4);
  L.logits = off; off = align256(off + (size_t)B * V * 4);
  L.part = off; off = align256(off + (size_t)B * V * 4);
  L.xh = off; off = align256(off + (size_t)B * D * 2);
  L.xsum = off; off = align256(off + (size_t)B * (D / 32 + 1) * 2 * 4);
  L.total = off;
  return L;
}

extern "C" size_t llama_head_scratch_bytes(int32_t batch, int32_t dim, int32_t vocab) {
  if (batch <= 0 || dim <= 0 || vocab <= 0) return 0;
  return head_layout(batch, dim, vocab).total;
}

// The next-id rule of the generate loop: temperature <= 0 = greedy, else a draw
// (u[*u_off]) from the nucleus of softmax(logits / temperature).
struct Sampling {
  float temperature = 0.f, top_p = 1.f;
  const float* u = nullptr;
  const int32_t* u_off = nullptr;
};

static llama_status head_enqueue(const llama_linear* head, int wf, int gs, int dt, const void* fnorm, float eps,
                                 const void* x, int B, int D, int V, float* logits, int32_t* ids, void* scratch,
                                 size_t sbytes, hipStream_t s, const Sampling& smp = Sampling()) {
  if (!head || !head->w || !fnorm || !x || !ids || !scratch)
    return fail(LLAMA_ERR_INVALID_ARG, "head, final_norm, x, ids and scratch must be non-NULL");
  if (B <= 0 || D <= 0 || V <= 0) return fail(LLAMA_ERR_INVALID_ARG, "batch, dim and vocab must be positive");
  if (wf == LLAMA_W_Q4) {
    if (dt != LLAMA_BF16 || gs != 64 || D % 64 || B > 4 || !head->scales || !head->biases)
      return fail(LLAMA_ERR_UNSUPPORTED, "4-bit head needs bf16 activations, group 64, dim % 64 == 0, batch <= 4");
  } else if (wf != LLAMA_W_DENSE) {
    return fail(LLAMA_ERR_INVALID_ARG, "unknown weight_format");
  }
  if (dt != LLAMA_F32 && dt != LLAMA_BF16) return fail(LLAMA_ERR_INVALID_ARG, "unknown act_dtype");
  if (wf == LLAMA_W_DENSE && dt == LLAMA_BF16 && (D % 32 || V % 64))
    return fail(LLAMA_ERR_UNSUPPORTED, "dense bf16 head needs dim % 32 == 0 and vocab % 64 == 0");
  HLayout L = head_layout(B, D, V);
  if (sbytes < L.total) return fail(LLAMA_ERR_CAPACITY, "head scratch too small: %zu < %zu", sbytes, L.total);
  char* sc = (char*)scratch;
  float* out = logits ? logits : (float*)(sc + L.logits);
  if (wf == LLAMA_W_Q4) {
    float* gam = (float*)(sc + L.gam);
    launch_to_f32<bf16_t>((const bf16_t*)fnorm, gam, D, s);
    launch_gemv_q4((const bf16_t*)x, 1, RowStat(), eps, gam, (const uint32_t*)head->w, (const bf16_t*)head->scales,
                   (const bf16_t*)head->biases, out, B, V, D, gs, (_Float16*)(sc + L.xh), (float*)(sc + L.xsum), s);
  } else if (dt == LLAMA_F32) {
    launch_rmsnorm_apply<float>((const float*)x, (const float*)fnorm, B, D, eps, (float*)(sc + L.xn), s);
    launch_gemm_simt<float>((const float*)(sc + L.xn), (const float*)head->w, out, B, V, D, s);
  } else {
    launch_rmsnorm_apply<bf16_t>((const bf16_t*)x, (const bf16_t*)fnorm, B, D, eps, (bf16_t*)(sc + L.xn), s);
    launch_gemv_bf16((const bf16_t*)(sc + L.xn), (const bf16_t*)head->w, false, out, B, V, D, 1, nullptr, s);
  }
  if (smp.temperature > 0.f) launch_sample(out, B, V, smp.temperature, smp.top_p, smp.u, smp.u_off, ids, s);
  else launch_argmax(out, B, V, ids, s);
  return hip_check("lm_head_argmax");
}

extern "C" llama_status llama_lm_head_argmax(const llama_linear* head, int32_t wf, int32_t gs, int32_t dt,
                                             const void* fnorm, float eps, const void* x, int32_t B, int32_t D,
                                             int32_t V, float* logits, int32_t* ids, void* scratch, size_t sbytes,
                                             void* stream) {
  TraceRange trace_("llama_lm_head_argmax");
  return head_enqueue(head, wf, gs, dt, fnorm, eps, x, B, D, V, logits, ids, scratch, sbytes, (hipStream_t)stream);
}

extern "C" llama_status llama_sample(const float* logits, int32_t batch, int32_t vocab, float temperature,
                                     float top_p, const float* u, int32_t* ids, void* stream) {
  TraceRange trace_("llama_sample");
  if (!logits || !ids || (temperature > 0.f && !u))
    return fail(LLAMA_ERR_INVALID_ARG, "logits, ids and (temperature > 0) u must be non-NULL");
  if (batch <= 0 || vocab <= 0) return fail(LLAMA_ERR_INVALID_ARG, "batch and vocab must be positive");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(LLAMA_ERR_INVALID_ARG, "top_p must lie in (0, 1]");
  if (temperature != temperature) return fail(LLAMA_ERR_INVALID_ARG, "temperature is NaN");
  launch_sample(logits, batch, vocab, temperature, top_p, u, nullptr, ids, (hipStream_t)stream);
  return hip_check("sample");
}

// ---------------------------------------------------------------- greedy generate
// The generation loop of "生成过程" (MLX page): the prompt pass fills every
// layer's cache and yields the first id; each decode step embeds the newest id
// (read on the device, never copied to the host), runs every block on its cache
// and yields the next.  One decode step is captured into a HIP graph and replayed.
struct llama_stack {
  std::vector<llama_block*> blocks;
  const void* emb;
  int vocab;
  const void* fnorm;
  llama_linear head;
  Sampling smp;     // u_off is filled in by generate
};

extern "C" llama_status llama_stack_create(llama_block* const* blocks, int32_t n_layers, const void* embedding,
                                           int32_t vocab, const void* final_norm, const llama_linear* output,
                                           llama_stack** out) {
  if (!blocks || n_layers <= 0 || !embedding || !final_norm || !output || !output->w || !out || vocab <= 0)
    return fail(LLAMA_ERR_INVALID_ARG, "stack: NULL argument or non-positive size");
  for (int i = 0; i < n_layers; ++i) {
    if (!blocks[i]) return fail(LLAMA_ERR_INVALID_ARG, "stack: block %d is NULL", i);
    const llama_block_config &a = blocks[0]->cfg, &b = blocks[i]->cfg;
    if (std::memcmp(&a, &b, sizeof a)) return fail(LLAMA_ERR_INVALID_ARG, "stack: block %d has another config", i);
  }
  const llama_block_config& c = blocks[0]->cfg;
  if (c.act_dtype != LLAMA_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "stack: bf16 activations only");
  if (c.weight_format == LLAMA_W_Q4 && (!output->scales || !output->biases))
    return fail(LLAMA_ERR_INVALID_ARG, "stack: 4-bit head needs scales and biases");
  llama_stack* st = new llama_stack();
  st->blocks.assign(blocks, blocks + n_layers);
  st->emb = embedding;
  st->vocab = vocab;
  st->fnorm = final_norm;
  st->head = *output;
  *out = st;
  return LLAMA_OK;
}

extern "C" void llama_stack_destroy(llama_stack* st) { delete st; }

struct StLayout {
  size_t x, blk, head, cur, cursor, seq, total, blk_bytes, head_bytes;
};
static StLayout stack_layout(const llama_stack* st, int max_prompt, int max_seq) {
  const llama_block_config& c = st->blocks[0]->cfg;
  StLayout L{};
  size_t off = 0;
  L.x = off; off = align256(off + (size_t)max_prompt * c.dim * 2);
  const Dims& d = st->blocks[0]->dm;
  L.blk_bytes = std::max(scratch_layout(c, d, max_prompt, 1, max_seq, false).total,
                         scratch_layout(c, d, 1, 1, max_seq, true, kStackSplit).total);
  L.blk = off; off = align256(off + L.blk_bytes);
  L.head_bytes = head_layout(1, c.dim, st->vocab).total;
  L.head = off; off = align256(off + L.head_bytes);
  L.cur = off; off = align256(off + 4);
  L.cursor = off; off = align256(off + 4);
  // the growing sequence of the recompute loop: up to max_prompt ids
  L.seq = off; off = align256(off + ((size_t)max_prompt + 1) * 4);
  L.total = off;
  return L;
}

extern "C" llama_status llama_stack_set_sampling(llama_stack* st, float temperature, float top_p, const float* u) {
  if (!st) return fail(LLAMA_ERR_INVALID_ARG, "stack must be non-NULL");
  if (temperature > 0.f && !u) return fail(LLAMA_ERR_INVALID_ARG, "temperature > 0 needs the draws u");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(LLAMA_ERR_INVALID_ARG, "top_p must lie in (0, 1]");
  if (temperature != temperature) return fail(LLAMA_ERR_INVALID_ARG, "temperature is NaN");
  st->smp.temperature = temperature;
  st->smp.top_p = top_p;
  st->smp.u = temperature > 0.f ? u : nullptr;
  return LLAMA_OK;
}

extern "C" size_t llama_stack_scratch_bytes(const llama_stack* st, int32_t max_prompt, int32_t max_seq) {
  if (!st || max_prompt <= 0 || max_seq <= 0) return 0;
  return stack_layout(st, max_prompt, max_seq).total;
}

// A stack's prompt pass hands each block the statistic of its input: the
// embedding writes x's sums of squares per 128 columns into the block scratch
// where the first block's prefill reads them, and every block's W2 epilogue
// writes them for the next (model dims up to 64 partials per row).  Returns
// where they go in the block scratch of a T-row pass, or null without them.
static float* stack_x_stats(const llama_stack* st, void* bs, int T) {
  const Dims& d = st->blocks[0]->dm;
  if (!d.bf16 || d.D % 128 != 0 || d.D / 128 > kGemmMaxRowPartials) return nullptr;
  return (float*)((char*)bs + scratch_layout(st->blocks[0]->cfg, d, T, 1, st->blocks[0]->cfg.max_seq, false).ssx);
}

// prompt-pass flags of layer l over n rows (bf16_prefill's xstat): statistics
// of x from its writer when xs; with 4-bit layers whose W2 residual runs as a
// kernel of its own, each layer's fp16 A written by the layer before it
static int stack_xstat(const llama_stack* st, int l, int n, bool xs) {
  const int NL = (int)st->blocks.size();
  int f = xs ? 1 | (l + 1 < NL ? 2 : 0) : 0;
  if (q4_x16_chain(st->blocks[l]->dm, n)) {
    if (l + 1 < NL) f |= 4;
    if (l > 0) f |= 8;
  }
  return f;
}

extern "C" llama_status llama_stack_generate(llama_stack* st, llama_kvcache* cache, const int32_t* prompt, int32_t P,
                                             int32_t n_steps, int32_t* ids_out, float* logits_out, void* scratch,
                                             size_t sbytes, int32_t use_graph, void* stream) {
  TraceRange trace_("llama_stack_generate");
  if (!st || !cache || !prompt || !ids_out || !scratch)
    return fail(LLAMA_ERR_INVALID_ARG, "stack, cache, prompt, ids_out and scratch must be non-NULL");
  if (P <= 0 || n_steps < 0) return fail(LLAMA_ERR_INVALID_ARG, "prompt_len must be > 0 and n_steps >= 0");
  hipStream_t s = (hipStream_t)stream;
  if (use_graph && !s) return fail(LLAMA_ERR_INVALID_ARG, "graph capture needs a non-null stream");
  const int NL = (int)st->blocks.size();
  const llama_block_config& c = st->blocks[0]->cfg;
  if (cache->cfg.n_layers < NL) return fail(LLAMA_ERR_INVALID_ARG, "cache has %d layers, stack %d", cache->cfg.n_layers, NL);
  for (int l = 0; l < NL; ++l)
    if (cache->lens_host[(size_t)l * cache->cfg.max_batch] != 0)
      return fail(LLAMA_ERR_INVALID_ARG, "cache layer %d of sequence 0 is not empty", l);
  const int cap = std::min(cache->cfg.max_seq, c.max_seq);
  if ((long)P + n_steps > cap) return fail(LLAMA_ERR_CAPACITY, "prompt + steps (%d) exceed capacity %d", P + n_steps, cap);
  StLayout L = stack_layout(st, P, cache->cfg.max_seq);
  if (sbytes < L.total) return fail(LLAMA_ERR_CAPACITY, "stack scratch too small: %zu < %zu", sbytes, L.total);
  char* sc = (char*)scratch;
  bf16_t* x = (bf16_t*)(sc + L.x);
  void* bs = sc + L.blk;
  void* hs = sc + L.head;
  int32_t* cur = (int32_t*)(sc + L.cur);
  int32_t* cursor = (int32_t*)(sc + L.cursor);
  float* hlog = (float*)((char*)hs + head_layout(1, c.dim, st->vocab).logits);
  const int D = c.dim, V = st->vocab;
  llama_status r;
  auto head = [&](const bf16_t* row) {
    // (the draw of emitted id j is u[j]: the cursor counts the ids emitted so far)
    Sampling smp = st->smp;
    smp.u_off = cursor;
    return head_enqueue(&st->head, c.weight_format, c.group_size, LLAMA_BF16, st->fnorm, c.norm_eps, row, 1, D, V,
                        hlog, cur, hs, L.head_bytes, s, smp);
  };

  launch_fill_i32(cursor, 1, 0, s);
  float* xs = stack_x_stats(st, bs, P);
  launch_embed<bf16_t>((const bf16_t*)st->emb, V, D, prompt, P, x, s, xs);
  for (int l = 0; l < NL; ++l) {
    const int xstat = stack_xstat(st, l, P, xs != nullptr);
    if ((r = enqueue(st->blocks[l], cache, l, x, x, 1, P, bs, L.blk_bytes, false, 0, 0, s, nullptr, xstat,
                     l + 1 < NL ? st->blocks[l + 1]->gamma1 : nullptr)) != LLAMA_OK)
      return r;
  }
  if ((r = head(x + (size_t)(P - 1) * D)) != LLAMA_OK) return r;
  launch_emit(cur, ids_out, cursor, hlog, logits_out, V, s);

  // one sequence: short key splits (more wavefronts for a short cache), fixed
  // for the whole capture
  const int Wst = c.sliding_window;
  const int span = Wst > 0 ? std::min(P + n_steps, Wst + 64) : P + n_steps;
  const int n_splits = (span + kStackSplit - 1) / kStackSplit;
  auto step = [&]() -> llama_status {
    launch_embed<bf16_t>((const bf16_t*)st->emb, V, D, cur, 1, x, s);
    for (int l = 0; l < NL; ++l) {
      llama_status q = enqueue(st->blocks[l], cache, l, x, x, 1, 1, bs, L.blk_bytes, true, n_splits, kStackSplit, s);
      if (q != LLAMA_OK) return q;
    }
    llama_status q = head(x);
    if (q != LLAMA_OK) return q;
    launch_emit(cur, ids_out, cursor, hlog, logits_out, V, s);
    return hip_check("decode step");
  };
  if (n_steps > 0) {
    if (use_graph) {
      hipGraph_t graph = nullptr;
      hipGraphExec_t exec = nullptr;
      HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "begin capture");
      llama_status q = step();
      hipError_t e = hipStreamEndCapture(s, &graph);
      if (q != LLAMA_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return q;
      }
      if (e != hipSuccess) return fail(LLAMA_ERR_HIP, "end capture: %s", hipGetErrorString(e));
      e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      if (e == hipSuccess)
        for (int i = 0; i < n_steps && e == hipSuccess; ++i) e = hipGraphLaunch(exec, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (exec) (void)hipGraphExecDestroy(exec);
      (void)hipGraphDestroy(graph);
      if (e != hipSuccess) return fail(LLAMA_ERR_HIP, "graph replay: %s", hipGetErrorString(e));
    } else {
      for (int i = 0; i < n_steps; ++i)
        if ((r = step()) != LLAMA_OK) return r;
    }
  }
  HIP_TRY(hipStreamSynchronize(s), "generate");
  for (int l = 0; l < NL; ++l) cache->lens_host[(size_t)l * cache->cfg.max_batch] = P + n_steps;
  return LLAMA_OK;
}

// The loop without the cache's reuse (LLaMA.generate on page 二 runs the model
// over the whole sequence for every new token; the reading-notes page times
// generation with and without the KV cache, "流处理与 KV Cache"): each emitted
// id re-runs the prompt pass over the prompt and the ids so far, from an empty
// cache; the ids stay on the device.
extern "C" llama_status llama_stack_generate_recompute(llama_stack* st, llama_kvcache* cache, const int32_t* prompt,
                                                       int32_t P, int32_t n_steps, int32_t* ids_out,
                                                       float* logits_out, void* scratch, size_t sbytes,
                                                       void* stream) {
  TraceRange trace_("llama_stack_generate_recompute");
  if (!st || !cache || !prompt || !ids_out || !scratch)
    return fail(LLAMA_ERR_INVALID_ARG, "stack, cache, prompt, ids_out and scratch must be non-NULL");
  if (P <= 0 || n_steps < 0) return fail(LLAMA_ERR_INVALID_ARG, "prompt_len must be > 0 and n_steps >= 0");
  hipStream_t s = (hipStream_t)stream;
  const int NL = (int)st->blocks.size();
  const llama_block_config& c = st->blocks[0]->cfg;
  if (cache->cfg.n_layers < NL) return fail(LLAMA_ERR_INVALID_ARG, "cache has %d layers, stack %d", cache->cfg.n_layers, NL);
  const int cap = std::min(cache->cfg.max_seq, c.max_seq);
  const int Pmax = P + n_steps;
  if ((long)Pmax > cap) return fail(LLAMA_ERR_CAPACITY, "prompt + steps (%d) exceed capacity %d", Pmax, cap);
  StLayout L = stack_layout(st, Pmax, cache->cfg.max_seq);
  if (sbytes < L.total) return fail(LLAMA_ERR_CAPACITY, "stack scratch too small: %zu < %zu", sbytes, L.total);
  char* sc = (char*)scratch;
  bf16_t* x = (bf16_t*)(sc + L.x);
  void* bs = sc + L.blk;
  void* hs = sc + L.head;
  int32_t* cur = (int32_t*)(sc + L.cur);
  int32_t* cursor = (int32_t*)(sc + L.cursor);
  int32_t* seq = (int32_t*)(sc + L.seq);
  float* hlog = (float*)((char*)hs + head_layout(1, c.dim, st->vocab).logits);
  const int D = c.dim, V = st->vocab, MB = cache->cfg.max_batch;
  HIP_TRY(hipMemcpyAsync(seq, prompt, (size_t)P * 4, hipMemcpyDeviceToDevice, s), "recompute prompt copy");
  launch_fill_i32(cursor, 1, 0, s);
  for (int t = 0; t <= n_steps; ++t) {
    const int n = P + t;
    // an empty cache for sequence 0 in every layer
    launch_fill_strided_i32(cache->lens, NL, MB, 0, s);
    for (int l = 0; l < NL; ++l) cache->lens_host[(size_t)l * MB] = 0;
    float* xs = stack_x_stats(st, bs, n);
    launch_embed<bf16_t>((const bf16_t*)st->emb, V, D, seq, n, x, s, xs);
    for (int l = 0; l < NL; ++l) {
      const int xstat = stack_xstat(st, l, n, xs != nullptr);
      llama_status r = enqueue(st->blocks[l], cache, l, x, x, 1, n, bs, L.blk_bytes, false, 0, 0, s, nullptr, xstat,
                               l + 1 < NL ? st->blocks[l + 1]->gamma1 : nullptr);
      if (r != LLAMA_OK) return r;
    }
    Sampling smp = st->smp;
    smp.u_off = cursor;
    llama_status r = head_enqueue(&st->head, c.weight_format, c.group_size, LLAMA_BF16, st->fnorm, c.norm_eps,
                                  x + (size_t)(n - 1) * D, 1, D, V, hlog, cur, hs, L.head_bytes, s, smp);
    if (r != LLAMA_OK) return r;
    // emitted id t -> seq[P + t] (the next pass's last token) and logits row t
    launch_emit(cur, seq + P, cursor, hlog, logits_out, V, s);
  }
  HIP_TRY(hipMemcpyAsync(ids_out, seq + P, (size_t)(n_steps + 1) * 4, hipMemcpyDeviceToDevice, s), "recompute ids");
  HIP_TRY(hipStreamSynchronize(s), "generate (recompute)");
  return LLAMA_OK;
}

/*
 * llama_block.h -- C ABI of the MI355X (gfx950) LLaMA-style pre-norm decoder block.
 *
 * One block computes, for every new token t of every sequence b
 * (LLaMABlock / LLaMAAttention / LLaMAMLP / LLaMARMSNorm / LLaMARoPE in section 二
 * of the page "LLaMA架构深度解析：从开源大模型设计到高效推理的工程实现全流程"; the
 * module tree and "核心模块实现" 2-5 of the page "iOS设备上运行LLaMA2-13B：基于苹果
 * MLX框架的完整技术指南"; the data flow of "老码农和你一起学AI系列：关于LLaMA解码器"):
 *
 *     xn = attention_norm(x)            RMSNorm: x / sqrt(mean(x^2) + eps) * gamma
 *     q, k, v = wq xn, wk xn, wv xn      no bias, nn.Linear [out, in] weights
 *     q, k = RoPE(q, k, position)       position = tokens already cached + index
 *     cache[b] += (k, v)                cache holds rotated keys
 *     o = softmax(q k^T / sqrt(d)) v    causal, kv head = query head / (H / G)
 *     h = x + wo o
 *     y = h + w2( silu(w1 n) * (w3 n) ),  n = ffn_norm(h)
 *
 * Prefill runs this over a whole prompt at once; decode runs it for one new token
 * per sequence against the cache ("第三章" and "流处理与 KV Cache" of the page
 * "《Hands-On Large Language Models》阅读笔记(二)").
 *
 * Conventions for every entry point
 *  - Pointers named *_dev are device pointers (HIP device memory on the current
 *    device); pointers named *_host are host pointers.  Weight, activation and
 *    cache pointers are device pointers.  The library never allocates device
 *    memory: the caller passes every buffer, and owns it.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; no entry point synchronises the device unless stated.
 *  - Every call validates its arguments on the host before enqueuing anything.
 *    A failed call returns a negative llama_status, enqueues no work and leaves
 *    caches, lengths and outputs unchanged; llama_last_error() then describes it.
 *    A HIP error seen at launch returns LLAMA_ERR_HIP.  Errors of earlier
 *    asynchronous work surface at a later synchronisation, not here.
 *  - Activation dtype is LLAMA_F32 (fp32) or LLAMA_BF16 (bf16, fp32 accumulate).
 *  - Nothing in the library is thread-safe against concurrent calls on the same
 *    handle; distinct handles may be used from distinct threads.
 *  - Tracing: every block, stack, head, sampling and embedding entry point opens
 *    a roctx range named after itself (seen by rocprofv3 --marker-trace); with
 *    the environment variable LLAMA_LOG set to a value other than 0 the library
 *    prints each launch plan it picks to stderr (read once per process).
 */
#ifndef LLAMA_BLOCK_H_
#define LLAMA_BLOCK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLAMA_OK = 0,
  LLAMA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shape */
  LLAMA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. head_dim 96 in bf16) */
  LLAMA_ERR_CAPACITY = -3,      /* cache or scratch too small for the request */
  LLAMA_ERR_HIP = -4            /* a HIP runtime call failed */
} llama_status;

enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 };            /* activation / dense weight dtype */
enum { LLAMA_W_DENSE = 0, LLAMA_W_Q4 = 1 };         /* weight format */

/* Block hyper-parameters, named as the pages name them (config.json of the MLX
 * page: dim, n_heads, norm_eps; LLaMAConfig of page 二: num_kv_heads,
 * intermediate_size, rope_theta; RoPE(128, traditional=True) of the MLX module
 * tree for the pair layout).
 *   head_dim = dim / n_heads.  fp32: head_dim in {64, 128}; bf16: head_dim 128,
 *   dim % 64 == 0, ffn_dim % 64 == 0.  n_heads % n_kv_heads == 0.
 *   rope_traditional: 1 = rotate adjacent pairs (2i, 2i+1); 0 = rotate pairs
 *   (i, i + head_dim/2).  Both use angle = position * rope_theta^(-2i/head_dim).
 *   weight_format LLAMA_W_Q4 (bf16 activations only): every linear weight is 4-bit
 *   group-affine, W = scale * code + bias per group of group_size (= 64) inputs.
 *   max_seq: positions 0 .. max_seq-1 may occur (sizes the RoPE table).
 *   sliding_window: 0 = every query attends all keys up to its position; W > 0 =
 *   only the W most recent positions, its own included (sliding-window attention,
 *   named in "流处理与 KV Cache" of the reading-notes page without a window rule;
 *   the cache still keeps every position). */
typedef struct {
  int32_t dim, n_heads, n_kv_heads, ffn_dim;
  float norm_eps, rope_theta;
  int32_t rope_traditional;
  int32_t act_dtype;
  int32_t weight_format, group_size;
  int32_t max_seq;
  int32_t sliding_window;
} llama_block_config;

/* One linear weight [out, in] (nn.Linear convention).
 *   dense: w = act_dtype [out, in] row-major; scales = biases = NULL.
 *   q4:    w = uint32 [out, in/8], code k of a row at bits 4*(k%8) of word k/8
 *          (unsigned 0..15); scales, biases = bf16 [out, in/group_size]. */
typedef struct {
  const void *w, *scales, *biases;
} llama_linear;

/* attention_norm, ffn_norm: act_dtype [dim] (bf16 for q4). */
typedef struct {
  const void *attention_norm, *ffn_norm;
  llama_linear wq, wk, wv, wo, w1, w2, w3;
} llama_block_weights;

typedef struct llama_block llama_block;
typedef struct llama_kvcache llama_kvcache;
typedef struct llama_stack llama_stack;

/* ------------------------------------------------------------------ block */

/* Bytes of device memory a block keeps for its repacked weights and RoPE table.
 * Returns 0 for an invalid config. */
size_t llama_block_weight_bytes(const llama_block_config* cfg);

/* Repack the weights into dev_mem (>= llama_block_weight_bytes bytes, 256-byte
 * aligned): wq/wk/wv concatenated, w1/w3 interleaved, norm weights folded into
 * the dense weights that follow them, a float64-built RoPE table.  Enqueued on
 * `stream` and then waited for (the source weights may be freed on return).
 * *out receives a host handle; dev_mem must outlive it. */
llama_status llama_block_create(const llama_block_config* cfg, const llama_block_weights* weights,
                                void* dev_mem, size_t dev_bytes, void* stream, llama_block** out);
void llama_block_destroy(llama_block* blk);

/* Bytes of scratch device memory a prefill of up to max_tokens tokens (batch *
 * seq_len) or a decode of up to max_batch sequences needs, for a cache of up to
 * max_seq positions.  Scratch holds only transient values: one scratch buffer
 * may serve any number of blocks whose calls are ordered on one stream. */
size_t llama_scratch_bytes(const llama_block_config* cfg, int32_t max_tokens, int32_t max_batch,
                           int32_t max_seq);

/* Prefill: x, y = act_dtype [batch, seq_len, dim] device buffers (y may alias x).
 * Token l of sequence b sits at position lens[layer][b] + l; its key and value
 * are appended to the cache, every query attends causally to all cached keys up
 * to its own position, and lens[layer][b] grows by seq_len.
 * Errors: LLAMA_ERR_CAPACITY if lens + seq_len exceeds the cache's max_seq or
 * the scratch is smaller than llama_scratch_bytes(cfg, batch*seq_len, batch, max_seq). */
llama_status llama_block_prefill(llama_block* blk, llama_kvcache* cache, int32_t layer, const void* x,
                                 void* y, int32_t batch, int32_t seq_len, void* scratch,
                                 size_t scratch_bytes, void* stream);

/* Ragged prefill: the sequences of one call bring different numbers of new
 * tokens (a chunked prefill of several prompts at once).  The position of a new
 * token is the number of tokens its sequence has cached plus its index
 * ("2. 注意力机制" on the MLX page: RoPE offset = cache length, new keys and
 * values appended), so every sequence continues from its own lens[layer][b].
 *   seq_lens_host: int32 [batch] host array, seq_lens_host[b] >= 0 new tokens of
 *   sequence b (0 = the sequence is left untouched); T = their sum, T > 0.
 *   x, y = act_dtype [T, dim] device buffers (y may alias x), packed: sequence
 *   b's tokens are rows off_b .. off_b + seq_lens_host[b] - 1, with off_b the sum
 *   of the counts before b.
 * Token l of sequence b sits at position lens[layer][b] + l, attends causally to
 * every cached key up to its position, and lens[layer][b] grows by
 * seq_lens_host[b].  The call reads seq_lens_host before it returns.
 * Errors: LLAMA_ERR_INVALID_ARG for a NULL seq_lens_host, a negative count or a
 * zero total; LLAMA_ERR_CAPACITY if some lens + count exceeds max_seq or the
 * scratch is smaller than llama_scratch_bytes(cfg, T, batch, max_seq). */
llama_status llama_block_prefill_ragged(llama_block* blk, llama_kvcache* cache, int32_t layer, const void* x,
                                        void* y, int32_t batch, const int32_t* seq_lens_host, void* scratch,
                                        size_t scratch_bytes, void* stream);

/* Decode: x, y = act_dtype [batch, dim] (y may alias x); sequence b's token sits
 * at position lens[layer][b], attends to keys 0 .. lens[layer][b] and is
 * appended; lens[layer][b] grows by 1.  Same errors as prefill. */
llama_status llama_block_decode(llama_block* blk, llama_kvcache* cache, int32_t layer, const void* x,
                                void* y, int32_t batch, void* scratch, size_t scratch_bytes,
                                void* stream);

/* Decode without a scratch buffer, for callers that cannot allocate device
 * memory (code under HIP graph capture, fixed serving loops, harnesses that
 * forbid allocation): the same computation, kernels and results as
 * llama_block_decode, with its transient values in a fixed 64 MiB array that
 * the library keeps on each device it runs on until the process ends.  Every
 * call on a device shares that device's array: calls that overlap on one device
 * (concurrent streams, threads) race and must be ordered by the caller.  No
 * allocation happens inside the call.  Same arguments (minus the scratch) and
 * errors as llama_block_decode, plus LLAMA_ERR_CAPACITY when the call would need
 * more than the 64 MiB (about: 64 sequences of a dim-8192 block against a
 * 4.2k-position cache fit; llama_scratch_bytes(cfg, 0, batch, max_seq) gives the
 * need). */
llama_status llama_block_decode_noalloc(llama_block* blk, llama_kvcache* cache, int32_t layer, const void* x,
                                        void* y, int32_t batch, void* stream);

/* Diagnostics: after a prefill/decode call with the same token count and
 * scratch, points *ptr at a transient of that call inside scratch:
 *   LLAMA_DIAG_ATTN = attention output before wo, act_dtype [tokens, n_heads*head_dim];
 *   LLAMA_DIAG_H    = x + wo o, act_dtype [tokens, dim];
 *   LLAMA_DIAG_FFN  = the feed-forward branch w2(silu(w1 n) * (w3 n)) before the
 *                     residual add, act_dtype [tokens, dim]; written only while
 *                     llama_block_set_diag(blk, 1) is in effect (one extra store).
 * Valid until the next call using scratch. */
enum { LLAMA_DIAG_ATTN = 0, LLAMA_DIAG_H = 1, LLAMA_DIAG_FFN = 2 };
llama_status llama_block_diag(const llama_block* blk, void* scratch, int32_t which, int32_t tokens,
                              void** ptr);
llama_status llama_block_set_diag(llama_block* blk, int32_t enable);

/* Per-phase timing (profiling aid).  profile_start arms HIP events for the next
 * max_calls prefill/decode calls of this block: each call records an event on its
 * stream at the boundaries of the phases selected by phase_mask (bit p = phase p;
 * 0 = every phase).  Each event costs a few microseconds of stream time, so a
 * mask with one phase disturbs the timing least.  profile_read waits for the
 * device, writes the summed milliseconds of each phase over the recorded calls to
 * phase_ms[0 .. *n_phases) (at most max_phases; 0 for phases not selected), the
 * number of calls to *n_calls, and disarms.  Phases, in launch order:
 *   bf16 prefill : rms(x), qkv gemm+rope+append, attention, wo gemm+residual
 *                  (+ h statistics), w1/w3 gemm+swiglu, w2 gemm+residual    (6)
 *   fp32         : rms(x), qkv projection, qkv finish, attention, wo projection,
 *                  residual, w1/w3 projection, swiglu, w2 projection, residual (10)
 *   bf16 decode  : qkv projection (+ x statistics), qkv finish, attention,
 *                  wo projection, residual (+ h statistics), w1/w3
 *                  projection + swiglu, w2 projection, residual             (8)
 *   4-bit decode : one sequence: qkv projection+rope+append, attention, wo
 *                  projection+residual, w1/w3 projection+swiglu, w2
 *                  projection+residual (5); more: as bf16 decode, the w1/w3
 *                  projection and swiglu apart                              (9)
 * Not for calls captured into a graph. */
llama_status llama_block_profile_start(llama_block* blk, int32_t max_calls, uint32_t phase_mask);
llama_status llama_block_profile_read(llama_block* blk, float* phase_ms, int32_t max_phases, int32_t* n_phases,
                                      int32_t* n_calls);

/* ------------------------------------------------------------------ cache */

/* The KV cache of "2. 注意力机制" (MLX page): per layer, the rotated keys and the
 * values of every position a sequence has seen, new positions appended at the
 * end (the position offset of a new token is the cache's length).  Here it is
 * preallocated and paged instead of concatenated.
 * Paged KV cache: per layer a pool of pages; page p of layer l holds, for every
 * kv head g, page_size positions of keys as [g][slot][head_dim] and of values
 * transposed as [g][head_dim][slot].  A block table [max_batch][pages_per_seq]
 * (pages_per_seq = ceil(max_seq / page_size)) maps a sequence's logical page to
 * a physical page (identity after init); lens [n_layers][max_batch] on the
 * device count the cached positions, mirrored on the host for validation.
 * page_size must be a multiple of 64.  dtype = LLAMA_F32 | LLAMA_BF16. */
typedef struct {
  int32_t n_layers, max_batch, max_seq, n_kv_heads, head_dim, page_size, dtype;
} llama_kvcache_config;

size_t llama_kvcache_bytes(const llama_kvcache_config* cfg);

/* Lay the cache out in dev_mem (>= llama_kvcache_bytes, 256-byte aligned): identity
 * block table, all lens 0.  Enqueued on stream and waited for. */
llama_status llama_kvcache_alloc(const llama_kvcache_config* cfg, void* dev_mem, size_t dev_bytes,
                                 void* stream, llama_kvcache** out);
void llama_kvcache_free(llama_kvcache* cache);

/* Replace the block table (table_host: int32 [max_batch][pages_per_seq], a
 * permutation of 0 .. max_batch*pages_per_seq-1).  Copied synchronously. */
llama_status llama_kvcache_set_block_table(llama_kvcache* cache, const int32_t* table_host, void* stream);

/* Set lens[layer][0..batch) (host values, each <= max_seq); copied synchronously.
 * layer = -1 sets every layer. */
llama_status llama_kvcache_set_lens(llama_kvcache* cache, int32_t layer, const int32_t* lens_host,
                                    int32_t batch, void* stream);

/* Host mirror of lens[layer][0..batch). */
llama_status llama_kvcache_get_lens(const llama_kvcache* cache, int32_t layer, int32_t* lens_host,
                                    int32_t batch);

/* Copy n positions pos0 .. pos0+n-1 of sequence `seq` between the paged cache and
 * dense device buffers k_dev, v_dev = dtype [n, n_kv_heads, head_dim] (keys as
 * stored, i.e. after RoPE).  write does not change lens; read reads whatever the
 * slots hold.  Positions must lie below max_seq. */
llama_status llama_kvcache_write(llama_kvcache* cache, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                                 const void* k_dev, const void* v_dev, void* stream);
llama_status llama_kvcache_read(const llama_kvcache* cache, int32_t layer, int32_t seq, int32_t pos0,
                                int32_t n, void* k_dev, void* v_dev, void* stream);

/* ------------------------------------------------------------ stack ends */

/* Embedding lookup ("1. 嵌入层" of the MLX page): out[i] = table[ids_dev[i]],
 * table = dtype [vocab, dim], out = dtype [n, dim].  ids outside [0, vocab) give
 * a zero row. */
llama_status llama_embed(const void* table, int32_t vocab, int32_t dim, int32_t dtype,
                         const int32_t* ids_dev, int32_t n, void* out, void* stream);

/* Final RMSNorm, output head and greedy choice (module tree of the MLX page;
 * argmax at temperature 0, "生成过程"): for each of `batch` rows of x
 * (act_dtype [batch, dim]), logits = head(final_norm(x)) in fp32 and
 * ids_dev[b] = the index of the largest logit, lowest index on ties.
 * head: dense act_dtype [vocab, dim] or q4 (weight_format); final_norm:
 * act_dtype [dim].  logits_dev (fp32 [batch, vocab]) may be NULL.
 * scratch: >= llama_head_scratch_bytes(batch, dim, vocab).  4-bit heads: batch <= 4. */
size_t llama_head_scratch_bytes(int32_t batch, int32_t dim, int32_t vocab);
llama_status llama_lm_head_argmax(const llama_linear* head, int32_t weight_format, int32_t group_size,
                                  int32_t act_dtype, const void* final_norm, float eps, const void* x,
                                  int32_t batch, int32_t dim, int32_t vocab, float* logits_dev,
                                  int32_t* ids_dev, void* scratch, size_t scratch_bytes, void* stream);

/* Sampled next id ("生成过程", MLX page: greedy argmax at temperature 0, a
 * multinomial draw from softmax(logits / temperature) above it; LLaMA.generate,
 * page 二: the draw limited to the nucleus, the most probable tokens up to and
 * including the first at which their cumulative probability exceeds top_p).
 * logits_dev: fp32 [batch, vocab]; u_dev: fp32 [batch] draws in [0, 1) (the
 * caller's random numbers; unused and may be NULL at temperature <= 0);
 * ids_dev: int32 [batch].  Row b takes the first index, in vocabulary order, at
 * which the cumulative kept probability exceeds u_dev[b] times the kept
 * probability; tokens tied with the last nucleus token are kept; top_p = 1 keeps
 * every token.  Temperature <= 0: the argmax, lowest index on ties.
 * Errors: LLAMA_ERR_INVALID_ARG for NULL pointers, batch or vocab <= 0, top_p
 * outside (0, 1], or a NaN temperature. */
llama_status llama_sample(const float* logits_dev, int32_t batch, int32_t vocab, float temperature, float top_p,
                          const float* u_dev, int32_t* ids_dev, void* stream);

/* ------------------------------------------------------- greedy generate */

/* A stack of n_layers blocks (same config) + embedding + final norm + head,
 * driving the generation loop of "生成过程" (MLX page): the prompt pass fills
 * every layer's cache and emits the first id; each of n_steps decode steps
 * embeds the newest id (read on the device), runs every block, and emits the
 * next id.  The decode step is captured once into a HIP graph and replayed.
 * blocks: n_layers handles (kept, not owned).  cache: n_layers layers, batch 1. */
llama_status llama_stack_create(llama_block* const* blocks, int32_t n_layers, const void* embedding,
                                int32_t vocab, const void* final_norm, const llama_linear* output,
                                llama_stack** out);
void llama_stack_destroy(llama_stack* st);

/* Next-id rule of later llama_stack_generate calls: temperature <= 0 (the
 * default) = greedy; above 0, the draw of llama_sample with u_dev[j] for the
 * j-th emitted id (j = 0 from the prompt pass), u_dev: fp32 [n_steps + 1] on the
 * device, read during generate (kept, not owned).  Errors as llama_sample. */
llama_status llama_stack_set_sampling(llama_stack* st, float temperature, float top_p, const float* u_dev);

/* Scratch for llama_stack_generate with a prompt of up to max_prompt tokens. */
size_t llama_stack_scratch_bytes(const llama_stack* st, int32_t max_prompt, int32_t max_seq);

/* prompt_dev: int32 [prompt_len] device ids; ids_out_dev: int32 [n_steps + 1];
 * logits_out_dev: fp32 [n_steps + 1, vocab] or NULL.  The cache's lens for
 * sequence 0 must be 0 in every layer on entry.  use_graph = 0 launches each
 * step's kernels directly (same results).  stream must not be the null stream
 * when use_graph = 1.  Synchronises the stream before returning. */
llama_status llama_stack_generate(llama_stack* st, llama_kvcache* cache, const int32_t* prompt_dev,
                                  int32_t prompt_len, int32_t n_steps, int32_t* ids_out_dev,
                                  float* logits_out_dev, void* scratch, size_t scratch_bytes,
                                  int32_t use_graph, void* stream);

/* The same loop without reusing the cache (LLaMA.generate on page 二 re-runs
 * the model over the whole sequence for each new token; "流处理与 KV Cache" on
 * the reading-notes page times generation with and without the cache): emitted
 * id j re-runs the prompt pass over the prompt and ids 0 .. j-1 from an empty
 * cache (sequence 0's lens set to 0 in every layer first).  Same arguments and
 * next-id rule as llama_stack_generate; scratch >= llama_stack_scratch_bytes(st,
 * prompt_len + n_steps, max_seq).  Kernels are launched directly (no graph).
 * On return the cache holds the last pass: prompt_len + n_steps positions. */
llama_status llama_stack_generate_recompute(llama_stack* st, llama_kvcache* cache, const int32_t* prompt_dev,
                                            int32_t prompt_len, int32_t n_steps, int32_t* ids_out_dev,
                                            float* logits_out_dev, void* scratch, size_t scratch_bytes,
                                            void* stream);

/* ------------------------------------------------------ measurement aid */

/* Not part of the block: a loop of bf16 matrix-core instructions on register
 * operands (no memory traffic), `blocks` workgroups of 4 wavefronts, each
 * wavefront issuing 8 * iters v_mfma_f32_32x32x16_bf16 (32768 flops each), to
 * time the rate the matrix cores sustain on this part beside the published
 * peak.  sink_dev: fp32 [blocks * 256] device buffer that receives the
 * accumulator sums (so the loop is not optimised away).  Errors:
 * LLAMA_ERR_INVALID_ARG for blocks or iters <= 0 or a NULL sink. */
llama_status llama_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink_dev, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* llama_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LLAMA_BLOCK_H_ */

/*
 * gqa_attn.h -- grouped-query attention over a bf16 KV cache on AMD MI355X
 * (gfx950).  C ABI of libgqa_attn.so.
 *
 * Pages cited (by title):
 *   [transformer架构]  "Agentic RL入门3：transformer架构" (xiaored5.github.io)
 *   [注意力变体与MoE]  "注意力变体与 MoE" (notes.cassieliang.com)
 *   [attention]        "attention" (my-site-6ix.pages.dev, posts/attention)
 *   [稀疏注意力]        "稀疏注意力：省了什么，没省什么" (geekvape-learning, C11 lesson 5)
 *   [注意力机制进化史]  "注意力机制进化史：从MHA、MQA、GQA、MLA到NSA、MoBA！" (CSDN)
 *
 * Conventions shared by every entry point
 *   - Tensors are plain device pointers to dense, row-major arrays; bf16 is the
 *     IEEE-754 binary16-brain format (1-8-7), stored as 16-bit words.
 *   - MHA, GQA and MQA are one operation: n_kv_head = n_head, n_head / g and 1.
 *     q head h reads kv head floor(h / g) with g = n_head / n_kv_head, the map
 *     the pages' GQA code builds by repeating each K/V head g times along the
 *     head axis ([注意力变体与MoE] "MQA 与 GQA"; [attention] GQA).  No K/V is
 *     ever copied: the g heads of a group read the same bytes.
 *   - Arithmetic: bf16 inputs, fp32 accumulation, bf16 outputs rounded once
 *     (round to nearest even).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on it; results are ready when the stream is synchronized.
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     workspace.  The library allocates no device memory and holds no mutable
 *     global state; calls on different streams with disjoint buffers may run
 *     concurrently.
 *   - Errors: arguments are validated on the host before anything is launched.
 *     On GQA_ERR_INVALID_ARGUMENT, GQA_ERR_UNSUPPORTED or
 *     GQA_ERR_WORKSPACE_TOO_SMALL nothing is launched and nothing is written.
 *     GQA_ERR_DEVICE reports a failed launch (hipGetLastError); faults inside
 *     a kernel surface at the caller's next synchronization.  Values read
 *     from device memory (seq_lens, positions) cannot be checked on the host:
 *     seq_lens outside [1, S_max] is undefined behaviour (loads are still
 *     clamped to the cache so no access leaves the buffers).
 *   - Pointers must be 16-byte aligned; head_dim must be a multiple of 8.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARGUMENT = 1,     /* bad size, null or misaligned pointer, bad RoPE setting */
    GQA_ERR_UNSUPPORTED = 2,          /* valid but not instantiated (head_dim, rotary_dim, ...) */
    GQA_ERR_WORKSPACE_TOO_SMALL = 3,
    GQA_ERR_DEVICE = 4
} gqa_status;

/* RoPE frequency scalings, [transformer架构] §1.1 (plain) and §1.2 ①-③. */
typedef enum {
    GQA_ROPE_NONE = 0,   /* no rotation */
    GQA_ROPE_PLAIN = 1,  /* theta_i = base^(-2i/d), angle m*theta_i                     (§1.1) */
    GQA_ROPE_PI = 2,     /* position interpolation: angle (m/s)*theta_i                    (§1.2 ①) */
    GQA_ROPE_NTK = 3,    /* NTK-aware: base' = base * s^(d/(d-2))                          (§1.2 ②) */
    GQA_ROPE_YARN = 4,   /* NTK-by-parts ramp gamma(r_i), r_i = L_train*theta_i/(2 pi),
                            theta_i' = (1-gamma) theta_i/s + gamma theta_i, and cos/sin
                            multiplied by 0.1 ln s + 1 when yarn_mscale != 0            (§1.2 ③) */
    GQA_ROPE_DYNAMIC_NTK = 5  /* NTK with s = max(1, L_cur / L_train) chosen per call from the
                            current sequence length L_cur (the token being processed
                            included): T in a prefill, seq_lens[b] in a decode step (q and
                            the appended key), current_len in rope_apply.  factor must be 1;
                            L_train = original_max_position.                       (§1.2 ④) */
} gqa_rope_scaling;

/* All fields explicit; the library applies no hidden defaults. */
typedef struct {
    int32_t scaling;               /* gqa_rope_scaling */
    int32_t rotary_dim;            /* even, multiple of 8, <= head_dim and <= 256; 0 means head_dim.
                                      Pairs are adjacent dims (2i, 2i+1) of the first rotary_dim dims;
                                      later dims pass through unchanged. */
    double  base;                  /* > 1, e.g. 1e4, 5e5, 1e6 */
    double  factor;                /* s >= 1 for PI / NTK / YaRN; must be 1 for PLAIN and DYNAMIC_NTK */
    int32_t original_max_position; /* L_train (YaRN and DYNAMIC_NTK), > 0 */
    int32_t yarn_mscale;           /* YaRN only: nonzero folds the temperature into cos/sin */
    double  yarn_alpha;            /* YaRN ramp lower edge (page default 1) */
    double  yarn_beta;             /* YaRN ramp upper edge (page default 32), > alpha */
    int32_t current_len;           /* DYNAMIC_NTK in rope_apply only: L_cur >= 1 (the other
                                      entry points take L_cur from their own lengths) */
} gqa_rope_params;

/*
 * rope_apply -- rotate the adjacent pairs of the first rotary_dim dims of
 * every (token, head) row by its token's position:
 *     (x_2i, x_2i+1) <- (x_2i cos a - x_2i+1 sin a, x_2i sin a + x_2i+1 cos a) * amp,
 *     a = m_eff * theta_i,
 * [transformer架构] §1.1 (the 2x2 rotation R(m, theta_i)) with the scalings of §1.2.
 * Apply it to Q and K only ([transformer架构] §1.1: V carries no position).
 *
 *   in, out      bf16; element (t, h, d) at t*stride_tok + h*stride_head + d
 *                (strides in elements, multiples of 8; the same strides for in
 *                and out).  out may equal in (in place); otherwise dims at or
 *                after rotary_dim are copied.
 *   positions    device int32 [n_tok], >= 0 (the m of each token)
 *   n_tok >= 0 (0 is a no-op), n_heads >= 1, head_dim multiple of 8 in [8, 1024].
 * Angles are formed in fp64 and reduced to [-pi, pi] before an fp32 sin/cos,
 * so positions up to 2^31 keep full fp32 accuracy.
 */
gqa_status rope_apply(const void* in, void* out, const int32_t* positions,
                      int64_t n_tok, int32_t n_heads, int32_t head_dim,
                      int64_t stride_tok, int64_t stride_head,
                      const gqa_rope_params* rope, void* stream);

/*
 * gqa_decode -- one new token per sequence attends to its whole KV cache
 * (the decode step of [注意力变体与MoE] "生成时的瓶颈": the new q against every
 * cached K/V; the new token's own k/v are already appended, as in
 * [注意力机制进化史] "解码中的KV Cache").  For batch b and q head h:
 *     q~   = RoPE(q[b][h], position seq_lens[b]-1)          (q_rope, may be NONE)
 *     s_j  = scale * q~ . K[b][h/g][j],   j < seq_lens[b]
 *     out  = sum_j softmax(s)_j V[b][h/g][j]
 *
 *   q          bf16 [B][Hq][D]
 *   k_cache    bf16 [B][Hkv][S_max][D], keys already rotated (post-RoPE)
 *   v_cache    bf16 [B][Hkv][S_max][D]
 *   seq_lens   device int32 [B], each in [1, S_max]
 *   q_rope     NULL or GQA_ROPE_NONE: q is used as given
 *   out        bf16 [B][Hq][D]
 *   workspace  >= gqa_decode_workspace_size(B, Hq, Hkv, D, S_max) bytes, device,
 *              256-byte aligned; its contents on entry do not matter.
 * Supported: D in {64, 128}; Hq % Hkv == 0; g = Hq/Hkv <= 64.
 * The work is split over the context (split-K) with a log-sum-exp merge;
 * the result does not depend on the split.
 */
size_t gqa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max);

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                      int32_t D, int32_t S_max, float scale,
                      const gqa_rope_params* q_rope, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* As gqa_decode with the number of work ranges chosen by the caller:
 * the rows of all B*Hkv contexts, taken in (batch, kv head, row) order, are
 * cut into n_parts equal ranges (n_parts in [1, 2^20]; 0 = the library's
 * default); each group of four consecutive ranges is streamed by the four
 * wavefronts of one workgroup, which take its 32-row tiles in turn.  The
 * workspace must then hold gqa_decode_workspace_size_parts(...) bytes (it
 * grows with n_parts). */
size_t gqa_decode_workspace_size_parts(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t S_max, int32_t n_parts);

gqa_status gqa_decode_parts(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t S_max, float scale,
                            const gqa_rope_params* q_rope, void* out,
                            void* workspace, size_t workspace_bytes,
                            int32_t n_parts, void* stream);

/*
 * gqa_decode_noalloc -- gqa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument, the per-piece softmax states go
 * to a static scratch array of 16 MiB (16777216 bytes) that each device
 * holds for the life of the process.  The call allocates nothing; its first
 * call on a device looks up that device's copy of the array.
 *   Limit: gqa_decode_workspace_size(B, Hq, Hkv, D, S_max) <= 16777216, else
 *   GQA_ERR_WORKSPACE_TOO_SMALL and nothing is launched (the 32K and 4K
 *   workloads of 16 sequences x 64 q heads need about 4.8 MB).
 *   Sharing: every call on one device uses the same scratch, so calls that
 *   overlap in time on one device (different streams, or host threads) race
 *   and give wrong results; serialise them (one stream, or events).  Nothing
 *   in the scratch needs to start at any value.
 * Arguments, outputs, results (bit for bit those of gqa_decode) and other
 * errors as gqa_decode.
 */
gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t S_max, float scale,
                              const gqa_rope_params* q_rope, void* out, void* stream);

/*
 * Two-phase decode: gqa_decode_parts == gqa_decode_partial then
 * gqa_decode_combine with the same arguments.  The partial phase leaves in
 * the workspace one softmax state per piece (a run of rows of one context
 * inside one work range):
 *     m = max_j t_j,  l = sum_j 2^(t_j - m),  o[d] = sum_j 2^(t_j - m) V[j][d],
 *     t_j = scale * log2(e) * (q~ . K[j])        (base-2 logits)
 * and the combine phase returns, per (batch, q head),
 *     sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
 * which equals the one-pass softmax exactly in real arithmetic.  The state
 * layout is internal to the pair; callers merging states of disjoint row
 * ranges themselves (e.g. a context split across devices) apply the same
 * formula to their own (m, l, o).
 */
gqa_status gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t S_max, float scale,
                              const gqa_rope_params* q_rope,
                              void* workspace, size_t workspace_bytes,
                              int32_t n_parts, void* stream);

gqa_status gqa_decode_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t S_max,
                              const void* workspace, size_t workspace_bytes,
                              int32_t n_parts, void* out, void* stream);

/*
 * gqa_decode_append -- a whole decode step: the new token's key and value
 * are written into the caches, then the token attends as in gqa_decode
 * ([注意力机制进化史] "解码中的KV Cache": the new k/v are concatenated to the
 * past ones before attending; [transformer架构] §1.1: the key is rotated at
 * its own position, the value is not).  For batch b and kv head j, with
 * L = seq_lens[b] (which counts the new token):
 *     k_cache[b][j][L-1] = bf16(RoPE(k_new[b][j], position L-1))  (q_rope's
 *                          settings, YaRN amplitude included; as given when
 *                          q_rope is NULL or NONE)
 *     v_cache[b][j][L-1] = v_new[b][j]
 * and out = gqa_decode(q, k_cache, v_cache, seq_lens, ...) over the updated
 * caches.  The write is fused into the decode kernel: the wave that streams
 * row L-1 takes it from k_new/v_new and stores it, so the step reads the
 * caches once and launches the same two kernels as gqa_decode.
 *
 *   k_new, v_new  bf16 [B][Hkv][D], device, 16-byte aligned; k_new not rotated
 *   k_cache, v_cache  as in gqa_decode, written at row seq_lens[b]-1 only
 * Other arguments, limits and errors as gqa_decode.  Nothing is written when
 * an error status is returned.
 */
gqa_status gqa_decode_append(const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max,
                             float scale, const gqa_rope_params* q_rope, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_decode_window -- gqa_decode (optionally with gqa_decode_append's cache
 * write) over a sliding window or a rolling-buffer cache.
 * Sliding window ([transformer架构] §2.5.1): the query at position i sees
 * keys i-w+1 .. i.  With a linear cache (rolling = 0, row = position,
 * seq_lens[b] in [1, S_max]) the new token (position L-1, L = seq_lens[b])
 * attends to rows max(0, L-window) .. L-1; window 0 means no window.
 * Rolling buffer ([transformer架构] §2.5.2, rolling = 1): position t lives in
 * slot t mod S_max, so the cache holds the last S_max positions; L may exceed
 * S_max.  With window 0 the new token attends to every filled slot,
 * min(L, S_max) of them; with 0 < window <= S_max to the slots of positions
 * max(0, L-window) .. L-1, which wrap around the buffer's end when
 * (L-window) mod S_max > (L-1) mod S_max.  q is rotated at its absolute
 * position L-1 in both caches; keys are cached after RoPE, so nothing is
 * re-rotated.
 *
 *   k_new, v_new  NULL (no cache write) or, both, as in gqa_decode_append: the
 *                 new row goes to row L-1 (linear) or slot (L-1) mod S_max
 *                 (rolling) before the attention reads it
 *   window        >= 0; at most S_max when rolling = 1 (window 0: the buffer)
 *   rolling       0 or 1
 * Other arguments, limits and errors as gqa_decode / gqa_decode_append.
 */
gqa_status gqa_decode_window(const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max,
                             int32_t window, int32_t rolling, float scale,
                             const gqa_rope_params* q_rope, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_decode_sink_window -- gqa_decode_window with StreamingLLM sink tokens
 * ([attention] "Slide Window Attention (SWA)", 修复方案 1. StreamingLLM: the
 * effective context is the first s tokens followed by the sliding window;
 * [transformer架构] §2.5.4: the band mask with the first k columns kept).
 * Linear cache (rolling = 0): the new token at position L-1 attends to rows
 * 0 .. min(sinks, lo)-1 and lo .. L-1, lo = max(0, L-window); window 0 means
 * no window (every row; sinks are then moot).  Rolling buffer (rolling = 1,
 * 0 <= sinks < S_max): slots 0 .. sinks-1 keep positions 0 .. sinks-1 for
 * good and position t >= sinks lives in slot sinks + (t - sinks) mod
 * (S_max - sinks) (the ring); with window 0 the new token attends to every
 * filled slot (min(L, S_max) of them), with 0 < window <= S_max - sinks to
 * the sinks and the slots of positions max(0, L-window) .. L-1 (each once);
 * the fused write (k_new, v_new) goes to its position's slot.  sinks = 0 is
 * exactly gqa_decode_window.
 *   sinks  >= 0 (< S_max when rolling = 1)
 *   window >= 0 (<= S_max - sinks when rolling = 1)
 * Other arguments, limits and errors as gqa_decode_window.
 */
gqa_status gqa_decode_sink_window(const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const int32_t* seq_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max,
                                  int32_t sinks, int32_t window, int32_t rolling, float scale,
                                  const gqa_rope_params* q_rope, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_causal -- causal GQA attention over a whole prompt
 * ([注意力变体与MoE] "MQA 与 GQA", attention(): scores q k^T / sqrt(hd) with the
 * strict upper triangle masked to -inf, softmax, weighted sum of V):
 *     q~_i = RoPE(q_i, i), k~_j = RoPE(k_j, j),  positions 0..T-1
 *     out_i = sum_{j<=i} softmax_j(scale * q~_i . k~_j) v_j
 *
 *   q    bf16 [B][Hq][T][D]        (pre-RoPE)
 *   k    bf16 [B][Hkv][T][D]       (pre-RoPE)
 *   v    bf16 [B][Hkv][T][D]
 *   rope NULL or GQA_ROPE_NONE: no rotation
 *   out  bf16 [B][Hq][T][D]
 *   workspace >= gqa_prefill_workspace_size(B, Hkv, T, D, rope) bytes, device,
 *             256-byte aligned (it receives the rotated K as hi and lo bf16
 *             rows and an fp16 copy of V, tiled for the matrix cores);
 *             contents on entry do not matter.
 * Supported: D in {8, 16, 32, 64, 128}; T >= 1; Hq % Hkv == 0; B*Hq <= 65535;
 * T * D * 2 < 2^31.
 * Precision: the rotated Q (times scale*log2 e) and the rotated K enter the
 * matrix cores as hi + lo bf16 terms and each score is the sum of the three
 * products hi.hi + hi.lo + lo.hi (about 2^-17 relative, so a sharp softmax
 * keeps the output within 2e-3 + 1e-2 |ref|); the probabilities and V enter
 * the PV product as fp16 with fp32 accumulation, so |v| must stay below
 * 65504 and V values below 2^-14 in magnitude lose bits as fp16 subnormals
 * (an absolute error under 2^-25 each).  gqa_prefill_fp16 trades the score
 * precision for speed.
 */
size_t gqa_prefill_workspace_size(int32_t B, int32_t Hkv, int32_t T, int32_t D,
                                  const gqa_rope_params* rope);

gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v,
                              int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                              float scale, const gqa_rope_params* rope, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_window -- gqa_prefill_causal with a sliding window
 * ([transformer架构] §2.5.1, the band mask): row i attends to keys
 * max(0, i-window+1) .. i, so
 *     out_i = sum_{i-window < j <= i} softmax_j(scale * q~_i . k~_j) v_j
 * window >= 0; 0 (or any window >= T) is gqa_prefill_causal.  Key tiles wholly
 * below a query tile's window are not read.  Arguments, workspace, limits
 * and errors as gqa_prefill_causal.
 */
gqa_status gqa_prefill_window(const void* q, const void* k, const void* v,
                              int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t window, float scale, const gqa_rope_params* rope,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_sink_window -- gqa_prefill_window with StreamingLLM sink tokens
 * ([attention] "Slide Window Attention (SWA)", 修复方案 1; [transformer架构]
 * §2.5.4: the band plus the first k columns): row i attends to keys
 * 0 .. min(sinks, lo)-1 and lo .. i, lo = max(0, i-window+1), so
 *     out_i = sum_{j <= i, j < sinks or j > i-window} softmax_j(scale * q~_i . k~_j) v_j
 * sinks >= 0, window >= 0; sinks = 0 is gqa_prefill_window, and window 0 (or
 * >= T) is gqa_prefill_causal whatever sinks is.  Key tiles holding neither
 * sinks nor band keys are not read.  Arguments, workspace, limits, precision
 * and errors as gqa_prefill_causal.
 */
gqa_status gqa_prefill_sink_window(const void* q, const void* k, const void* v,
                                   int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t sinks, int32_t window, float scale,
                                   const gqa_rope_params* rope, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_fp16 -- gqa_prefill_sink_window with one-term fp16 scores: the
 * rotated, scaled Q and the rotated K are rounded to fp16 (11-bit
 * significand) and each score is one product, about half the matrix-core
 * work of the default.  Each base-2 logit then carries an error of up to
 * about 2^-10 * scale * log2(e) * |q~| |k~| (|.| the Euclidean norm of the
 * rotated vectors): within 2e-3 + 1e-2 |ref| while the scores spread over
 * about one unit (q, k ~ N(0,1) with scale 1/sqrt(d)), not for a sharp
 * softmax.  |v|, |k| and the rotated, scaled |q| must stay below 65504.
 * Arguments, workspace, masks and errors as gqa_prefill_sink_window.
 */
gqa_status gqa_prefill_fp16(const void* q, const void* k, const void* v,
                            int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t sinks, int32_t window, float scale,
                            const gqa_rope_params* rope, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * topk_sparse_decode -- DSA-style sparse decode over an MLA latent cache,
 * o = Attn(q, KV[TopK(ReLU(K_I . q_I))]) ([稀疏注意力] "改进一：DSA", the
 * selection chain; [transformer架构] §2.2 (1)-(2)):
 *   1. indexer: score_j = ReLU(q_index[b] . k_index[b][j]) for j < seq_lens[b];
 *      the dot product is accumulated exactly (fp64) and rounded once to fp32.
 *   2. top-k: the min(top_k, seq_lens[b]) largest scores; equal scores go to
 *      the lower index; indices written ascending, the rest of the row -1.
 *   3. attention of each of the H heads over the selected latent rows only
 *      (the -inf token mask of [attention] DSA ③), every head reading the same
 *      single latent row (the MQA form of absorbed MLA, [attention] DSA ② and
 *      "乘法结合律" 的变换):
 *        s_j = scale * q[b][h] . latent[b][j][0:Dqk],  out = sum_j p_j latent[b][j][0:Dv]
 *
 *   q           bf16 [B][H][Dqk]   (absorbed query; its RoPE part already rotated)
 *   latent      bf16 [B][S_max][Dqk]; V is the first Dv columns of each row
 *   q_index     bf16 [B][D_idx]
 *   k_index     bf16 [B][S_max][D_idx]
 *   seq_lens    device int32 [B], each in [1, S_max]
 *   topk_idx    int32 [B][top_k]  (output)
 *   out         bf16 [B][H][Dv]   (output)
 *   workspace   >= topk_sparse_decode_workspace_size(B, H, S_max, top_k) bytes
 * Supported: Dqk = 576, Dv = 512, D_idx = 128, H a multiple of 16 up to 128,
 * 1 <= top_k <= min(S_max, 4096).
 */
size_t topk_sparse_decode_workspace_size(int32_t B, int32_t H, int32_t S_max, int32_t top_k);

gqa_status topk_sparse_decode(const void* q, const void* latent, const void* q_index,
                              const void* k_index, const int32_t* seq_lens,
                              int32_t B, int32_t H, int32_t Dqk, int32_t Dv, int32_t D_idx,
                              int32_t S_max, int32_t top_k, float scale,
                              int32_t* topk_idx, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * topk_sparse_decode_weighted -- topk_sparse_decode with the multi-head
 * weighted indexer ([稀疏注意力] DSA ①, the Lightning Indexer formula):
 *     I_s = sum_{j < H_I} w_j * ReLU(q_index[j] . k_index[s])
 * H_I query heads share the single key row; w_j is a per-head weight of
 * either sign.  The selection is the exact top_k of I_s (ties to the lower
 * index; indices ascending, -1 padded), as if I_s were computed exactly: the
 * indexer runs on the matrix cores with fp32 sums, and every key whose fp32
 * score lies within a proven bound of the k-th one (2^-14 * sum_j |w_j|
 * |q_index[j]| * max_s |k_index[s]|) is scored again in fp64 before the
 * final choice.  A run of more than 256 keys within that bound (near-equal
 * scores) keeps the fp32 order among them.  Step 3 and the outputs are
 * those of topk_sparse_decode.
 *
 *   q_index     bf16 [B][H_I][D_idx]
 *   w_index     fp32 [B][H_I] (device, 4-byte aligned)
 *   H_I         16, 32, 48 or 64 (others: GQA_ERR_UNSUPPORTED; < 1: invalid)
 *   other arguments, workspace (topk_sparse_decode_workspace_size), limits
 *   and errors as topk_sparse_decode.
 */
gqa_status topk_sparse_decode_weighted(const void* q, const void* latent, const void* q_index,
                                       const float* w_index, const void* k_index,
                                       const int32_t* seq_lens, int32_t B, int32_t H, int32_t H_I,
                                       int32_t Dqk, int32_t Dv, int32_t D_idx, int32_t S_max,
                                       int32_t top_k, float scale, int32_t* topk_idx, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_sparse_decode -- QSA decode ([attention] Qwen Sparse Attention ①-④):
 *   1. the first 4 * floor(L/4) indexer keys form 4-token micro-blocks; a
 *      block's key is the mean of its keys, normalised to unit length,
 *      rotated by block_rope at the block's first position 4 j;
 *   2. block score = sum over the H_I indexer heads of ReLU(q_index[h] . key);
 *   3. the 512 best blocks (ties to the lower block; all if there are fewer)
 *      are expanded to their 4 tokens and the L mod 4 tail tokens are added:
 *      token_idx[b] holds at most 2051 ascending positions, -1 after;
 *   4. standard GQA attention of every query head over those tokens of its
 *      kv head's cache:  out = softmax(scale * q . K[t]) V[t].
 * The block set is the exact top 512 of these scores (as if computed in
 * exact arithmetic): the blocks are scored on the matrix cores (block keys
 * in fp32, entering as hi + lo bf16 terms, fp32 sums), and every block whose
 * fp32 score lies within a proven bound of the 512th (about
 * 2^-13 * sum_h |q_index[h]|) is scored again in fp64, its block key rebuilt
 * in fp64, before the final choice.  A run of more than 256 blocks within
 * that bound keeps the fp32 order among them.
 *
 *   q          bf16 [B][Hq][D], already rotated at its position (post-RoPE cache)
 *   k_cache    bf16 [B][Hkv][S_max][D], v_cache the same
 *   q_index    bf16 [B][H_I][D_idx], already rotated at the query position
 *   k_index    bf16 [B][S_max][D_idx], indexer keys before RoPE
 *   seq_lens   device int32 [B], each in [1, S_max]
 *   block_rope NULL / NONE: no rotation; otherwise applied to the first
 *              rotary_dim dims of the block keys (Dynamic NTK: unsupported)
 *   token_idx  int32 [B][2051] (output), out bf16 [B][Hq][D] (output)
 *   workspace  >= qsa_sparse_decode_workspace_size(B, Hq, S_max) bytes, 256-byte aligned
 * Supported: D = 128, D_idx = 128, Hq/Hkv <= 16, H_I in {16, 32, 48, 64},
 * S_max * D * 2 < 2^31.  Errors as topk_sparse_decode.
 */
size_t qsa_sparse_decode_workspace_size(int32_t B, int32_t Hq, int32_t S_max);

gqa_status qsa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                             const void* q_index, const void* k_index, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t H_I,
                             int32_t D_idx, int32_t S_max, float scale,
                             const gqa_rope_params* block_rope, int32_t* token_idx, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode -- dense decode over an MLA latent cache in the absorbed form
 * ([attention] DSA ② and "乘法结合律" 的变换; [注意力变体与MoE] "MLA"): with
 * W_UK folded into the query and W_UV applied after the sum, every head
 * attends to the same single latent row, i.e. MQA with Dqk-dim keys and the
 * first Dv columns as values, over all rows j < seq_lens[b]:
 *     s_j = scale * q[b][h] . latent[b][j][0:Dqk],
 *     out[b][h] = sum_j softmax_j(s) latent[b][j][0:Dv]
 * This is topk_sparse_decode with every row selected.
 *
 *   q           bf16 [B][H][Dqk]   (absorbed query; its RoPE part already rotated)
 *   latent      bf16 [B][S_max][Dqk]; V is the first Dv columns of each row
 *   seq_lens    device int32 [B], each in [1, S_max] (clamped into that range)
 *   out         bf16 [B][H][Dv]   (output)
 *   workspace   >= mla_decode_workspace_size(B, H, S_max) bytes, 256-byte aligned;
 *               fp32 partial softmax states of the row ranges, owned by the caller
 * Supported: Dqk = 576, Dv = 512, H a multiple of 16 up to 128,
 * S_max * Dqk * 2 < 2^31.  Other Dqk/Dv or H: GQA_ERR_UNSUPPORTED; null or
 * misaligned pointers, non-finite scale: GQA_ERR_INVALID_ARGUMENT; short
 * workspace: GQA_ERR_WORKSPACE_TOO_SMALL.  Asynchronous on `stream`.
 */
size_t mla_decode_workspace_size(int32_t B, int32_t H, int32_t S_max);

gqa_status mla_decode(const void* q, const void* latent, const int32_t* seq_lens,
                      int32_t B, int32_t H, int32_t Dqk, int32_t Dv, int32_t S_max,
                      float scale, void* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * KV-cache bytes per token, exact integers ([注意力变体与MoE] "生成时的瓶颈":
 * 2 (K and V) x layers x n_kv_head x d_head x bytes; and "MLA": layers x
 * (d_latent + d_rope) x bytes, no factor 2 because K and V share the latent).
 * Return -1 for a negative argument or on int64 overflow.
 */
int64_t kv_bytes_per_token(int32_t layers, int32_t n_kv_heads, int32_t head_dim,
                           int32_t bytes_per_elem);
int64_t mla_kv_bytes_per_token(int32_t layers, int32_t d_latent, int32_t d_rope,
                               int32_t bytes_per_elem);

/* Static description of a status code (never NULL). */
const char* gqa_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */

/* orthrus.h -- C ABI of the Orthrus dual-view decode step on MI355X (gfx950).
 *
 * The method ("Orthrus: Memory-Efficient Parallel Token Generation via
 * Dual-View Diffusion"): a frozen autoregressive (AR) Transformer and a
 * trainable diffusion-attention path in every layer share ONE KV cache.  The
 * AR view pre-fills the cache (opentrain.ai page, abstract); the diffusion
 * view projects a block of K mask positions in one forward pass over that
 * cache (HN item page, "Idea"; atlas.scime.ai page, "Approach"); the AR view
 * verifies the block in a second pass, the longest prefix matching its greedy
 * argmax is accepted together with the AR bonus token, and only accepted
 * entries are committed to the cache (openai-hub.net page, "KV Cache
 * Overhead" and "Open-Source Code" steps).  The emitted sequence equals
 * plain greedy AR decoding of the frozen model.
 *
 * One step, for each sequence b with committed length n = seq_len[b] and
 * pending token x (the last emitted token, whose K/V is not yet cached):
 *   orthrus_draft_block    pass 1: the anchor row (x at position n, frozen
 *                          view, causal over slots [0, n], its K/V staged at
 *                          slot n) gives a_0; K mask rows (positions
 *                          n+1..n+K, diffusion view, attending to slots
 *                          [0, n] and bidirectionally to the whole block)
 *                          give the drafts d_1..d_K.  Block K/V live only in
 *                          the block scratch; nothing of the block reaches the
 *                          cache.
 *   orthrus_verify_accept  pass 2: the frozen view over d_1..d_K at
 *                          n+1..n+K, causal (row i sees slots [0, n+i]), K/V
 *                          staged at n+1..n+K, gives a_1..a_K; then
 *                          m = max{j <= K : d_i == a_{i-1} for all i <= j}.
 *   orthrus_commit_kv      commits slots n..n+m (seq_len <- n+1+m), emits
 *                          d_1..d_m and the bonus a_m, pending <- a_m.  Staged
 *                          slots past n+m are discarded (overwritten later).
 * block_k == 0 is plain greedy decoding with the same kernels: pass 1 is the
 * anchor row alone, verify_accept only sets accept_len = 0, and commit emits
 * a_0.
 *
 * Conventions
 *  - Return codes: ORTHRUS_OK (0) or a negative ORTHRUS_E* code; the string
 *    is orthrus_strerror(code).  All argument, capacity and call-order checks
 *    run on the host BEFORE anything is enqueued, so an error leaves device
 *    state untouched.  ORTHRUS_EHIP reports a failed HIP launch/copy
 *    (orthrus_last_hip_error() gives the hipError_t value).
 *  - Pointers: unless marked "host", every pointer argument is device memory
 *    owned by the caller.  The library never allocates or frees device
 *    memory; the sizes of the buffers it needs come from
 *    orthrus_query_sizes().  "stream" is a hipStream_t (NULL = default
 *    stream).  Every call only enqueues work on that stream (create also
 *    does a small host->device copy on it).
 *  - Token ids are int32.  Ids outside [0, vocab) are clamped when embedded.
 *  - One context is driven by one stream at a time; calls on a context must
 *    be serialized by the caller.
 *  - Call order per step: draft_block -> verify_accept -> commit_kv
 *    (ORTHRUS_ESTATE otherwise).  The host keeps an upper bound on every
 *    sequence's length (max_prompt_len, plus k + 1 per committed step) and
 *    refuses a step that could write past max_ctx (ORTHRUS_ECAPACITY).
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORTHRUS_OK = 0,
  ORTHRUS_EINVAL = -1,     /* bad shape, pointer, batch or token count */
  ORTHRUS_ECAPACITY = -2,  /* a sequence could grow past max_ctx */
  ORTHRUS_ESTATE = -3,     /* call out of order (e.g. verify without draft) */
  ORTHRUS_EHIP = -4        /* a HIP call failed */
};

enum { ORTHRUS_F32 = 0, ORTHRUS_BF16 = 1 };

/* Model and capacity.  The layer is Qwen3-style: RMSNorm (eps rms_eps), Q/K/V
 * projections, per-head QK RMSNorm, rotate-half RoPE (base rope_theta),
 * grouped-query attention (query head h reads KV head h / (n_q_heads /
 * n_kv_heads)), O projection + residual, RMSNorm, SwiGLU FFN + residual;
 * final RMSNorm and an untied LM head.  The diffusion path has its own
 * Q/K/V/O projections and QK-norm gains; norms, FFN, embedding and LM head
 * are shared.
 * BF16 models: bf16 weights, bf16 KV cache, fp32 residual stream, fp32
 * accumulation; requires head_dim 128, d_model, n_q_heads*head_dim and
 * ffn_dim multiples of 256, d_model <= 8192 and vocab a multiple of 128.
 * block_k is at most 63 for both dtypes (the draft block is one 64-key
 * attention tile, and acceptance is one 64-lane ballot).
 * F32 models: everything fp32 (small check models). */
typedef struct orthrus_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t block_k;        /* K, mask positions per block (0 = plain AR) */
  double rope_theta;
  double rms_eps;
  int32_t dtype;          /* ORTHRUS_F32 or ORTHRUS_BF16 */
  int32_t max_batch;      /* sequences per call, 1..256 */
  int32_t max_ctx;        /* KV slots per sequence (cache capacity) */
  int32_t attn_chunk;     /* keys per attention chunk: 0 = orthrus_default_attn_chunk(
                             max_batch, max_ctx, n_kv_heads), else a power of two in
                             [64, 4096].
                             Attention partials are folded per chunk of absolute cache
                             positions, so two contexts give bit-identical rows (e.g. a
                             block_k = 32 context and its block_k = 0 greedy twin, or a batch
                             and one of its sequences alone) only if their attn_chunk values
                             are equal. */
} orthrus_config;

typedef struct orthrus_sizes {
  uint64_t weights_bytes;    /* canonical weight buffer (see orthrus_weight_tensor) */
  uint64_t packed_bytes;     /* library-layout copy of the weights */
  uint64_t kv_bytes;         /* the shared KV cache */
  uint64_t scratch_bytes;    /* block K/V scratch: 2*L*max_batch*Hkv*K*head_dim*elt */
  uint64_t workspace_bytes;  /* activations, partial results, RoPE table */
  uint64_t kv_slots;         /* cache slots per (sequence, KV head), "cap": max_ctx
                                rounded up to a multiple of 64 */
  uint64_t prefill_rows;     /* prompt rows per sequence in one orthrus_prefill pass:
                                2048 / max_batch rounded down to a multiple of 32,
                                clamped to [32, 256] */
} orthrus_sizes;

typedef struct orthrus_ctx orthrus_ctx;

/* Buffer sizes for a config.  Host only; needs no GPU. */
int orthrus_query_sizes(const orthrus_config* cfg, orthrus_sizes* out);

/* Canonical weight buffer format: tensors concatenated in index order, each
 * starting at a multiple of 256 elements, elements fp32 or bf16 (per dtype),
 * matrices row-major [out][in].  Index 0 embedding [V][d], 1 LM head [V][d],
 * 2 final-norm gain [d], 3 mask embedding [d] (the diffusion view's input at
 * every mask position), then per layer l, at 4 + 17*l + j:
 *   j=0 attention-norm gain [d], 1 FFN-norm gain [d], 2 Wq [Hq*hd][d],
 *   3 Wk [Hkv*hd][d], 4 Wv [Hkv*hd][d], 5 Wo [d][Hq*hd], 6 q-norm gain [hd],
 *   7 k-norm gain [hd], 8..13 the diffusion path's Wq, Wk, Wv, Wo, q-norm and
 *   k-norm gains (same shapes), 14 W_gate [F][d], 15 W_up [F][d],
 *   16 W_down [d][F].
 * index == -1 returns the total element count.  Host only. */
int orthrus_weight_tensor(const orthrus_config* cfg, int32_t index, uint64_t* offset_elems,
                          uint64_t* numel);

/* Validate cfg, bind the caller's buffers and pack the canonical weights
 * (device, read only during this call; may be freed afterwards) into
 * `packed`.  Builds the RoPE table (float64 angles on the host, stored
 * fp32) into the workspace.  Errors: EINVAL (shape, null or misaligned
 * pointer: every buffer must be 256-byte aligned), EHIP. */
int orthrus_create(const orthrus_config* cfg, const void* weights, void* packed, void* kv_cache,
                   void* block_scratch, void* workspace, void* stream, orthrus_ctx** out);

/* Release the context (host memory only; the caller frees its buffers). */
int orthrus_destroy(orthrus_ctx* ctx);

/* AR-view prefill of `batch` prompts (the frozen view builds the cache:
 * opentrain.ai page, abstract).  tokens: device [batch][tokens_stride]
 * int32; prompt_len: device [batch], each in [1, max_prompt_len] (values
 * outside are clamped); max_prompt_len: host, in [1, tokens_stride], the
 * longest prompt.  Writes the cache slots [0, prompt_len), sets seq_len[b] =
 * prompt_len[b] and pending[b] = argmax of the last prompt row (the first
 * generated token).  The prompts run through the frozen view in passes of
 * up to 2048 / max_batch rows per sequence (32 to 256), causal within and
 * across passes, every sequence to max_prompt_len - 1 (rows past a shorter
 * prompt land in slots that no later step reads).  Only enqueues work; the
 * host's length bound of every sequence becomes max_prompt_len.  Resets the
 * call-order state.  Errors: EINVAL, ECAPACITY. */
int orthrus_prefill(orthrus_ctx* ctx, int32_t batch, const int32_t* tokens, int32_t tokens_stride,
                    const int32_t* prompt_len, int32_t max_prompt_len, int32_t* seq_len,
                    int32_t* pending, void* stream);

/* Pass 1 (see the top of this file).  seq_len, pending: [batch] (read);
 * drafts: [batch][K] (written); ar_tokens: [batch][K+1], only column 0
 * (a_0) is written.  Stages the anchor K/V at slot seq_len[b]; writes the
 * block scratch; the committed cache [0, seq_len) is not modified.
 * Errors: EINVAL, ECAPACITY, ESTATE (a draft is already outstanding). */
int orthrus_draft_block(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                        const int32_t* pending, int32_t* drafts, int32_t* ar_tokens, void* stream);

/* Pass 1 with a block of k <= block_k mask positions for this step only
 * (dynamic K: the openai-hub.net article, "Future Directions", item 1, block
 * size adjusted per step to the generation's certainty; the choice itself is
 * the caller's).  drafts and ar_tokens keep their [batch][block_k] and
 * [batch][block_k + 1] layouts; only the first k (drafts) and k + 1
 * (ar_tokens, after verify) columns are written.  The verify_accept and
 * commit_kv calls of the step follow this k: accept_len is in [0, k], the
 * host bound grows by k + 1.  k = 0 is one step of plain greedy decoding.
 * orthrus_draft_block is this call with k = block_k.  Errors: EINVAL (k out
 * of range), ECAPACITY, ESTATE. */
int orthrus_draft_block_k(orthrus_ctx* ctx, int32_t batch, int32_t k, const int32_t* seq_len,
                          const int32_t* pending, int32_t* drafts, int32_t* ar_tokens,
                          void* stream);

/* One more denoising pass over the outstanding block (the 2-step iterative
 * denoising variant the pages compare against single-step block
 * projection: atlas.scime.ai page, "Surprising findings"; HN item page,
 * "Results").  Taken as: the diffusion view runs again over the same k mask
 * positions n+1..n+k, each row now starting from the embedding of its
 * current draft instead of the mask embedding, with the same attention
 * (cache slots [0, n], the staged anchor included, and the whole block,
 * bidirectionally; the block K/V are rewritten in the block scratch); its
 * argmax replaces drafts[b][0..k).  The anchor row and a_0 are not
 * recomputed; nothing is written to the cache.  May be called more than
 * once between draft_block and verify_accept.  drafts: [batch][block_k]
 * (read, then written).  Errors: EINVAL, ESTATE (no outstanding draft). */
int orthrus_draft_refine(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                         int32_t* drafts, void* stream);

/* Pass 2 and acceptance.  drafts: [batch][K] (read; the caller may have
 * replaced the drafted ids since draft_block); ar_tokens: [batch][K+1]
 * (column 0 read, columns 1..K written); accept_len: [batch] (written, in
 * [0, K]).  Stages K/V at slots seq_len+1 .. seq_len+K; commits nothing.
 * Errors: EINVAL, ESTATE (no outstanding draft). */
int orthrus_verify_accept(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len,
                          const int32_t* drafts, int32_t* ar_tokens, int32_t* accept_len,
                          void* stream);

/* Commit.  accept_len [batch], ar_tokens [batch][K+1], drafts [batch][K]
 * (read); seq_len [batch] (read, then set to seq_len + 1 + m); pending
 * [batch] (set to a_m); commit_start [batch] (set to the old seq_len: the
 * committed slots are [commit_start, commit_start + m]); out_tokens
 * [batch*(K+1)] (the emitted tokens d_1..d_m, a_m of every sequence, packed
 * in batch order); out_off [batch+1] (exclusive prefix sum of m+1; out_off
 * [batch] = tokens emitted by the step).  Moves no KV bytes: the accepted
 * entries are already in place.  Errors: EINVAL, ESTATE (no verified
 * step). */
int orthrus_commit_kv(orthrus_ctx* ctx, int32_t batch, const int32_t* accept_len,
                      const int32_t* ar_tokens, const int32_t* drafts, int32_t* seq_len,
                      int32_t* pending, int32_t* commit_start, int32_t* out_tokens,
                      int32_t* out_off, void* stream);

/* Tighten the host's length bound of each sequence to seq_len_host[b]
 * (HOST array, values the caller read back from seq_len after a commit).
 * The bound otherwise grows by block_k + 1 per committed step, which is
 * what a caller that never reads lengths back must provision in max_ctx.
 * Values below 1 or above the current bound are rejected (EINVAL); the
 * device side never reads or writes past max_ctx whatever the bound says.
 * Host only; must not be called while a step is in flight (ESTATE). */
int orthrus_sync_lengths(orthrus_ctx* ctx, int32_t batch, const int32_t* seq_len_host);

/* For steps that run without these calls: replays of a HIP graph that
 * captured one draft_block(_k) -> verify_accept -> commit_kv step (every
 * call only enqueues kernels and device-to-device work on its stream, so
 * the three calls can be captured; greedy decoding only, since the
 * sampling step counter is host state).  Raises the host's length bound of
 * sequences 0..batch-1 by n_steps * (k + 1), as n_steps eager steps of
 * block k would; call it before replaying n_steps times.  Errors: EINVAL,
 * ESTATE (a step in flight, or never prefilled), ECAPACITY (a sequence
 * could grow past max_ctx: nothing is reserved). */
int orthrus_reserve_steps(orthrus_ctx* ctx, int32_t batch, int32_t k, int32_t n_steps);

/* Launch timing for profiling.  When enabled, the library records a pair
 * of hipEvents (host-created; no device memory) around every launch of the
 * selected classes on the call's stream.  Class = pass*8 + role with pass
 * 0 draft, 1 verify, 2 prefill and role 0 QKV GEMM, 1 attention (+ merge),
 * 2 O GEMM, 3 gate/up SwiGLU GEMM, 4 down GEMM, 5 LM head + argmax, 6 the
 * small kernels (embed, RMSNorm, QK-norm/RoPE/KV write), 7 accept and
 * commit (pass 1 only).  The gate/up GEMM is one kernel; its pair is
 * recorded by the kernel's dispatch (hipExtLaunchKernel), so it spans the
 * kernel alone; the other classes' pairs are recorded around their launches.
 * class_mask bit k selects class k; capacity = event pairs kept (launches
 * past it are not timed).  class_mask 0 turns timing
 * off.  orthrus_timing_read synchronizes on the recorded events, adds each
 * pair's elapsed time to ms[class] (milliseconds) and counts launches[class]
 * (both arrays ORTHRUS_TIMING_CLASSES long), then starts a new record;
 * ECAPACITY if launches were dropped.  Errors: EINVAL, EHIP. */
#define ORTHRUS_TIMING_CLASSES 24
int orthrus_timing_enable(orthrus_ctx* ctx, uint32_t class_mask, int32_t capacity);
int orthrus_timing_read(orthrus_ctx* ctx, double* ms, int64_t* launches);

/* Parity taps (optional; NULL disables).  logits: device fp32
 * [rows_cap][vocab]; every later LM-head pass writes its rows' logits there,
 * by pass row: pass 1 has the batch*K mask rows in sequence order (row
 * b*K + i), then padding up to RA = batch*K rounded up to a multiple of 16,
 * then the anchor rows (row RA + b); pass 2 has batch*K rows (b*K + i).
 * Padding rows are unspecified.  attn: device
 * [n_layers][rows_cap][n_q_heads*head_dim] in the model dtype; every later
 * pass writes each layer's attention output (the O projection's input).
 * A pass with more rows than rows_cap writes neither tap (both keep what an
 * earlier pass wrote).  Errors: EINVAL. */
int orthrus_set_debug(orthrus_ctx* ctx, float* logits, void* attn, int32_t rows_cap);

/* Sampling at temperature T > 0 with lossless rejection sampling (the
 * pages: greedy and rejection sampling only, the latter briefly described;
 * HN item page and atlas.scime.ai page, "Limitations").  temperature 0
 * (the default) is greedy decoding.  With T > 0, for every later step:
 *   draft_block   draws each mask row's draft d_i from q_i = softmax(z_i / T)
 *                 of the diffusion view (orthrus_draft_refine redraws from
 *                 the refined rows);
 *   verify_accept takes p_0 = softmax(z / T) of the anchor row and p_i of
 *                 verify row i; accepts d_i with probability
 *                 min(1, p_{i-1}(d_i) / q_i(d_i)) in order until the first
 *                 rejection (accept_len = m); the step's final token is a
 *                 sample of max(0, p_m - q_{m+1}) renormalised after a
 *                 rejection, of p_k after k acceptances; ar_tokens[b][0..m)
 *                 = the accepted drafts, ar_tokens[b][m] = the final token
 *                 (other columns unspecified);
 *   commit_kv     unchanged (emits d_1..d_m and ar_tokens[b][m]);
 *   prefill       the first generated token is a sample of the last prompt
 *                 row's p.
 * Each emitted token is distributed as the frozen model's own sample at its
 * position, whatever the diffusion view drafts (drafts a caller replaces
 * keep this only if they are draws of q).  Random numbers: Philox4x32-10
 * keyed by seed, counter (index, sequence, step, purpose), uniform =
 * (x0 >> 8) * 2^-24 with x0 the first output word; step counts the
 * committed steps since this call; purposes 1 (draft of mask row i, index
 * i), 2 (acceptance of draft i, index i, 1-based), 3 (the final token, index
 * 0), 4 (the prefill's first token, index 0).  Host only; not while a step is
 * in flight (ESTATE).  Errors: EINVAL (T negative or not finite). */
int orthrus_set_sampling(orthrus_ctx* ctx, float temperature, uint64_t seed);

/* Per-layer parity taps (optional; NULL disables), for holding the library
 * to a reference one layer at a time from the library's own layer inputs.
 * resid: device fp32 [n_layers + 1][rows_cap][d_model]: entry l < n_layers
 * receives every later pass's layer-l input residual rows, entry n_layers
 * the final norm's input rows.  attn32: device fp32
 * [n_layers][rows_cap][n_q_heads*head_dim]: each layer's attention output
 * before its rounding to bf16 (bf16 models only; EINVAL otherwise).  Rows
 * are pass rows as for orthrus_set_debug; a pass with more rows than
 * rows_cap writes neither.  Errors: EINVAL. */
int orthrus_set_debug_layers(orthrus_ctx* ctx, float* resid, float* attn32, int32_t rows_cap);

/* Kernel (a) alone: block attention of `batch` sequences, bf16.  q: [batch]
 * [rows][n_q_heads][128]; k_cache: [batch][n_kv_heads][cap][128]; v_cache
 * in the library's tiled layout: [batch][n_kv_heads][cap/64][128][64] where
 * key j of a 64-key tile sits at column (j/32)*32 + ((j%16)/4)*8 +
 * ((j%32)/16)*4 + j%4; k_block: [batch][n_kv_heads][kpad][128]; v_block:
 * [batch][n_kv_heads][128][kpad] in the same column order per 32 keys
 * (kpad = block_len rounded up to 32).  Each row sees cache keys
 * [0, ctx_len) and all block_len block keys (the pages' mask-row view).
 * out: [batch][rows][n_q_heads][128] bf16.  workspace: at least
 * orthrus_attention_workspace(...) bytes.  cap must be a multiple of 64;
 * rows and block_len at most 64.  Errors: EINVAL, EHIP. */
int orthrus_block_attention(int32_t batch, int32_t rows, int32_t n_q_heads, int32_t n_kv_heads,
                            const void* q, const void* k_cache, const void* v_cache, int32_t cap,
                            int32_t ctx_len, const void* k_block, const void* v_block,
                            int32_t block_len, void* out, void* workspace, uint64_t workspace_bytes,
                            void* stream);
uint64_t orthrus_attention_workspace(int32_t batch, int32_t rows, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t ctx_len);

/* Kernel (a) alone without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results as
 * orthrus_block_attention, with the chunk partials in a scratch array that
 * the library's device code object holds on every GPU it runs on, for the
 * life of the process: ORTHRUS_NOALLOC_SCRATCH_BYTES (48 MiB; enough for
 * every point of the 32-row, 32/8-head microbenchmark up to 16 sequences x
 * 32768 keys).  The call allocates and frees nothing.  Calls needing more
 * than that (orthrus_attention_workspace) fail with ECAPACITY before
 * anything is enqueued.  All calls on one GPU share its array: calls that
 * may overlap on one GPU (several streams or host threads) race and must be
 * serialized by the caller.  Nothing in the array needs clearing between
 * calls (every partial the merge reads is written by the same call).  The
 * array's address is looked up on the first call on each device.  Arguments
 * and layouts as orthrus_block_attention.  Errors: EINVAL, ECAPACITY, EHIP. */
#define ORTHRUS_NOALLOC_SCRATCH_BYTES (48u << 20)
int orthrus_block_attention_noalloc(int32_t batch, int32_t rows, int32_t n_q_heads,
                                    int32_t n_kv_heads, const void* q, const void* k_cache,
                                    const void* v_cache, int32_t cap, int32_t ctx_len,
                                    const void* k_block, const void* v_block, int32_t block_len,
                                    void* out, void* stream);

/* The attention key chunk a context gets for attn_chunk = 0.  Every (chunk,
 * KV head, sequence) is one workgroup that writes a 64 KB partial, read back
 * once per pass.  The rule (measured on the decode workloads): the smallest
 * power of two in [128, 4096] that gives at most 64 chunks per sequence and
 * at most 1100 (chunk, KV head, sequence) workgroups, and at least 1024
 * whenever 1024-key chunks still give 512 of them (cap = the context's
 * kv_slots, see orthrus_sizes).  Kernel (a) alone (orthrus_block_attention)
 * chunks its ctx_len keys by its own rule: the smallest power of two in
 * [64, 16384] with at most 64 chunks per sequence and at most 512
 * workgroups (one round of two per compute unit).  Errors: EINVAL
 * (returned as a negative value). */
int32_t orthrus_default_attn_chunk(int32_t max_batch, int32_t max_ctx, int32_t n_kv_heads);

/* Measurement aid: the launch shape the library uses for a bf16 GEMM of m
 * rows (plus m2 rows of a second weight segment, as the draft pass's
 * projections have), n output features and k inputs, with epilogue 1
 * (residual), 2 (SwiGLU), 3 (LM-head argmax) or 4 (Q/K/V + QK-norm + RoPE).
 * plan (host, 6 ints): row tiles of 16 per workgroup, waves per workgroup,
 * 1 if K is split over workgroups (8 slices), 16-column tiles per wave
 * (column-split form) or per workgroup (row-split form), workgroups, and
 * the form: 0 = column-split (k_gemm_bf16: the waves of a workgroup split
 * its columns), 1 = row-split (k_gemm_rows: the waves split its rows), 2 =
 * row-split with two weight segments.  Host only.  Errors: EINVAL. */
int orthrus_gemm_plan(int32_t m, int32_t m2, int32_t n, int32_t k, int32_t epilogue,
                      int32_t* plan);

/* Measurement aid (not part of the decode step): n_workgroups workgroups
 * read the device buffer buf (bytes, a multiple of 16, 256-byte aligned)
 * once with 16-byte loads and write one XOR fold per workgroup to the device
 * array out[n_workgroups].  Timing it gives the device's achievable HBM
 * read rate for comparison with the published peak.  Errors: EINVAL, EHIP. */
int orthrus_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int32_t n_workgroups,
                        void* stream);

const char* orthrus_strerror(int code);
int orthrus_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ORTHRUS_H */

/*
 * i4decode -- int4 weight-streaming decode for MI355X (gfx950).
 *
 * One decode step of a dense grouped-query-attention decoder stack whose
 * weights are int4 codes plus bf16 group scales (the batch-1 path the pages
 * build their roofline argument on).  Per layer the library computes
 *
 *   h   = RMSNorm(x) * g1                          (Primer 1.1)
 *   q,k,v = Wq h, Wk h, Wv h                       (Primer 1.1; int4 expanded
 *                                                   in registers: Unsloth
 *                                                   article 二.3)
 *   q,k = RoPE(q, k; pos)                          (Roofline reply 五)
 *   cache[pos] = bf16(k), bf16(v)                  (Primer 1.2: append)
 *   o   = softmax(q K^T / sqrt(hd)) V over 0..pos  (Primer 1.1, 1.2; query head
 *                                                   h reads KV head h / (Hq/Hkv):
 *                                                   Unsloth article 二.2)
 *   y   = x + Wo o
 *   act = SiLU(Wg RMSNorm(y) g2) * (Wu RMSNorm(y) g2)   (Unsloth article 二.1)
 *   z   = y + Wd act
 *
 * and, for the LM head, the greedy token argmax_v (W_lm h)_v computed over the
 * vocabulary in chunks without materialising the logits (Unsloth article 三;
 * Primer 1.2).
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless the comment says "host".  Every
 *    buffer is allocated, owned and freed by the caller; the library never
 *    allocates, frees, synchronises or keeps state between calls.
 *  - bf16 values are carried as uint16_t bit patterns.  Activations are fp32.
 *  - `stream` is a hipStream_t passed as void*; all device work is enqueued on
 *    it, in order.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    negative return code means nothing was enqueued.  Faults inside kernels
 *    (a position outside the cache, a grid barrier that timed out) cannot be
 *    returned synchronously: they set a status word in the workspace that
 *    i4d_read_device_status() reports, and the kernels skip the offending work
 *    instead of touching memory out of bounds.
 *  - The workspace is caller-allocated device memory of at least
 *    i4d_workspace_size() bytes (never less than I4D_WS_MIN_BYTES), 256-byte
 *    aligned, initialised once with i4d_workspace_init() before first use (it
 *    clears the status word).  It is scratch between calls: no call reads what
 *    an earlier call left there.  Calls that share a workspace must be ordered
 *    on one stream.
 */
#ifndef I4DECODE_H
#define I4DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define I4D_OK            0
#define I4D_EINVAL       -1   /* null pointer, bad shape or group, Hq % Hkv != 0, ... */
#define I4D_EALIGN       -2   /* a pointer or pitch misses its required alignment */
#define I4D_EWORKSPACE   -3   /* workspace missing or smaller than i4d_workspace_size() */
#define I4D_ERANGE       -4   /* max_pos >= capacity, chunk_rows <= 0, batch out of range */
#define I4D_EHIP         -5   /* a HIP launch failed (hipGetLastError) */
#define I4D_EUNSUPPORTED -6   /* valid request this build does not implement */

/* smallest workspace any entry point accepts (header + LM-head argmax keys);
 * batches above 8 need more (i4d_workspace_size) */
#define I4D_WS_MIN_BYTES (16384 + 4096 * 32 * 8)

/* device status word bits (i4d_read_device_status) */
#define I4D_DEV_BAD_POS       1   /* pos[b] < 0, > max_pos or >= capacity: that sequence was skipped */
#define I4D_DEV_BARRIER_TIMEOUT 2 /* the streaming kernel gave up waiting for another workgroup's values */
#define I4D_DEV_BAD_TOKEN     4   /* a token id outside the embedding table: that row became zeros */
#define I4D_DEV_BAD_PAGE      8   /* a KV page id outside the pool: read as page 0, append dropped */
#define I4D_DEV_NONFINITE    16   /* an activation staged for a weight product was inf or NaN (used as 0) */

/* ---- weight matrices ---- */
#define I4D_WEIGHT_INT4 0
#define I4D_WEIGHT_BF16 1

/* A weight matrix W of n output rows and k inputs, applied as y = W x.
 *  I4D_WEIGHT_INT4: data   = uint8  codes  [n][k/2], row-major, two 4-bit
 *                            codes per byte, input index 2i in the low nibble;
 *                   scales = bf16   [n][ceil(k/group)], row-major; input i of
 *                            row r stands for (code - 8) * scales[r][i/group].
 *                   k % 8 == 0, group % 8 == 0, data 16-byte aligned.
 *  I4D_WEIGHT_BF16: data   = bf16 [n][k] row-major, scales = NULL, group
 *                   ignored, k % 8 == 0, data 16-byte aligned.              */
typedef struct i4d_mat {
    const void* data;
    const void* scales;
    int32_t n, k, group, dtype;
} i4d_mat;

/* One decoder layer (host struct of device pointers).  Shapes, with
 * qw = n_q_heads*head_dim, kvw = n_kv_heads*head_dim, D = d_model, F = d_ff:
 *   wq [qw][D], wk [kvw][D], wv [kvw][D], wo [D][qw], wg [F][D], wu [F][D],
 *   wd [D][F]; attn_norm, ffn_norm: bf16 [D].  All seven matrices share one
 *   dtype (and one group for int4).                                         */
typedef struct i4d_layer {
    const uint16_t* attn_norm;
    i4d_mat wq, wk, wv, wo;
    const uint16_t* ffn_norm;
    i4d_mat wg, wu, wd;
} i4d_layer;

/* Model shape.  head_dim must be 64 or 128; n_q_heads / n_kv_heads <= 16.
 * exec_mode selects how decode_layer/decode_stack run their phases:
 *   0 = auto: the streaming kernel (2) when the request qualifies, otherwise
 *       one launch per phase,
 *   1 = one kernel launch per phase,
 *   2 = the streaming kernel: one persistent launch per call runs every
 *       layer, its workgroups handing values to each other through tagged
 *       exchange words in the workspace (batch 1, int4 weights with groups of
 *       128, head_dim 128, d_model, d_ff and n_q_heads*128 multiples of 512,
 *       d_model and n_q_heads*128 <= 8192, contiguous caches of one capacity, at most 128
 *       layers; I4D_EUNSUPPORTED otherwise).                                */
typedef struct i4d_config {
    int32_t d_model, n_q_heads, n_kv_heads, head_dim, d_ff;
    float   rms_eps;
    double  rope_base;
    int32_t exec_mode;
} i4d_config;

/* KV cache of one layer, in tiles of 16 positions (each attention load then
 * reads whole cache lines).
 *
 * Contiguous (pages == NULL).  For sequence b, KV head j, position t, dim d:
 *   k (after RoPE): bf16 element at [b][j][t / 16][d / 32][t % 16][d % 32]
 *   v:              bf16 element at [b][j][t / 16][d][t % 16]
 * i.e. k is [B][n_kv_heads][capacity/16][head_dim/32][16][32] and v is
 * [B][n_kv_heads][capacity/16][head_dim][16].  capacity % 16 == 0.  Slot t of
 * sequence b holds the token at position t.
 *
 * Paged (pages != NULL; batches of sequences with their own lengths share one
 * pool).  k and v are pools of n_pages pages of page_size positions
 * (page_size % 16 == 0, capacity % page_size == 0), laid out per page as one
 * sequence's cache of capacity page_size: k [n_pages][n_kv_heads]
 * [page_size/16][head_dim/32][16][32], v [n_pages][n_kv_heads]
 * [page_size/16][head_dim][16].  pages is a device int32 table
 * [B][capacity / page_size]: position t of sequence b lives in page
 * pages[b * (capacity / page_size) + t / page_size] at offset
 * t % page_size.  capacity is the longest sequence the table can map.  Page
 * ids outside 0..n_pages-1 are never dereferenced: attention reads page 0
 * instead, the append is dropped, and I4D_DEV_BAD_PAGE is set in the
 * workspace status word.  The streaming kernel (exec_mode 2) does not take
 * paged caches (I4D_EUNSUPPORTED).                                            */
typedef struct i4d_kv {
    uint16_t* k;
    uint16_t* v;
    int32_t capacity;
    const int32_t* pages;    /* NULL: contiguous */
    int32_t page_size;       /* paged only */
    int32_t n_pages;         /* paged only */
} i4d_kv;

/* Bytes of workspace needed to run up to n_layers layers per call for this
 * shape, batch, largest position and vocabulary (0 if no LM head is used).
 * Pure host arithmetic; 0 for invalid arguments.                            */
size_t i4d_workspace_size(const i4d_config* cfg, int32_t n_layers, int32_t batch, int32_t max_pos, int32_t vocab);

/* Zero a fresh workspace, status word included (a fill kernel, no
 * hipMemset).  Needed once per workspace.                                   */
int i4d_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* One decoder layer for `batch` sequences (1 <= batch <= 32).
 * Batches of 1..8 stream the weights through the vector-ALU matrix-vector
 * core.  Batches of 9..32 run each projection as an int4 dequant-GEMM on the
 * matrix cores (the roofline reply, 二-三: batching raises the arithmetic
 * intensity past what the vector units sustain); that path needs int4
 * weights with groups of 128 or 256, an even number of groups per row,
 * 4-byte aligned scales, and d_model, d_ff and n_q_heads*head_dim multiples
 * of 256 (I4D_EUNSUPPORTED otherwise, before anything is enqueued).
 *   x_in  [B][D] fp32: hidden state of each sequence's new token.
 *   x_out [B][D] fp32: layer output z; must not alias x_in.
 *   pos   [B] int32 (device): number of cached tokens = position of the new
 *         token; attention covers slots 0..pos[b].  Slot pos[b] of every KV
 *         head is written (K after RoPE, V), no other slot is touched.
 *   max_pos (host): an upper bound on pos[b], < kv->capacity; it sizes the
 *         split of the key axis.                                            */
int i4d_decode_layer(const i4d_config* cfg, const i4d_layer* layer, int32_t batch,
                     const float* x_in, float* x_out, const i4d_kv* kv,
                     const int32_t* pos, int32_t max_pos,
                     void* ws, size_t ws_bytes, void* stream);

/* n_layers decoder layers applied in order (Primer 1.2's decode loop), each
 * layer's output feeding the next.  `layers` and `kv` are HOST arrays of
 * n_layers entries.  Same contract as i4d_decode_layer otherwise.           */
int i4d_decode_stack(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t batch,
                     const float* x_in, float* x_out, const i4d_kv* kv,
                     const int32_t* pos, int32_t max_pos,
                     void* ws, size_t ws_bytes, void* stream);

/* A chunk of n_tokens (1..32) consecutive prompt tokens of ONE sequence
 * through the stack at once (Primer 1.2: prefill computes, for every prompt
 * token, what decoding the tokens one after another would).  x_in/x_out
 * [n_tokens][D]; kv holds that sequence's cache (its batch dimension is 1);
 * pos [n_tokens] (device) gives each token's position, distinct and normally
 * consecutive (pos0, pos0+1, ...): token t attends to slots 0..pos[t] and its
 * K/V are appended at pos[t], so the cache must already hold the tokens before
 * pos[0].  Same weights, workspace (sized for batch = n_tokens) and
 * conditions as i4d_decode_stack; exec_mode 2 is not supported here.       */
int i4d_prefill_chunk(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t n_tokens,
                      const float* x_in, float* x_out, const i4d_kv* kv, const int32_t* pos, int32_t max_pos,
                      void* ws, size_t ws_bytes, void* stream);

/* Prefill of a whole prompt (Primer 1.2: prefill computes, for every prompt
 * token, what decoding the tokens one after another would): n_tokens
 * consecutive tokens of ONE sequence, at positions pos0 .. pos0+n_tokens-1,
 * through the n_layers layers at once.  The int4 projections run as GEMMs
 * with the prompt as the wide dimension (weights read once per 64-token
 * tile, not once per token), and attention is a causal attention tiled over
 * the prompt (Roofline reply 四): token t attends slots 0..pos0+t, where
 * slots below pos0 hold the sequence's earlier tokens and the prompt's own
 * K/V (bf16, RoPE applied to K) are appended at pos0+t.
 * x_in / x_out: [n_tokens][d_model] fp32 device, 16-byte aligned; x_out may
 * be x_in.  layers, kv: HOST arrays of n_layers entries; each kv is the
 * sequence's cache (batch dimension 1, contiguous or paged, row 0 of the page
 * table) and needs capacity > pos0+n_tokens-1.  Weights: int4, groups of 128
 * or 256 (one group size for all layers), every K a multiple of 256, d_model,
 * d_ff and Hq*head_dim multiples of 256; otherwise I4D_EUNSUPPORTED.
 * 1 <= n_tokens <= I4D_PREFILL_MAX_TOKENS.  ws: ws_bytes >=
 * i4d_prefill_workspace_size(cfg, n_tokens), 256-byte aligned, status word
 * as for the decode calls.  Enqueues kernels only (no memset, no
 * allocation), so the call can be captured in a graph.  Numerics:
 * activations enter the projections as fp16 (k and v rows: fp16 + fp16
 * remainder) times a power of two per token, accumulated in fp32.
 * Enqueued on `stream`; returns after enqueueing.                         */
#define I4D_PREFILL_MAX_TOKENS 65536
size_t i4d_prefill_workspace_size(const i4d_config* cfg, int32_t n_tokens);
int i4d_prefill(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t n_tokens,
                const float* x_in, float* x_out, const i4d_kv* kv, int32_t pos0,
                void* ws, size_t ws_bytes, void* stream);

/* Greedy LM head (Unsloth article 三; Primer 1.2): for each of `batch` hidden
 * states h [B][D] fp32, token_out[b] = lowest v maximising (W_lm h_b)_v and
 * max_logit_out[b] = that logit (fp32).  w_lm is int4 [V][D].  The page's
 * chunking bounds the logits held at once; here no logit leaves the
 * registers of the workgroup that computed it (each keeps a running argmax),
 * so the vocabulary is swept in passes as large as the kernel's per-workgroup
 * budget allows whatever chunk_rows is (chunk_rows > 0 is still required).
 * The result does not depend on chunk_rows.  1 <= batch <= 32; batches above
 * 8 run on the matrix cores (same weight conditions as i4d_decode_layer) and
 * need ws_bytes >= i4d_workspace_size(cfg, 1, batch, 0, V) for D = k;
 * otherwise ws_bytes >= I4D_WS_MIN_BYTES.                                    */
int i4d_lm_head_chunked(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows,
                        int32_t* token_out, float* max_logit_out,
                        void* ws, size_t ws_bytes, void* stream);

/* i4d_lm_head_chunked without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * i4d_lm_head_chunked for 1 <= batch <= 8 (the matrix-vector path); batch
 * above 8 returns I4D_ERANGE.  The per-workgroup argmax keys live in a
 * 256 KiB device array of the library (one per GPU, held until the process
 * ends); the entry point calls no allocator.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.                               */
int i4d_lm_head_chunked_noalloc(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows,
                                int32_t* token_out, float* max_logit_out, void* stream);

/* Temperature sampling from the same LM head (Primer 1.2 ends the step by
 * sampling a token from the logits; the pages name no sampler).  token_out[b]
 * is a draw from softmax((W_lm h_b) / temperature) by the Gumbel-max method:
 * the lowest v maximising logit_v / temperature + g_v, with
 * g_v = -log(-log(u_v)), u_v = (floor(x / 512) + 1/2) / 2^23 and x the first
 * output word of Philox4x32-10 (Salmon et al., SC'11) at counter
 * (v, b, counter[b], 0) and key (seed & 0xFFFFFFFF, seed >> 32).  The draw
 * depends only on those inputs, so any split of the vocabulary gives the same
 * token.  score_out[b] = the winning perturbed score.  temperature: positive
 * and finite with a normal fp32 reciprocal (else I4D_EINVAL).  counter: [B]
 * int32 (device), read by the kernels.  Everything else is as for
 * i4d_lm_head_chunked.                                                       */
int i4d_lm_head_sample(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows,
                       float temperature, uint64_t seed, const int32_t* counter,
                       int32_t* token_out, float* score_out,
                       void* ws, size_t ws_bytes, void* stream);

/* Top-k sampling (the decode loop's sample step of Primer 1.2 with the
 * optional top-k restriction): token_out[b] is a draw from
 * softmax(logits / temperature) renormalised over the top_k largest logits of
 * sequence b (equal logits ranked by lower id), i.e. the lowest v maximising
 * the perturbed score of i4d_lm_head_sample (same noise, same counter words)
 * among those top_k rows only.  top_k = V gives i4d_lm_head_sample's token,
 * top_k = 1 the greedy token.  score_out[b] = the winning perturbed score.
 * 1 <= top_k <= min(64, V), ceil(V / 1024) * top_k <= 16384 (else
 * I4D_ERANGE / I4D_EUNSUPPORTED).  Unlike the greedy and temperature heads,
 * the step's logits [B][V] (fp32) are written to the workspace, whose size
 * must be at least i4d_topk_workspace_size(w_lm, batch, top_k) (initialised
 * as for the decode calls).  Other arguments and conditions as for
 * i4d_lm_head_sample.                                                        */
size_t i4d_topk_workspace_size(const i4d_mat* w_lm, int32_t batch, int32_t top_k);
int i4d_lm_head_sample_topk(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t top_k,
                            float temperature, uint64_t seed, const int32_t* counter,
                            int32_t* token_out, float* score_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Embedding lookup (Primer 1.2: the decode loop starts from the embedding of
 * the last token): x_out[b] = fp32 of row tokens[b] of the bf16 table
 * [vocab][d_model] (row-major).  tokens [B] int32 (device); an id outside
 * 0..vocab-1 gives a zero row and sets I4D_DEV_BAD_TOKEN in the workspace
 * status word.  1 <= batch <= 32; ws is an initialised workspace (only its
 * status word is used, ws_bytes >= 16384).                                  */
int i4d_embed(const uint16_t* table, int32_t vocab, int32_t d_model, int32_t batch, const int32_t* tokens,
              float* x_out, void* ws, size_t ws_bytes, void* stream);

/* One whole greedy decode step (Primer 1.2's loop: embed the last token, run
 * every layer while appending its K/V, logits, pick the next token), all on
 * the device and in stream order, so a caller can capture it in a graph and
 * replay it per token:
 *   x      = i4d_embed(embed, tokens)          embed: bf16 [V][D], V = w_lm->n
 *   z      = i4d_decode_stack(x)               same contract as i4d_decode_stack
 *   tokens = argmax of w_lm z                  written IN PLACE over the input
 *                                              ids; max_logit_out [B] as in
 *                                              i4d_lm_head_chunked
 *   pos[b] += 1                                (device), after the step
 * x_buf: device scratch of 2 * batch * d_model fp32 (16-byte aligned) holding
 * x and z; z (the last hidden state) is left in its second half.  max_pos is
 * the host bound of i4d_decode_stack for this step's positions.  Every
 * argument of the four parts is validated before anything is enqueued.      */
int i4d_decode_step(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                    const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* max_logit_out, int32_t* pos,
                    int32_t max_pos, float* x_buf, const i4d_kv* kv, void* ws, size_t ws_bytes, void* stream);

/* i4d_decode_step with the token drawn as by i4d_lm_head_sample (Gumbel-max
 * at `temperature` with `seed`); the counter word of sequence b is pos[b] as
 * it is before this step's advance, so each step (and each replay of a
 * captured step) draws fresh noise.  score_out [B]: the winning perturbed
 * score.                                                                     */
int i4d_decode_step_sample(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                           const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* score_out, int32_t* pos,
                           int32_t max_pos, float* x_buf, const i4d_kv* kv, float temperature, uint64_t seed,
                           void* ws, size_t ws_bytes, void* stream);

/* i4d_decode_step with the token drawn by top-k sampling
 * (i4d_lm_head_sample_topk at top_k, temperature and seed; counter word of
 * sequence b = pos[b] before this step's advance).  ws_bytes must be at least
 * both i4d_workspace_size(cfg, n_layers, batch, max_pos, V) and
 * i4d_topk_workspace_size(w_lm, batch, top_k); at batch 1 the sampling
 * scratch must also end before the streaming kernel's region (true for
 * vocabularies up to about 200k), else I4D_EUNSUPPORTED.                     */
int i4d_decode_step_sample_topk(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                                const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* score_out, int32_t* pos,
                                int32_t max_pos, float* x_buf, const i4d_kv* kv, int32_t top_k, float temperature,
                                uint64_t seed, void* ws, size_t ws_bytes, void* stream);

/* Expand an int4 matrix to fp32 out [n][k]: out = (code - 8) * scale, exact
 * (Unsloth article 二.3).  A test hook for the int4 format.                 */
int i4d_dequant_int4(const i4d_mat* w, float* out, void* stream);

/* Plain y[b] = W x[b] through the core every projection of the layer uses
 * (x [B][k], y [B][n] fp32, 1 <= batch <= 32).  A test hook.  Batches of 1..8
 * take the matrix-vector core and ignore ws; batches of 9..32 take the
 * matrix-core GEMM (conditions as for i4d_decode_layer) and need an
 * initialised workspace of at least 2 MiB + 128 * k * (1 + n / 64) bytes.    */
int i4d_gemv(const i4d_mat* w, int32_t batch, const float* x, float* y,
             void* ws, size_t ws_bytes, void* stream);

/* Decode attention alone (Primer 1.1; Unsloth article 二.2; Roofline reply
 * 四): q [B][n_q_heads][head_dim] fp32 (already rotated), the cache of one
 * layer holding slots 0..pos[b], o [B][n_q_heads][head_dim] fp32.  Reads no
 * slot beyond pos[b].                                                        */
int i4d_attention(const i4d_config* cfg, int32_t batch, const float* q, const i4d_kv* kv,
                  const int32_t* pos, int32_t max_pos, float* o,
                  void* ws, size_t ws_bytes, void* stream);

/* Copy the workspace's device status word to *status_out (host) after the
 * stream's prior work; blocks until it is available.                       */
int i4d_read_device_status(const void* ws, int32_t* status_out, void* stream);

/* Measurement aid: time every launch of one kernel of the library.
 * Between i4d_launch_timing_start() and i4d_launch_timing_stop(), each launch
 * of `kernel` (one of I4D_TIME_*) is bracketed by two HIP events recorded on
 * the stream that the launch goes to, for at most max_launches launches
 * (1 <= max_launches <= 65536; later launches are not timed).  stop() waits
 * for the last event, writes the summed event-to-event time (ms) and the
 * number of timed launches, and turns timing off.  Process-wide state with
 * one user at a time: calls from several host threads race.  start() while
 * timing is on restarts it.  I4D_EINVAL for an unknown kernel or a bad
 * count, I4D_EHIP if an event cannot be made or read.                      */
/* Each kind names one phase of a layer; the kernel timed is the one that
 * phase runs on the path taken (phase launches, the batched matrix-core path,
 * or i4d_prefill's GEMMs and prompt attention).                            */
#define I4D_TIME_QKV        1   /* k_gemv_qkv / k_mfma_qkv / k_pf_qkv: QKV projection + RoPE + KV append */
#define I4D_TIME_ATTENTION  2   /* k_attention (split-K decode attention with its merge) / k_pf_attn */
#define I4D_TIME_WO         3   /* k_gemv_rows / k_mfma_rows / k_pf_rows on Wo (+ residual) */
#define I4D_TIME_GATE_UP    4   /* k_gemv_swiglu / k_mfma_swiglu / k_pf_swiglu: gate/up + SwiGLU */
#define I4D_TIME_DOWN       5   /* k_gemv_rows / k_mfma_rows / k_pf_rows on W_down (+ residual) */
#define I4D_TIME_LM_HEAD    6   /* k_lm_head / k_mfma_lm (one chunk of the LM head's rows), or the
                                   logits GEMV of top-k sampling */
#define I4D_TIME_STREAM     7   /* k_stream_decode: every layer of one call (events around the launch) */
int i4d_launch_timing_start(int32_t kernel, int32_t max_launches);
int i4d_launch_timing_stop(float* total_ms, int32_t* launches);

/* Measurement aid (not part of the decode path): read `bytes` of device
 * memory at buf once with 16-byte nontemporal loads (one 512-thread workgroup
 * per compute unit, four loads in flight per lane) and XOR every word into
 * *sink (device uint32, caller-owned).  The achievable streaming-read rate
 * the decode kernels are measured against.  buf 16-byte aligned, bytes a
 * multiple of 16 (I4D_EALIGN otherwise), bytes > 0 (I4D_EINVAL).           */
int i4d_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* i4d_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* I4DECODE_H */

/*
 * dlm.h -- C ABI of the block-diffusion denoising-round library for MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by title and section):
 *   [ORL-blog] "ORL: diffusion LLMs get a learnable 'tokens per forward' -- 2,788 tok/s
 *              on one RTX 5090, 7,708 on 8x B200, fully open source", section "What shipped":
 *              generation in blocks; each denoising round yields a distribution over the
 *              still-unresolved tokens; the previous round's distribution is fed back
 *              through a self-conditioning adapter on the tied embedding; positions that
 *              clear the commit bar are committed; the round loop of a block runs on the
 *              device with the continue decision taken after every round and the host only
 *              launching the block and reading tokens back.
 *   [ORL-card] "QwenDLM-4B-ORL" model card, section "The paper's evaluation pipeline":
 *              block decoding against a prefix KV cache, fused per-row statistics of the
 *              head, the commit step inside a captured graph.
 *
 * Conventions shared by every call:
 *   - Every call returns an int status (dlm_status).  Arguments are validated on the host,
 *     synchronously, before anything is enqueued; a failed call enqueues nothing.
 *     dlm_last_error() returns a thread-local description of the last failure.
 *   - Every call is enqueue-only on the caller's stream (a hipStream_t passed as void*;
 *     NULL is the default stream).  Device faults surface at the caller's next sync.
 *   - The caller owns every device buffer (weights, packed weights, KV cache, workspaces,
 *     outputs).  The library never allocates device memory.  dlm_model is a host-side
 *     handle holding pointers and shapes only.
 *   - Layouts are row-major and contiguous.  [out, in] is the weight convention.
 *     Token ids are int32; commit flags are uint8 0/1.
 *   - Data-dependent conditions (max rounds hit, non-finite statistics) are not errors;
 *     they are bits in the device-side round state (DLM_FLAG_*).
 *   - Results are bitwise deterministic for identical inputs (no float atomics).  Calls
 *     that share a workspace must not run concurrently.
 */
#ifndef DLM_H_
#define DLM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLM_ABI_VERSION 2
#define DLM_MAX_ROWS 64
#define DLM_MAX_ROUNDS 64

typedef enum {
  DLM_OK = 0,
  DLM_ERR_ARG = -1,         /* null pointer where one is required, negative size */
  DLM_ERR_SHAPE = -2,       /* unsupported or inconsistent shape */
  DLM_ERR_DTYPE = -3,       /* unsupported dtype */
  DLM_ERR_WORKSPACE = -4,   /* workspace too small */
  DLM_ERR_HIP = -5,         /* HIP launch / API failure */
  DLM_ERR_UNSUPPORTED = -6  /* device is not gfx950 */
} dlm_status;

typedef enum { DLM_F32 = 0, DLM_BF16 = 1, DLM_MXFP4 = 2, DLM_FP8_E4M3 = 3 } dlm_dtype;

typedef enum { DLM_COMMIT_THRESHOLD = 0, DLM_COMMIT_FIXED_K = 1 } dlm_commit_mode;

enum { DLM_FLAG_HIT_MAX_ROUNDS = 1, DLM_FLAG_NONFINITE = 2 };

int dlm_abi_version(void);
const char* dlm_last_error(void);

/* ------------------------------------------------------------------------------------
 * dlm_block_attn -- attention of a block of B query positions to a prefix KV cache of
 * length L plus the block's own B keys, with no mask: every block query sees all L + B
 * keys ([ORL-blog] "What shipped": a block's unresolved tokens are predicted together;
 * [ORL-card] evaluation pipeline: block decoding against a prefix KV cache).
 * Grouped-query attention: query head h reads kv head h / (hq / hkv).
 *
 *   q        [B, hq, D]     query rows, RoPE already applied.
 *   k_cache  [hkv, cap, D]  keys; rows [0, L) are the prefix, [L, L+B) the block.
 *   v_cache  [hkv, cap/32, D, 32]  values, stored transposed in blocks of 32 key positions:
 *                           column j of key position t of kv head h is
 *                           v_cache[h][t / 32][j][t % 32], so consecutive keys of one value
 *                           column are contiguous and a 32-key block is one contiguous run;
 *                           positions as for k_cache.  cap % 32 == 0.
 *   out      [B, hq, D]     o = softmax(scale * q k^T) v, same dtype as q.
 *   L is desc->prefix_len, or *desc->prefix_len_dev when that device pointer is non-null
 *   (so a captured graph can replay with a growing prefix).  Shapes: D in {64, 128},
 *   hq % hkv == 0, 1 <= B <= 64, L + B <= cap.
 *   ws: device scratch of at least dlm_block_attn_ws_bytes(desc) bytes (the key splits'
 *   partial outputs; no zeroing needed: every partial read was written by the same call).
 *   FP8 cache (kv_dtype = DLM_FP8_E4M3, with dtype = DLM_BF16): k_cache and v_cache hold one
 *   OCP FP8 e4m3 code per element in the same layouts, and the stored key (value) is
 *   k_scale (v_scale) times the code's value; q and out stay bf16.  [ORL-blog] "What shipped"
 *   states that the engine keeps its KV cache in FP8 on Blackwell; it gives no element format
 *   or scaling, and one e4m3 code per element with one scale per cache is this library's
 *   reading.
 *   The caller writes the codes; NaN codes must not occur at positions below L + B.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int dtype;            /* DLM_BF16 or DLM_F32 (q and out; the caches too unless kv_dtype says FP8) */
  int hq, hkv, head_dim, block, cap;
  float softmax_scale;  /* usually 1/sqrt(head_dim) */
  int prefix_len;       /* host value of L (used if prefix_len_dev is NULL) */
  const int32_t* prefix_len_dev;
  int max_prefix_len;   /* upper bound of L when prefix_len_dev is used (sizes the workspace) */
  int kv_dtype;         /* equal to dtype, or DLM_FP8_E4M3 (dtype DLM_BF16 only) */
  float k_scale, v_scale;   /* FP8 cache scales: finite and > 0 (ignored otherwise) */
} dlm_attn_desc;

size_t dlm_block_attn_ws_bytes(const dlm_attn_desc* desc);
int dlm_block_attn(const dlm_attn_desc* desc, const void* q, const void* k_cache,
                   const void* v_cache, void* out, void* ws, size_t ws_bytes, void* stream);

/* dlm_block_attn_noalloc -- dlm_block_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the split partials in a scratch area the library holds on
 * each GPU it runs on (dlm_block_attn_noalloc_max_bytes() bytes, 16 MiB, kept until the process
 * ends); no allocating call is made.  Arguments and errors as dlm_block_attn, without the
 * workspace; DLM_ERR_WORKSPACE when dlm_block_attn_ws_bytes(desc) exceeds the scratch (at
 * 32 / 8 heads of 128 and 32 queries the largest plan needs 8,650,752 bytes).  All calls on one GPU
 * share its scratch: calls that overlap in time on one GPU (concurrent streams) race. */
size_t dlm_block_attn_noalloc_max_bytes(void);
int dlm_block_attn_noalloc(const dlm_attn_desc* desc, const void* q, const void* k_cache,
                           const void* v_cache, void* out, void* stream);

/* ------------------------------------------------------------------------------------
 * dlm_head_rowstats -- tied-embedding head fused with per-row statistics and the p.E
 * feedback mix ([ORL-blog] "What shipped": per-round distribution, self-conditioning on
 * the tied embedding; [ORL-card] evaluation pipeline: fused row statistics).  For every
 * open row i (committed == NULL or committed[i] == 0), with l = h_i E^T over the whole
 * vocabulary (never written to memory):
 *   lse = max l + ln sum exp(l - max l);  entropy = -sum p ln p (nats);
 *   maxprob = max p;  argmax = lowest id with l == max l;  pe = sum_v p_v E_v.
 * Committed rows get argmax = -1, lse = entropy = maxprob = 0 and a zero pe row.
 *
 *   h          [rows, d]  final-normed hidden rows (dtype).
 *   emb        [V, d]     tied embedding (dtype).
 *   committed  [rows] u8 or NULL.
 *   lse, entropy, maxprob [rows] f32;  argmax [rows] i32;  pe [rows, d] f32 or NULL.
 *   logits_dbg [rows, V] f32 or NULL (tests only; costs an extra write of the logits).
 * Shapes: 1 <= rows <= 64, d % 32 == 0, d <= 4096, V >= 1.
 * ws: at least dlm_head_rowstats_ws_bytes(desc) bytes (no zeroing needed).
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int dtype;
  int rows, d, vocab;
} dlm_head_desc;

size_t dlm_head_rowstats_ws_bytes(const dlm_head_desc* desc);
int dlm_head_rowstats(const dlm_head_desc* desc, const void* h, const void* emb,
                      const uint8_t* committed, float* lse, float* entropy, float* maxprob,
                      int32_t* argmax, float* pe, float* logits_dbg, void* ws, size_t ws_bytes,
                      void* stream);

/* ------------------------------------------------------------------------------------
 * dlm_commit -- one round's confidence commit ([ORL-blog] "What shipped": positions that
 * clear the commit bar are committed; more clearing means fewer rounds per block).
 *   THRESHOLD: commit open rows with maxprob >= tau, plus (forced_top1) the open row with
 *              the largest maxprob.   FIXED_K: the min(k, n_open) open rows with the
 *              largest maxprob.  Ties rank the lower row first; NaN ranks as -inf.
 *   In round max_rounds - 1 every open row is committed (DLM_FLAG_HIT_MAX_ROUNDS if that
 *   committed more than the rule would).  A committed row is never reopened; its token
 *   is its argmax.
 *   maxprob [rows] f32, argmax [rows] i32 (inputs); committed [rows] u8, tokens [rows] i32
 *   (updated in place); state: device dlm_round_state (round, n_open, cont, flags,
 *   n_new[round] updated).  Does nothing when state->cont == 0.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int mode;         /* dlm_commit_mode */
  float tau;
  int k;
  int forced_top1;
  int max_rounds;   /* 1 .. DLM_MAX_ROUNDS */
} dlm_commit_rule;

typedef struct {
  int32_t round;    /* rounds run so far in this block */
  int32_t n_open;   /* open rows */
  int32_t cont;     /* 1 while the block loop continues */
  int32_t flags;    /* DLM_FLAG_* */
  int32_t n_new[DLM_MAX_ROUNDS];  /* commits per round */
} dlm_round_state;

int dlm_commit(const dlm_commit_rule* rule, int rows, const float* maxprob,
               const int32_t* argmax, uint8_t* committed, int32_t* tokens,
               dlm_round_state* state, void* stream);

/* Reset a block: committed = 0, tokens = 0, state = {0, rows, 1, 0, 0...}. */
int dlm_block_reset(int rows, uint8_t* committed, int32_t* tokens, dlm_round_state* state,
                    void* stream);

/* ------------------------------------------------------------------------------------
 * dlm_selfcond -- the round's input rows ([ORL-blog] "What shipped": the previous round's
 * distribution is fed back through a self-conditioning adapter on the tied embedding, so
 * each round starts from the model's own last guess).
 *   x_i = E[tokens_i]                       if committed_i
 *   x_i = mask_emb + W_sc . bf(pe_prev_i)   otherwise (pe_prev NULL: x_i = mask_emb)
 *   tokens [rows] i32, committed [rows] u8, emb [V, d], mask_emb [d], w_sc [d, d] (dtype;
 *   for DLM_BF16 w_sc is the packed form written by dlm_pack_matrix), pe_prev [rows, d] f32
 *   or NULL, x_out [rows, d] f32.  bf() rounds to the dtype (bf16 for DLM_BF16).
 * ws: at least dlm_selfcond_ws_bytes(desc) bytes, zeroed once before first use.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int dtype;
  int rows, d, vocab;
} dlm_selfcond_desc;

size_t dlm_selfcond_ws_bytes(const dlm_selfcond_desc* desc);
int dlm_selfcond(const dlm_selfcond_desc* desc, const int32_t* tokens, const uint8_t* committed,
                 const void* emb, const void* mask_emb, const void* w_sc, const float* pe_prev,
                 float* x_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Weight packing.  bf16 matrices used by the skinny GEMMs are re-laid out once, at model
 * load, so that every 32-row x 16-column tile is one contiguous 1 KiB run in the order
 * the matrix cores consume it (v_mfma_f32_32x32x16_bf16 A operand: lane l holds the 8
 * columns 8(l/32).. of row l%32).  dlm_pack_matrix packs W[n_rows, k] (bf16, [out, in]);
 * rows are taken in the order given by row_map (NULL = identity; row_map[i] is the source
 * row of packed row i).  n_rows % 32 == 0, k % 32 == 0.  dst holds n_rows * k bf16.
 * ------------------------------------------------------------------------------------ */
int dlm_pack_matrix(const void* src, int n_rows, int k, const int32_t* row_map_dev, void* dst,
                    void* stream);

/* ------------------------------------------------------------------------------------
 * dlm_linear -- y = x W^T for the block's rows with a packed bf16 weight: the stream-K skinny
 * matrix-core GEMM that the round uses for its split-K projections (attention output, FFN
 * down, self-conditioning adapter), with a plain f32 store as its epilogue.
 *   w_packed [n, k] packed by dlm_pack_matrix;  x: 32 x k bf16 in the packed activation
 *   order written by dlm_pack_activations (rows >= m are read but ignored);  y [m, n] f32.
 *   1 <= m <= 32, n % 32 == 0, k % 32 == 0.  ws: dlm_linear_ws_bytes(n, k) bytes, zeroed
 *   once before first use.
 * dlm_pack_activations -- x [rows, k] bf16 row-major -> the packed activation order: for
 *   16-column step kt the 64 lanes' 16-byte pieces X[l % 32][16 kt + 8 (l / 32) .. +8] form one
 *   contiguous 1 KiB run (rows >= `rows` up to 32 are zero).  x_packed holds 32 * k bf16.
 * ------------------------------------------------------------------------------------ */
size_t dlm_linear_ws_bytes(int n, int k);
int dlm_linear(const void* w_packed, const void* x, int m, int n, int k, float* y, void* ws,
               size_t ws_bytes, void* stream);
int dlm_pack_activations(const void* x, int rows, int k, void* x_packed, void* stream);

/* ------------------------------------------------------------------------------------
 * Model.  Weight pointers (device) in natural layout for DLM_F32; for DLM_BF16 the
 * matrices wqkv / wgu / wo / wd / w_sc must be packed by dlm_pack_model into one buffer
 * of dlm_packed_bytes(desc) bytes (see dlm_pack_model).
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int dtype;                 /* DLM_F32 or DLM_BF16 */
  int n_layers, d, hq, hkv, head_dim, ffn, vocab, block;
  float rope_base, eps;
  int n_experts, expert_ffn, top_k, n_shared;  /* 0 for dense models */
  int layer_path;            /* DLM_LAYERS_PER_OP (0): one kernel per step of a layer;
                                DLM_LAYERS_FUSED (1): one launch per sublayer with XCD-local
                                synchronisation, for dense bf16 models with 8 kv heads of 4 query
                                heads of 128, 32-row blocks, d % 512 == 0 and ffn % 256 == 0
                                (other models take the per-op kernels);
                                DLM_LAYERS_ATTN_OUT (2): the per-op kernels, except that the
                                attention and its output projection run as one launch (forwards
                                of 32 and 64 rows) on dense bf16 models with 8 kv heads of 4
                                query heads of 128, 32-row blocks, d % 512 == 0 and d <= 3072.
                                The packed layout depends on it: pack and create with the same
                                value. */
} dlm_model_desc;

enum { DLM_LAYERS_PER_OP = 0, DLM_LAYERS_FUSED = 1, DLM_LAYERS_ATTN_OUT = 2 };

typedef struct {
  const void* attn_norm;     /* [d] */
  const void* wq;            /* [hq*D, d] */
  const void* wk;            /* [hkv*D, d] */
  const void* wv;            /* [hkv*D, d] */
  const void* wo;            /* [d, hq*D] */
  const void* ffn_norm;      /* [d] */
  const void* wg;            /* [F, d] (dense) */
  const void* wu;            /* [F, d] (dense) */
  const void* wd;            /* [d, F] (dense) */
  const void* router;        /* [n_experts, d] bf16 (MoE) */
  const void* x_w13;         /* MoE experts: packed MXFP4 gate/up  (see dlm_moe_layout) */
  const void* x_w13_scale;
  const void* x_w2;          /* MoE experts: packed MXFP4 down */
  const void* x_w2_scale;
} dlm_layer_weights;

typedef struct dlm_model dlm_model;

/* Creates a host handle.  emb [V, d], mask_emb [d], w_sc [d, d], final_norm [d]; layers
 * is an array of n_layers entries (copied).  packed: the buffer written by dlm_pack_model
 * (DLM_BF16; NULL for DLM_F32).  No device memory is allocated. */
int dlm_model_create(const dlm_model_desc* desc, const void* emb, const void* mask_emb,
                     const void* w_sc, const void* final_norm, const dlm_layer_weights* layers,
                     const void* packed, dlm_model** out);
void dlm_model_destroy(dlm_model* m);

/* Bytes of the packed-weights buffer of a bf16 model (0 for f32). */
size_t dlm_packed_bytes(const dlm_model_desc* desc);
/* Pack every bf16 GEMM matrix of the model (natural layouts in emb/w_sc/layers) into dst.
 * row_map_ws: device scratch of at least dlm_pack_ws_bytes(desc) bytes. */
size_t dlm_pack_ws_bytes(const dlm_model_desc* desc);
int dlm_pack_model(const dlm_model_desc* desc, const void* w_sc, const dlm_layer_weights* layers,
                   void* dst, void* row_map_ws, size_t ws_bytes, void* stream);

/* One sublayer of a packed dense bf16 model on its own, with the kernel and launch plan that
 * dlm_decode_block uses for it: layer `layer`'s FFN gate/up projection fused with SwiGLU,
 * act = silu(x Wg^T) * (x Wu^T), for the block's rows (the FFN form of the layer that the
 * round forwards; the largest weight stream of the round).
 *   x_packed: bf16 32 x d and act_packed: bf16 32 x ffn, both in the packed activation order
 *   of dlm_pack_activations.  ws: dlm_ffn_gate_up_ws_bytes(m) bytes, zeroed once before first
 *   use.  Errors: DLM_ERR_DTYPE for f32 or MoE models, DLM_ERR_ARG for a layer out of range. */
size_t dlm_ffn_gate_up_ws_bytes(const dlm_model* m);
int dlm_ffn_gate_up(const dlm_model* m, int layer, const void* x_packed, void* act_packed, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * KV cache.  k[l]: device base of layer l's keys [hkv, cap, D]; v[l]: its values stored
 * transposed in 32-position blocks, [hkv, cap/32, D, 32] (as for dlm_block_attn); model
 * dtype, or FP8 for bf16 models (kv_dtype = DLM_FP8_E4M3: one e4m3 code per element, the
 * stored value being k_scale (v_scale) times the code's value; the layers write the code of
 * their bf16 k (v) divided by the scale, nearest-even, saturating at 448, and attend as
 * dlm_block_attn does over such a cache); cap % 32 == 0.
 * len_dev: device int32 holding the committed prefix length L.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  void* const* k;            /* host array of n_layers device pointers */
  void* const* v;
  int cap;
  int32_t* len_dev;
  int max_len;               /* largest L + block the caller will use (sizes workspaces) */
  int kv_dtype;              /* the model dtype, or DLM_FP8_E4M3 (bf16 models) */
  float k_scale, v_scale;    /* FP8 cache scales: finite and > 0 (ignored otherwise) */
} dlm_kv;

/* ------------------------------------------------------------------------------------
 * dlm_decode_block -- decode one block of `block` fully masked positions after the cached
 * prefix, entirely on the device ([ORL-blog] "What shipped": one launch per block, the
 * denoising loop stays on the GPU, the continue decision is taken after every round, the
 * host only reads tokens back).  Enqueues ceil(block / k) rounds (FIXED_K) or max_rounds
 * rounds (THRESHOLD; rounds after the block is complete exit immediately), each round =
 * self-conditioning input, every layer, final norm, head statistics, commit; then a commit
 * pass that forwards the committed tokens and writes their K/V at [L, L + block), and
 * L += block.  No host synchronisation inside; the first call with a given set of buffers
 * captures the sequence into a HIP graph that later calls replay.
 *   tokens [block] i32 (out), state: device dlm_round_state (out; n_new per round,
 *   rounds used, flags).  ws: dlm_decode_ws_bytes(model, kv) bytes, zeroed once before
 *   first use.  Every device input must stay valid while the captured graph may replay.
 * ------------------------------------------------------------------------------------ */
size_t dlm_decode_ws_bytes(const dlm_model* m, const dlm_kv* kv);
int dlm_decode_block(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                     int32_t* tokens, dlm_round_state* state, void* ws, size_t ws_bytes,
                     void* stream);

/* dlm_decode_block_pipelined -- dlm_decode_block with the block's own commit pass left
 * pending, so that the next block can carry it.  The call decodes the block in `tokens`
 * exactly as dlm_decode_block does, but first completes the PREVIOUS block's pending commit
 * pass (prev_tokens: that block's committed tokens [block] i32, device; NULL when no block is
 * pending) and ends without appending this block's K/V: after it, L has grown by the previous
 * block only, and this block is pending.  A run of blocks is therefore
 *   pipelined(prev = NULL, t0), pipelined(t0, t1), ..., pipelined(t_{n-2}, t_{n-1}),
 *   dlm_commit_pass(t_{n-1})
 * and produces the same tokens and cache as dlm_decode_block on each block in turn: the commit
 * pass is the forward of the clean block whose K/V the next block attends to ([ORL-blog]
 * "What shipped"), and nothing in round 0 of the next block depends on it other than those
 * K/V.  For bf16 models (dense and MoE) with block = 32 the commit rows ride along with round
 * 0 as one 64-row forward (rows 0..31: the previous block at positions L .. L + 31; rows
 * 32..63: round 0 at L + 32 .., attending to the prefix, the previous block and each other;
 * in a MoE layer all 64 rows are routed together), so the layer weights stream once for
 * both; f32 models run the commit pass on its own first.
 *   prev_tokens must not alias tokens and must hold the previous block's final tokens until
 *   the call's work has run.  The cache must have room for both blocks: L + 2 block <=
 *   max_len at the call (the kernels write no K/V at or past cap).  Other arguments and
 *   errors as dlm_decode_block; DLM_ERR_ARG when prev_tokens == tokens.
 *   The debug views' x after a pipelined round 0 holds the 64 rows of the fused forward. */
int dlm_decode_block_pipelined(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                               const int32_t* prev_tokens, int32_t* tokens, dlm_round_state* state,
                               void* ws, size_t ws_bytes, void* stream);

/* dlm_decode_block for threshold rules without the rounds that run after the block is done.
 * A graph cannot branch on the device here (HIP graphs have no conditional nodes), so
 * dlm_decode_block enqueues max_rounds rounds and every kernel of a round after the block's
 * end reads the continue flag and exits -- still one launch each.  This call replays graphs of
 * seg_rounds rounds instead, one segment ahead of the one it waits for: after each segment
 * the continue flag is copied to pinned host memory behind an event, the calling thread
 * waits for that event, and no further segment is launched once the block is done; then it
 * enqueues the commit pass and returns.  So at most one segment (seg_rounds rounds) runs
 * without work, and the device never waits on the host while work remains.  Same tokens,
 * state and cache as dlm_decode_block ([ORL-blog] "What shipped": the loop stops when the
 * block is done).  Blocks the calling thread (unlike the other calls); a fixed-k rule (whose
 * round count is known) takes dlm_decode_block's graph and does not block.  Calls on one
 * model are serialised.  Other arguments and errors as dlm_decode_block; DLM_ERR_ARG for
 * seg_rounds < 1. */
int dlm_decode_block_gated(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                           int32_t* tokens, dlm_round_state* state, void* ws, size_t ws_bytes,
                           int seg_rounds, void* stream);

/* The prompt: forwards over the n / block consecutive blocks of ids (device int32 [n], n %
 * block == 0) that append every block's K/V; L += n.  Each forward takes several blocks at
 * once, block-causally (a block's rows attend to the cached prefix, to the earlier blocks of
 * the forward and to each other), so its K/V are those of one commit pass per block, and the
 * weights stream once per forward instead of once per block.  The prompt is processed as a
 * whole, compute-dense pass, unlike the decode steps ([ORL-news] "dLLM 是什么，为什么能并行生成",
 * on the prefill and decode phases).  Dense bf16 models with block = 32 take up to 8 blocks (256
 * rows) per forward, the other bf16 models with block = 32 (MoE) 2 blocks, f32 models 1; a
 * last forward takes what is left.  ws as for dlm_decode_block. */
int dlm_prefill(const dlm_model* m, const int32_t* ids, int n, const dlm_kv* kv, void* ws,
                size_t ws_bytes, void* stream);

/* dlm_prefill with at most max_rows rows per forward (max_rows >= block; rounded down to whole
 * blocks and to what the model takes): max_rows = block gives one commit pass per block.  The
 * caches agree with dlm_prefill's up to float summation order (a wider forward sums its GEMMs'
 * products in another order).  DLM_ERR_ARG for max_rows < block. */
int dlm_prefill_rows(const dlm_model* m, const int32_t* ids, int n, const dlm_kv* kv, void* ws,
                     size_t ws_bytes, int max_rows, void* stream);

/* Debug/test hooks on the decode workspace (device pointers into ws; NULL if absent). */
typedef struct {
  float* x;          /* [block, d] residual stream of the last forward ([64, d] after a fused
                        round 0 of dlm_decode_block_pipelined) */
  void* hn;          /* [block, d] final-normed rows (model dtype) */
  float* pe;         /* [block, d] p.E of the last round */
  float* lse;        /* [block] */
  float* entropy;    /* [block] */
  float* maxprob;    /* [block] */
  int32_t* argmax;   /* [block] */
  uint8_t* committed;/* [block] */
  void* xn;          /* 32 x d bf16 in the packed activation order: the last RMSNorm output that
                        fed a GEMM (for MoE models, the input of the last routed-expert FFN) */
  /* MoE models, state of the last routed-expert FFN that ran (NULL for dense models):
   * router logits [32][E] f32; f as MXFP8: codes [32][d] e4m3 and e8m0 scales [32][d/32];
   * each row's top-k experts by rank [32][top_k] i32 and their probabilities [32][top_k] f32;
   * act as MXFP8 per slot (row * NS + rank, shared experts after the routed ranks): codes
   * [32*NS][F], scales [32*NS][F/32]; weighted expert outputs per slot y [32*NS][d] f32
   * (NS = top_k + n_shared). */
  float* moe_logits;
  uint8_t* moe_xq;
  uint8_t* moe_xs;
  int32_t* moe_ids;
  float* moe_wts;
  uint8_t* moe_aq;
  uint8_t* moe_as;
  float* moe_y;
  int32_t* moe_hits;   /* [n_layers]: running count, per layer, of the distinct experts (shared
                          included) each routed-expert FFN used since the workspace was zeroed */
  int32_t* sync_err;   /* models whose kernels synchronise inside an XCD -- the fused layer
                          path, and bf16 models with 32-row blocks whose attention has 8 groups
                          of (kv head, up to 4 of its query heads), which merge the key splits
                          inside the attention launch -- 288 words: word 0 is 0 unless an
                          XCD-local barrier gave up waiting (bit 0) or a workgroup did not share
                          the XCD of its group, blockIdx % 8 (bit 1) -- then the results are not
                          to be trusted; word 32 (1 + g) holds the XCC id group g ran on in the
                          last launch.  NULL for other models */
} dlm_decode_views;
int dlm_decode_views_get(const dlm_model* m, const dlm_kv* kv, void* ws, size_t ws_bytes,
                         dlm_decode_views* out);

/* Graph cache diagnostics (host only, no device work).  dlm_block_graph_key writes the key
 * under which dlm_decode_block (pipelined = 0) or dlm_decode_block_pipelined (pipelined = 1)
 * caches its captured graph for these arguments into words[0 .. n) and returns n (or a
 * negative status; DLM_ERR_ARG when max_words < n): the rule, the tokens, state, workspace and
 * prefix-length addresses, every layer's K and V base, the cache capacity, max_len, format and
 * scales.  Launches whose keys differ never share a graph.  dlm_model_graph_count returns the
 * number of graphs the model holds. */
int dlm_block_graph_key(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                        const int32_t* prev_tokens, int pipelined, const int32_t* tokens,
                        const dlm_round_state* state, const void* ws, uint64_t* words, int max_words);
int dlm_model_graph_count(const dlm_model* m);

/* One round only (no commit pass), from the state held in ws (tests: lockstep parity).
 * round_index is the index of this round in the block (device state is used for the
 * commit; the host value only selects nothing and is accepted for logging). */
int dlm_decode_round(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                     int32_t* tokens, dlm_round_state* state, void* ws, size_t ws_bytes,
                     void* stream);
/* Reset the block state held in ws (committed = 0, pe = 0) and state. */
int dlm_decode_begin(const dlm_model* m, const dlm_kv* kv, int32_t* tokens,
                     dlm_round_state* state, void* ws, size_t ws_bytes, void* stream);
/* The commit pass alone: forwards tokens [block] at [L, L+block) and sets L += block. */
int dlm_commit_pass(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, void* ws,
                    size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H_ */

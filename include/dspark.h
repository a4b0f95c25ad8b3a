/*
 * dspark.h -- C ABI of the MI355X (gfx950) DSpark draft-round library.
 *
 * One draft round of the DeepSpec DSpark semi-autoregressive drafter, as the
 * page "@mlx-bun/inference 0.0.0-stage -> 1.0.0,
 * package/src/models/speculative/deepspec.ts" (cited "deepspec.ts") and its
 * earlier revision "mlx-bun 0.2.0 -> 0.4.0,
 * package/src/spec/dspark/deepspec-module.ts" (cited "deepspec-module.ts")
 * transcribe it:
 *   context rows -> per-layer context K/V   (dspark_project_context_kv)
 *   [anchor, MASK x (gamma-1)] -> backbone -> softcapped logits -> greedy
 *   Markov walk                              (dspark_draft_rows / _block)
 *
 * Conventions for every call:
 *  - Pointers named *_dev are device pointers on the current HIP device;
 *    *_host are host pointers read before the call returns.
 *  - Every check runs on the host before any HIP call.  A non-OK status
 *    means nothing was enqueued and no output was touched;
 *    dspark_last_error() then describes the problem (thread-local).
 *  - Work is enqueued on `stream` and is asynchronous; device faults surface
 *    at the caller's next synchronisation of that stream.
 *  - The library allocates no device memory.  Weights are borrowed for the
 *    model's lifetime; every other pointer only for the duration of the call
 *    and the work it enqueues.  No C++ exception crosses this boundary.
 *  - Calls on one model may overlap only if they use distinct workspaces.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, id or position out of range */
  DSPARK_ERR_SHAPE = 2,       /* sizes that disagree with the model or with each other */
  DSPARK_ERR_UNSUPPORTED = 3, /* config variant the drafter refuses, or a dtype/shape not built */
  DSPARK_ERR_WORKSPACE = 4,   /* workspace or aux buffer too small / misaligned */
  DSPARK_ERR_HIP = 5          /* a HIP launch error, with hipGetErrorString in the message */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1, DSPARK_Q4 = 2 } dspark_dtype;

/* Drafter config: the config.json fields of deepspec.ts, DeepspecConfig and
 * readConfig.  readConfig refuses attention_k_eq_v == 0, a Markov head other
 * than "vanilla" when markov_rank > 0, and any activation other than
 * gelu_pytorch_tanh; dspark_model_create refuses the same with
 * DSPARK_ERR_UNSUPPORTED, except the RNN head (markov_head_rnn below). */
typedef struct {
  int32_t hidden_size;                /* H */
  int32_t num_hidden_layers;
  int32_t num_attention_heads;        /* nH */
  int32_t global_head_dim;            /* hd: 64, 128 or 256 */
  int32_t num_global_key_value_heads; /* nKv, divides nH */
  int32_t intermediate_size;          /* I */
  int32_t vocab_size;                 /* V */
  int32_t block_size;                 /* gamma, 1..32 */
  int32_t mask_token_id;
  int32_t markov_rank;                /* r; 0 = no Markov head (plain argmax) */
  int32_t attention_k_eq_v;           /* must be 1 */
  int32_t markov_head_vanilla;        /* must be 1 when markov_rank > 0 */
  int32_t activation_gelu_tanh;       /* must be 1 */
  int32_t fc_in;                      /* taps * target hidden; 0 = no fc / hidden_norm */
  double rope_theta;
  double partial_rotary_factor;
  double rms_norm_eps;
  double final_logit_softcapping;     /* <= 0: no softcap */
  int32_t weight_dtype;               /* matmul weights and gather tables: F32, BF16 or Q4 */
  int32_t act_dtype;                  /* norm vectors, layer_scalar, context K/V, X inputs: F32 or BF16 */
  int32_t group_size;                 /* Q4 group along the input axis (64) */
  /* deepspec.ts, DeepspecConfig: the confidence head (a Linear(confDim, 1)
   * with bias, "confidence_head.proj.weight" [1, confDim] in the weight dtype
   * and "confidence_head.proj.bias" [1] in the act dtype; confDim = H, plus
   * markov_rank when it also reads markov_w1[previous token]) and the
   * truncation threshold (<= 0: every row keeps its whole block). */
  int32_t enable_confidence_head;
  int32_t confidence_head_with_markov;  /* needs markov_rank > 0 */
  double confidence_threshold;
  /* The RNN sequential head (markov_head_type "rnn"; markov_head_vanilla 0):
   * the bias of block slot k is markov_w2 s_k with
   * s_k = tanh(s_{k-1} W_H + markov_w1[prev_k] + b_H), s_{-1} = 0
   * (the rnn head of the mlx-bun 0.2.0 -> 0.4.0 drafter, forwardRows; P1's
   * readConfig notes such heads ship markov_w1/w2 too).  Extra tensors:
   * "markov_head.rnn_wh.weight" [r, r] (weight dtype, applied as s @ W_H)
   * and "markov_head.rnn_bh.bias" [r] (act dtype).  Other non-vanilla heads
   * (the gated one, whose form the pages do not print) are refused. */
  int32_t markov_head_rnn;
} dspark_config;

/* One checkpoint tensor (deepspec.ts, DeepspecDrafter constructor keys, e.g.
 * "layers.0.self_attn.q_proj.weight", "markov_head.markov_w1.weight").
 * Matrices are [rows=out, cols=in] row-major and are read in that storage
 * order, never transposed or copied.  Vectors ([n]) use rows = n, cols = 1.
 * Q4: data = uint32 [rows, cols/8], code j of a word in bits 4j..4j+3;
 * scales, biases = bf16 [rows, cols/group]; value = scale * code + bias. */
typedef struct {
  const char* name;
  int32_t dtype;
  const void* data;
  const void* scales;
  const void* biases;
  int64_t rows;
  int64_t cols;
} dspark_weight;

typedef struct dspark_model dspark_model;

/* Validate the config and the weight table and build a model handle that
 * borrows the device pointers.  Missing, misshapen or mistyped tensors give
 * DSPARK_ERR_SHAPE; refused variants DSPARK_ERR_UNSUPPORTED. */
dspark_status dspark_model_create(const dspark_config* cfg, const dspark_weight* table, int n,
                                  dspark_model** out);
void dspark_model_destroy(dspark_model* m);

/* GEMMs over at least `rows` activation rows (a batch of draft rows, a long
 * context to project) run as a tiled bf16 MFMA GEMM over a product buffer in
 * the workspace, followed by the GEMM's epilogue (gate|up and lm_head form
 * theirs in the tiled kernel's store when one K slice holds the product);
 * fewer rows stream the weights once per 16-row tile.  Both compute the same product (fp32
 * activations as bf16 hi + lo planes); the context projection's k_proj
 * switches at 1024 rows or four times `rows`, whichever is more.  rows <= 0
 * keeps every GEMM on the weight-streaming kernel; a draft round's gate|up
 * switches at two thirds of `rows`.  Default 48 (draft rounds of three or
 * more blocks of 16; gate|up from two).  Workspace sizes depend on it: set it
 * before sizing workspaces.  DSPARK_ERR_INVALID_ARG for a null model. */
dspark_status dspark_model_set_tall_rows(dspark_model* m, int rows);

/* Per-model derived data the Markov walk uses to skip vocabulary entries that
 * cannot win a step (row norms of markov_w2 and the largest markov_w1 row
 * norm).  The caller allocates `aux_bytes` of device memory, calls prepare
 * once (asynchronously on `stream`), and keeps the buffer alive and unchanged
 * while the model is used. */
size_t dspark_model_aux_bytes(const dspark_model* m);
dspark_status dspark_model_prepare(dspark_model* m, void* aux_dev, size_t aux_bytes, hipStream_t stream);

/* Input of dspark_project_context_kv. */
typedef enum {
  DSPARK_INPUT_CONTEXT_HIDDEN = 0, /* x [B, L, H] (act dtype): already projected context rows */
  DSPARK_INPUT_TARGET_FEATURES = 1 /* x [B, L, fc_in] (act dtype): concatenated target taps;
                                      runs fc then hidden_norm first (deepspec.ts, #projectContext) */
} dspark_input_kind;

size_t dspark_project_workspace_bytes(const dspark_model* m, int input_kind, int B, int L);

/* deepspec.ts, #projectContextKVRows (and deepspec-module.ts,
 * projectContextKV): for every layer, k = k_proj(ctx); V = weightless
 * RMSNorm(k); K = RoPE(RMSNorm(k; k_norm)) at positions pos0[b] + i.
 *   x_dev        input per `input_kind`, row-major, act dtype
 *   pos0_host[B] first absolute position of each batch row (>= 0)
 *   k_out_dev[l], v_out_dev[l]  per layer, [B, nKv, L, hd] act dtype;
 *                k_out_dev may be NULL: a V-only cache (V is the weightless
 *                norm of the same k, so K = RoPE(V * k_norm) can be rebuilt
 *                where it is read; dspark_draft_rows_ex takes such a cache)
 * Workspace: dspark_project_workspace_bytes(m, input_kind, B, L) bytes,
 * 256-byte aligned, any contents (the call clears what it needs). */
dspark_status dspark_project_context_kv(const dspark_model* m, int input_kind, const void* x_dev, int B, int L,
                                        const int32_t* pos0_host, void* const* k_out_dev, void* const* v_out_dev,
                                        void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* Workspace for dspark_draft_rows with A rows (1..64) whose context lengths
 * sum to at most total_ctx and none exceeds max_ctx.  Only the attention
 * partials scale with the contexts: a round holds at most
 * min(512, ceil(total_ctx / 32)) + 2A key splits.  A workspace sized for
 * total_ctx serves every call whose contexts sum to at most total_ctx.
 * 0 for an invalid model, A, negative lengths or total_ctx > A * max_ctx. */
size_t dspark_draft_workspace_bytes(const dspark_model* m, int A, int max_ctx, int64_t total_ctx);

/* deepspec.ts, draftRows at temperature 0 with confidence truncation off
 * (every row keeps its full block):
 *   ids = [anchor_a, MASK x (gamma-1)] -> #forwardBackbone over each row's own
 *   context K/V ++ its block -> #computeLogits -> sequential Markov walk.
 *   k_ctx_dev[l*A + a], v_ctx_dev[l*A + a]  row a's layer-l context K/V,
 *       [nKv, ctx_len[a], hd] act dtype (rows stored independently; each
 *       row attends only its own context)
 *   ctx_len_host[A]    0 <= ctx_len[a] <= max_ctx of the workspace
 *   anchors_host[A]    0 <= anchor < V
 *   positions_host[A]  absolute position of each block's first slot (>= 0)
 *   tokens_dev[A*gamma] int32 output, row-major [A, gamma]
 *   logits_dev          NULL, or float [A, gamma, V] base logits (after
 *                       softcap, before the Markov bias)
 *   aux_dev             the buffer filled by dspark_model_prepare
 * A is at most 64. */
dspark_status dspark_draft_rows(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                const int32_t* anchors_host, const int32_t* positions_host, int32_t* tokens_dev,
                                float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                hipStream_t stream);

/* deepspec.ts, draftRows with the confidence head (its #confidence and the
 * _confident_prefix_length rule in the draftRows doc comment): after the walk,
 *   c[a, k] = sigmoid(proj . [x_k ; markov_w1[prev_k]] + bias),
 * x_k the final-normed hidden row of block slot k, prev_0 = anchor,
 * prev_k = token k - 1, and each row's proposal length is the first slot k
 * with c[a, k] < thr[k] (slots with thr[k] <= 0 are not tested), else gamma;
 * 0 is an empty proposal.  Other arguments as dspark_draft_rows (tokens_dev
 * always receives the whole block).
 *   thresholds_host  NULL: the config's confidence_threshold for every slot;
 *                    else gamma per-slot thresholds (the per-position form
 *                    of calibrated draft-length pruning)
 *   conf_dev         NULL, or float [A, gamma]: every slot's confidence
 *                    (requires the head: DSPARK_ERR_INVALID_ARG otherwise)
 *   lengths_dev      NULL, or int32 [A]: the proposal lengths (gamma for
 *                    every row when the model has no confidence head)
 * The workspace is dspark_draft_workspace_bytes's. */
dspark_status dspark_draft_rows_conf(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                     const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                     const int32_t* anchors_host, const int32_t* positions_host,
                                     const float* thresholds_host, int32_t* tokens_dev, float* logits_dev,
                                     float* conf_dev, int32_t* lengths_dev, const void* aux_dev, void* ws_dev,
                                     size_t ws_bytes, hipStream_t stream);

/* Every input and output of one draft round, for dspark_draft_rows_ex.
 * Fields as the arguments of the same names of dspark_draft_rows_conf, plus:
 *   k_ctx_dev      NULL: a V-only context cache (dspark_project_context_kv
 *                  with k_out_dev NULL).  The attention rebuilds each context
 *                  key as K = RoPE(V * k_norm) at position ctx_pos0[a] + j
 *                  (V is the weightless norm of the same k, so this is the
 *                  stored K up to the rounding of V): half the context bytes.
 *                  Built for bf16 caches (DSPARK_ERR_UNSUPPORTED otherwise,
 *                  and for head_dim 64).
 *   ctx_pos0_host  [A] absolute position of each row's first context row
 *                  (the pos0 the projection used), or NULL: 0.  Only read
 *                  for a V-only cache. */
typedef struct {
  int32_t A;
  const void* const* k_ctx_dev;   /* [layers * A] or NULL (V-only) */
  const void* const* v_ctx_dev;   /* [layers * A] */
  const int32_t* ctx_len_host;    /* [A] */
  const int32_t* ctx_pos0_host;   /* [A] or NULL */
  const int32_t* anchors_host;    /* [A] */
  const int32_t* positions_host;  /* [A] */
  const float* thresholds_host;   /* [gamma] or NULL */
  int32_t* tokens_dev;            /* [A, gamma] */
  float* logits_dev;              /* [A, gamma, V] or NULL */
  float* conf_dev;                /* [A, gamma] or NULL */
  int32_t* lengths_dev;           /* [A] or NULL */
  const void* aux_dev;
  /* Sampling (the mlx-bun 0.2.0 -> 0.4.0 drafter's temperature > 0 path with
   * per-row key streams): temperature <= 0 is the greedy walk.  Otherwise
   * step k of row a draws from softmax(u / temperature), u the step's scores
   * (base logits plus the head's bias), by the Gumbel-max rule
   * argmax_v (u_v + T g_v), g_v = -log(-log U_v), U_v from Philox4x64-10
   * (Salmon et al., SC 2011) with key (seeds_host[a], 0) and counter
   * (v / 4, k, 0, 0), word v mod 4, U = (top 23 bits + 1/2) / 2^23.
   * seeds_host NULL: seed 0 for every row.  logits_dev receives the base
   * logits, without the noise.  The confidence head, when asked for, scores
   * the sampled tokens. */
  float temperature;
  const uint64_t* seeds_host;     /* [A] or NULL */
} dspark_draft_args;
dspark_status dspark_draft_rows_ex(const dspark_model* m, const dspark_draft_args* args, void* ws_dev,
                                   size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dspark_draft_rows with its workspace taken from a fixed scratch array that
 * the library holds on each GPU (dspark_draft_noalloc_max_bytes() bytes,
 * 64 MiB, held from the library's load until the process ends).  Arguments
 * as for dspark_draft_rows; the caller still passes every input and output.
 * A round whose workspace (dspark_draft_workspace_bytes for these contexts;
 * less when logits_dev is given) exceeds the array fails with
 * DSPARK_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing: its first call on a GPU only looks up the array's device address
 * there.  Every call on one GPU shares that GPU's array and the array keeps
 * the last call's contents (the round clears what it needs itself), so
 * calls that overlap on one GPU (several streams or threads) race and must
 * not be issued. */
dspark_status dspark_draft_rows_noalloc(const dspark_model* m, int A, const void* const* k_ctx_dev,
                                        const void* const* v_ctx_dev, const int32_t* ctx_len_host,
                                        const int32_t* anchors_host, const int32_t* positions_host,
                                        int32_t* tokens_dev, float* logits_dev, const void* aux_dev,
                                        hipStream_t stream);
size_t dspark_draft_noalloc_max_bytes(void);

/* deepspec-module.ts, draftBlock: draftRows with one row. */
dspark_status dspark_draft_block(const dspark_model* m, const void* const* k_ctx_dev, const void* const* v_ctx_dev,
                                 int32_t ctx_len, int32_t anchor, int32_t position, int32_t* tokens_dev,
                                 float* logits_dev, const void* aux_dev, void* ws_dev, size_t ws_bytes,
                                 hipStream_t stream);

/* Optional per-kernel timing (benchmarks and diagnostics).  While enabled,
 * each kernel launch is bracketed by two HIP events recorded on the launch
 * stream (created with hipEventDisableSystemFence: they only time the work,
 * so their records neither write back nor invalidate the caches).  dspark_profile_read waits for those events, writes up to `max`
 * records (one per kernel role, e.g. "gemm.lm_head", "attn"), returns the
 * number written and clears the log.  Process-wide; not for concurrent use. */
typedef struct {
  const char* name;  /* static string owned by the library */
  int32_t launches;
  double ms;         /* summed event-to-event time */
} dspark_kernel_time;
void dspark_profile_enable(int on);
int dspark_profile_read(dspark_kernel_time* out, int max);

/* Diagnostic (host only, no HIP call): the output tile (column tile *bx,
 * row tile *by) that workgroup `w` of a gx x gy grid of the tiled GEMM
 * computes.  The tiled kernel renumbers its workgroups so that the tiles
 * dealt to one XCD share operands in that XCD's L2; the map is a bijection
 * of [0, gx*gy) onto the tiles.  DSPARK_ERR_INVALID_ARG for non-positive
 * sizes, w outside [0, gx*gy) or null outputs. */
dspark_status dspark_tall_tile_of(int gx, int gy, int w, int* bx, int* by);

/* Diagnostic (host only, no HIP call): the column block *bx, K slice *by and
 * row block *bz that workgroup (x, y, z) of the weight-streaming GEMM
 * computes, in a grid of gx column blocks, S K slices and R row blocks of 16
 * rows.  With several row blocks the kernel renumbers its workgroups so that
 * the row blocks of a (column block, K slice) run back to back on one XCD and
 * share its weight tile in that XCD's L2; a bijection of the (x, y, z)
 * triples.  DSPARK_ERR_INVALID_ARG for non-positive sizes, (x, y, z) outside
 * the grid or null outputs. */
dspark_status dspark_stream_block_of(int gx, int S, int R, int x, int y, int z, int* bx, int* by, int* bz);

/* Diagnostic (host only, no HIP call): replays on the host every address
 * that the 4-bit branches of the kernels form for a round of A rows with
 * these anchors and a context projection of ctx_rows rows of input_kind
 * (streaming GEMM weight words and scales for q|k, o, gate|up, down,
 * lm_head, fc and k_proj under the launch plans the library makes; the
 * GEMM's per-group activation sums in LDS; embedding, Markov, RNN and
 * confidence table elements), using the kernels' own index functions, and
 * checks each against the size of the buffer it reads ([rows, cols/8] words,
 * [rows, cols/group] scales and biases).  DSPARK_OK when every address is in
 * range (*n_checked = the number checked), DSPARK_ERR_SHAPE naming the first
 * one that is not, DSPARK_ERR_INVALID_ARG for a config that is not 4-bit or
 * arguments out of range.  The config is checked as dspark_model_create
 * checks it, except that 4-bit weights are not refused. */
dspark_status dspark_q4_address_check(const dspark_config* cfg, int A, const int32_t* anchors_host,
                                      int64_t ctx_rows, int input_kind, int64_t* n_checked);

/* Thread-local description of the last non-OK status ("" if none). */
const char* dspark_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */

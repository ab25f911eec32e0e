/*
 * ssb.h — C ABI of the MI355X self-speculative block-decoding round engine.
 *
 * The engine runs greedy self-speculative decoding of a shared
 * autoregressive / block-diffusion decoder on one gfx950 GPU. One decoder
 * and one LM head serve both modes; the only extra parameter is the [M]
 * (mask) embedding row (GravityOCR review, section 3.1 "AR-to-Diffusion
 * Conversion").
 *
 * A round (GravityOCR review, section 3.2 and Appendix B.2; velog review,
 * round description):
 *   - draft: [x0, [M] x B] at positions p..p+B. The boundary row is causal;
 *     the mask rows see the cache and the whole window. Gives a0, d1..dB.
 *   - verify: [a0, d1..dB] at positions p+1..p+B+1, causal. Overwrites the
 *     mask KV slots with causal state. Gives a1..a(B+1).
 *   - accept: A = longest prefix with d_j == a_j. Commits a0, d1..dA, a(A+1)
 *     (2..B+2 tokens) and rolls back to length p+A+2. a(A+1) becomes the
 *     next boundary.
 *
 * Conventions for every call:
 *   - Return 0 (SSB_OK) or a negative SSB_E* code. ssb_last_error() gives a
 *     thread-local message. No C++ exception crosses this boundary.
 *   - Pointers named *_dev are device pointers. Others are host pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls that return host results synchronize that stream first.
 *   - On error, committed state (sequence length, boundary token) is
 *     unchanged.
 *   - One model with its pools and KV caches is used from one host thread
 *     at a time; there is no internal locking.
 */
#ifndef SSB_H
#define SSB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSB_OK 0
#define SSB_EINVAL (-1)  /* bad argument or configuration */
#define SSB_ENOKV (-2)   /* KV capacity or pool pages exhausted */
#define SSB_EHIP (-3)    /* a HIP runtime call failed (message has the HIP error) */
#define SSB_ESTATE (-4)  /* call not valid in the current state (e.g. round before prefill) */
#define SSB_ENOMEM (-5)  /* device allocation at init failed */

#define SSB_F32 0
#define SSB_BF16 1

#define SSB_MAX_BATCH 64 /* requests per batched call */
#define SSB_MAX_BLOCK 64 /* largest block size B */

/* Decoder shape. Pre-norm Llama-style block: RMSNorm, RoPE (rotate-half
 * pairing), grouped-query attention, SwiGLU MLP, no biases, untied LM head.
 * Constraints:
 *   - hidden, n_heads*head_dim and ffn are multiples of 128. The reduction
 *     lengths hidden, n_heads*head_dim and ffn are 128 times a power of two;
 *     hidden <= 2048, n_heads*head_dim <= 4096 (bf16) / 2048 (f32), and
 *     ffn <= 8192 (bf16) / 4096 (f32).
 *   - head_dim is 32 or 64.
 *   - n_heads/n_kv_heads is 1 or 4.
 *   - page_tokens == 16.
 *   - block_B <= SSB_MAX_BLOCK. */
typedef struct ssb_config {
  int n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  int mask_id;        /* id of the [M] embedding row; never produced as output */
  int eos_id;         /* end of sequence; committed, then decoding stops */
  int block_B;        /* largest block size rounds will use */
  int page_tokens;    /* KV page size in tokens (16) */
  int max_rows;       /* rows per forward pass: prefill chunk, batched windows */
  int max_positions;  /* largest position + 1 any sequence reaches */
  float rms_eps, rope_theta;
  int dtype;          /* SSB_BF16: bf16 weights, fp16 activations and KV cache; SSB_F32: all f32 */
  int max_batch;      /* requests per batched call (rounds, AR steps, serving cap): 1..SSB_MAX_BATCH,
                         0 = SSB_MAX_BATCH; sizes the per-row workspace of decode forwards */
  int features;       /* SSB_FEAT_SAMPLE: workspace for stochastic rounds (two fp32 logit planes of
                         max_batch * (block_B + 1) rows); without it the sampling calls fail with
                         SSB_EINVAL */
} ssb_config;
#define SSB_FEAT_SAMPLE 1

/* Weights: device pointers, row-major [out_features][in_features] in the
 * config dtype (bf16 as raw uint16 bits); norm gains are float32 [hidden].
 * The per-layer arrays are host arrays of n_layers device pointers.
 * ssb_init_model copies the weights into its own layout, so the caller may
 * free them once it returns. */
typedef struct ssb_weights {
  const void* embed;              /* [vocab][hidden], row mask_id is the [M] embedding */
  const void* lm_head;            /* [vocab][hidden] */
  const float* final_norm;        /* [hidden] */
  const float* const* attn_norm;  /* [n_layers] -> [hidden] */
  const float* const* mlp_norm;   /* [n_layers] -> [hidden] */
  const void* const* wq;          /* [n_layers] -> [n_heads*head_dim][hidden] */
  const void* const* wk;          /* [n_layers] -> [n_kv_heads*head_dim][hidden] */
  const void* const* wv;          /* [n_layers] -> [n_kv_heads*head_dim][hidden] */
  const void* const* wo;          /* [n_layers] -> [hidden][n_heads*head_dim] */
  const void* const* wg;          /* [n_layers] -> [ffn][hidden] */
  const void* const* wu;          /* [n_layers] -> [ffn][hidden] */
  const void* const* wd;          /* [n_layers] -> [hidden][ffn] */
} ssb_weights;

typedef struct ssb_model ssb_model;
typedef struct ssb_pool ssb_pool;
typedef struct ssb_kv ssb_kv;

/* Per-decode statistics (ssb_decode / ssb_decode_ar / ssb_decode_dd).
 * Accept counts exclude a0 and a(A+1) (GravityOCR review, section 4.1).
 * Forwards count draft and verify passes, not prefill. Direct diffusion
 * counts only the forwards that commit tokens; its cache-write forwards are
 * counted apart (GravityOCR review, Appendix C, forward accounting). */
typedef struct ssb_stats {
  int rounds;            /* rounds run (AR: steps; direct diffusion: blocks) */
  int forwards;          /* decode forwards: 2 per round, 1 per AR step, denoising steps */
  int tokens;            /* output tokens, y1 from prefill included */
  int accepted;          /* sum of A over rounds */
  double decode_us;      /* wall time of the decode loop, prefill excluded */
  double prefill_us;     /* wall time of prefill */
  int cache_forwards;    /* direct diffusion: cache-write forwards */
} ssb_stats;

const char* ssb_last_error(void);

/* Validates a configuration without touching the GPU: 0 or SSB_EINVAL. */
int ssb_check_config(const ssb_config* cfg);

/* Builds a model on the current device. Packs the weights and allocates
 * the engine's fixed workspace; nothing on the round path allocates
 * afterwards. *out is owned by the caller; release it with ssb_free_model.
 * A bf16 model's packed copy holds the weights as fp16 (the matrix cores'
 * operand type for its fp16 activations; exact for magnitudes in
 * [2^-17, 65504]): SSB_EINVAL if a weight's magnitude exceeds 65504. */
int ssb_init_model(const ssb_config* cfg, const ssb_weights* w, void* stream, ssb_model** out);
void ssb_free_model(ssb_model* m);

/* Device bytes the model holds: its packed weights (and RoPE table) and its
 * fixed workspace (activations of max_rows rows, per-row attention records of
 * max_batch windows, LM-head group records, stochastic logit planes with
 * SSB_FEAT_SAMPLE). Either output may be null. SSB_EINVAL for a null model. */
int ssb_model_memory(const ssb_model* m, size_t* weight_bytes, size_t* workspace_bytes);

/* KV page pool, in caller-owned device memory. ssb_pool_bytes returns the
 * size of n_pages pages: each page holds page_tokens positions of K and V
 * for every layer and KV head. The layout is [layer][page][K|V][kv_head]
 * [token][head_dim]. */
int ssb_pool_bytes(const ssb_model* m, int n_pages, size_t* bytes);
int ssb_pool_init(ssb_model* m, void* dev_buf, size_t bytes, int n_pages, ssb_pool** out);
/* Frees the pool (not its caller-owned buffer) after the device is idle; the
 * model's captured launch graphs that use this pool are destroyed with it.
 * Free every kv of the pool first. */
void ssb_pool_free(ssb_pool* p);
int ssb_pool_free_pages(const ssb_pool* p, int* n_free);

/* One sequence's KV cache. Pages come from the pool on demand. After a
 * round, pages wholly past what the next window can reach go back to the
 * pool. ssb_kv_create allocates a small device page table.
 * ssb_kv_reset releases all pages: length 0, no boundary. */
int ssb_kv_create(ssb_pool* p, int max_tokens, ssb_kv** out);
void ssb_kv_free(ssb_kv* kv);
int ssb_kv_reset(ssb_kv* kv);
/* State query: committed length n (positions with KV), boundary token x0
 * (-1 before prefill) and pages held. */
int ssb_kv_state(const ssb_kv* kv, int* seq_len, int32_t* x0, int* pages_held);

/* Rewinds the kv to an earlier committed state: length n <= the current
 * length, boundary token x0 (the token committed at position n, which the
 * caller must supply). KV at positions < n is causal state of the committed
 * prefix and stays valid. Pages past the next window are returned to the
 * pool. Used to repeat a round from the same state. */
int ssb_kv_rewind(ssb_kv* kv, int n, int32_t x0);

/* Prefill (GravityOCR review, section 4.1 counts it outside TPF). Runs a
 * causal forward over P prefix embeddings (device [P][hidden], config
 * dtype) and writes KV for positions 0..P-1. *first_token (host) gets
 * y1 = argmax of row P-1, which becomes the boundary x0. The kv must be
 * empty. */
int ssb_prefill(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int32_t* first_token,
                void* stream);

/* One self-speculative round from the kv's state (length p, boundary x0).
 *   B: block size, 0..block_B.
 *   max_commit: output budget, >= 1. Tokens past it are not committed.
 *   planted_dev: nullable device [B] of token ids, -1 = keep the draft's own
 *     token. It replaces drafts before verification. Test/benchmark hook;
 *     it does not change the rule.
 *   committed (host, capacity B+2): the committed tokens, cut after the
 *     first EOS (inclusive) and at max_commit.
 *   *n_committed, *accept_len: count and A.
 * Afterwards the kv has length p+A+2 and boundary a(A+1).
 * draft_logits_dev / verify_logits_dev (nullable, device fp32
 * [B+1][vocab]) receive the scaled logits of the two forwards. */
int ssb_round(ssb_model* m, ssb_kv* kv, int B, int max_commit, const int32_t* planted_dev,
              int32_t* committed, int32_t* n_committed, int32_t* accept_len, float* draft_logits_dev,
              float* verify_logits_dev, void* stream);

/* ssb_round for callers that cannot allocate device memory: tight serving
 * loops and harnesses that forbid allocation. Same arguments and results as
 * ssb_round without the logits outputs (bit-identical committed tokens,
 * accept length and kv state), and it calls no hipMalloc, hipFree or other
 * allocating routine: the forward workspace of the window (B+1 rows, one
 * request) lives in a file-scope device array of 16 MiB that each GPU holds
 * until the process ends, and the launches run eagerly, since instantiating
 * a launch graph allocates. A window that would need more than 16 MiB (for
 * hidden 1024, 16 heads and vocab 60000: B = 32 up to about 6,900 cached
 * positions, B = 64 up to about 3,200) fails with SSB_EINVAL, state unchanged. The kv's
 * pages come from its pool without allocating. Calls on one GPU share the
 * array: overlapping calls on the same GPU race. Synchronous on stream, like
 * ssb_round. */
int ssb_round_noalloc(ssb_model* m, ssb_kv* kv, int B, int max_commit, const int32_t* planted_dev,
                      int32_t* committed, int32_t* n_committed, int32_t* accept_len, void* stream);

/* One AR step: feed x0 at position p causally. *token gets the argmax,
 * which becomes the new boundary. Length becomes p+1. logits_dev is
 * nullable, fp32 [vocab]. */
int ssb_ar_step(ssb_model* m, ssb_kv* kv, int32_t* token, float* logits_dev, void* stream);

/* Greedy self-speculative decode: prefill, then rounds until EOS or max_len
 * output tokens. out (host, capacity max_len) gets y1..yN, N <= max_len,
 * the first EOS included. The kv must be empty.
 * Optional planting (benchmark hook):
 *   - cont_dev (device [cont_len]) is the AR greedy continuation y1...
 *   - astar (host [n_astar]) gives the planted accept length per round.
 *   - Round k plants d_j = y_{c+1+j} for j <= astar[k], and a token other
 *     than y_{c+astar+2} at j = astar+1 (c = tokens output so far).
 *   - Rounds past n_astar are not planted. */
int ssb_decode(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, int max_len,
               const int32_t* cont_dev, int cont_len, const int32_t* astar, int n_astar, int32_t* out,
               int32_t* n_out, ssb_stats* stats, void* stream);

/* Greedy AR decode with the same kernels (window of one row). */
int ssb_decode_ar(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int max_len, int32_t* out,
                  int32_t* n_out, ssb_stats* stats, void* stream);

/* R <= SSB_MAX_BATCH concurrent requests, one launch per stage. Each
 * request has its own kv, state, budget and page table. Every kv needs a
 * boundary token (prefilled). planted_dev: nullable device [R][B].
 * committed: host [R][B+2]. n_committed, accept_len: host [R].
 * draft_logits_dev, verify_logits_dev: nullable, fp32 [R*(B+1)][vocab],
 * request r's window rows at r*(B+1) .. r*(B+1)+B (the round then runs
 * without graph replay). A request's results, logits included, are bit-identical
 * to those of its own single round. */
int ssb_round_batch(ssb_model* m, ssb_kv* const* kvs, int R, int B, const int32_t* max_commit,
                    const int32_t* planted_dev, int32_t* committed, int32_t* n_committed,
                    int32_t* accept_len, float* draft_logits_dev, float* verify_logits_dev, void* stream);

/* Stochastic self-speculative round (GravityOCR review, section 2
 * "Speculative Decoding"; Trillion Labs blog, the speculative rejection rule
 * that preserves the sampling distribution; the rule itself is the standard
 * one of Leviathan et al. and Chen et al., 2023). Every distribution is
 * softmax(logits / temperature) over the vocabulary without [M]; a draw with
 * a uniform u takes the smallest token id whose cumulative mass exceeds u
 * times the total.
 *   - draft as in ssb_round; a0 and d1..dB are drawn from draft rows 0..B;
 *   - verify over [a0, d1..dB]; d_j is accepted while
 *     u_acc[j] * q_j(d_j) < p_j(d_j) (q_j: draft row j, p_j: verify row j-1);
 *     A = number accepted before the first rejection;
 *   - the next token t is drawn from max(0, p_{A+1} - q_{A+1}) (from p_{A+1}
 *     if that has no mass) when A < B, from p_{B+1} when A = B;
 *   - commits a0, d1..dA, t (cut after EOS and at max_commit); t becomes the
 *     boundary; rollback as in ssb_round.
 * u_dev: device float [2B+2], values in [0, 1): u_a0, u_d[1..B], u_acc[1..B],
 * u_t. temperature > 0. Other arguments as ssb_round (no planting). */
int ssb_round_sample(ssb_model* m, ssb_kv* kv, int B, int max_commit, float temperature, const float* u_dev,
                     int32_t* committed, int32_t* n_committed, int32_t* accept_len, float* draft_logits_dev,
                     float* verify_logits_dev, void* stream);

/* Prefill with y1 drawn from the last prefix row, then stochastic rounds
 * until EOS or max_len tokens. u_dev: device float [n_u_rows][2B+2]; row 0's
 * first value draws y1, row k drives round k (SSB_EINVAL if the rows run
 * out). */
int ssb_decode_sample(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, float temperature,
                      int max_len, const float* u_dev, int n_u_rows, int32_t* out, int32_t* n_out, ssb_stats* stats,
                      void* stream);

/* AR sampling with the same kernels: y1 from the last prefix row with
 * u_dev[0], token k (k >= 1) from an AR step with u_dev[k]. u_dev: device
 * float [max_len]. The output follows the same distribution as
 * ssb_decode_sample's, not the same tokens. */
int ssb_decode_ar_sample(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, float temperature, int max_len,
                         const float* u_dev, int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream);

/* Greedy self-speculative round with a multi-step draft schedule (Trillion
 * Labs blog, the draft-schedule passage; GravityOCR review, Appendix D
 * "Draft Schedule"). The draft window [x0, s_1..s_B] is refined by up to
 * `steps` draft-mode forwards: slot i (position p+i) holds the prediction of
 * window row i-1 (a0 for i = 1, d_{i-1} otherwise); each step commits the
 * open slots whose confidence is >= tau (the single most confident if none),
 * the last allowed step commits every open slot. d_B is window row B's
 * prediction in the last draft forward. Verify, accept and rollback are those
 * of ssb_round on [a0, d1..dB]; steps = 1 is exactly ssb_round's one-shot
 * draft, and the output is AR-identical for every schedule.
 * draft_forwards (host, nullable): draft forwards run (<= steps).
 * verify_logits_dev: nullable device fp32 [B+1][vocab]. B >= 1. */
int ssb_round_multistep(ssb_model* m, ssb_kv* kv, int B, int steps, float tau, int max_commit, int32_t* committed,
                        int32_t* n_committed, int32_t* accept_len, int32_t* draft_forwards, float* verify_logits_dev,
                        void* stream);

/* Prefill, then multi-step-draft rounds until EOS or max_len tokens.
 * stats.forwards counts draft and verify forwards. */
int ssb_decode_multistep(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, int steps, float tau,
                         int max_len, int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream);

/* Direct block-diffusion decoding of one block (GravityOCR review, section 2
 * "Block Diffusion" and Appendix B.1; Trillion Labs blog, "confidence
 * threshold" entry). The block is the B positions p+1..p+B after the
 * boundary x0 at p, all [M] at first. Each denoising step is one draft-mode
 * forward over [x0, s_1..s_B] (s_j: committed token or [M]); position j
 * takes the greedy token of window row j-1 (shift-by-one), its confidence
 * is that token's softmax probability over the vocabulary without [M].
 * Every undecided position with confidence >= tau is committed; if none,
 * the single most confident one (lowest position on ties). At most B steps.
 *   write_cache: 1 = run the cache-write forward (causal over s_1..s_{B-1}
 *     at p+1..p+B-1; it verifies nothing) and advance the kv to length p+B
 *     with boundary s_B; 0 = leave the kv's state at (p, x0).
 *   tokens: host [B], the block. n_tokens: tokens that belong to the output
 *     after the cut at the first EOS (inclusive) and at max_commit.
 *   steps: denoising forwards run. step_of: host [B], nullable: the step
 *     (0-based) that committed each position.
 *   step_conf / step_tok: host [B][B], nullable: per step, the confidence and
 *     greedy token of window rows 0..B-1 (rows of committed positions too).
 *   step_logits_dev: nullable device fp32 [B][B+1][vocab]: each step's logits.
 * Errors: SSB_ESTATE without a boundary token; SSB_EINVAL for B outside
 * [1, block_B], tau NaN or max_commit < 1; SSB_ENOKV past max_positions;
 * SSB_EHIP for NaN logits (the kv's state is then unchanged). */
int ssb_dd_block(ssb_model* m, ssb_kv* kv, int B, float tau, int max_commit, int write_cache, int32_t* tokens,
                 int32_t* n_tokens, int32_t* steps, int32_t* step_of, float* step_conf, int32_t* step_tok,
                 float* step_logits_dev, void* stream);

/* Prefill, then direct block-diffusion blocks until EOS or max_len output
 * tokens (y1 included). The block that ends the output (EOS inside, or the
 * budget reached) runs no cache-write forward. stats: rounds = blocks,
 * forwards = denoising forwards, cache_forwards = cache-write forwards. */
int ssb_decode_dd(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, float tau, int max_len,
                  int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream);

/* One greedy AR step for R <= SSB_MAX_BATCH requests (distinct prefilled
 * kvs of one pool), one launch per stage: request r feeds its boundary token
 * and gets the next one in tokens (host [R]). */
int ssb_ar_step_batch(ssb_model* m, ssb_kv* const* kvs, int R, int32_t* tokens, void* stream);

/* Continuous batching over a request queue (GravityOCR review, section 4.3,
 * Figure 6 "Throughput Scaling with Batch Size", and Appendix C: a full
 * client queue served under a cap on running requests). All n_reqs requests
 * are queued at the start, in array order. At most max_running run at once;
 * a free slot admits the next queued request, whose prefill runs between
 * decode launches. Each decode launch advances every running request by one
 * greedy AR step (mode SSB_SERVE_AR) or one self-speculative round of block
 * B (mode SSB_SERVE_SPEC). A request leaves at EOS or after max_len tokens.
 * The engine creates max_running kvs of max_tokens positions in `pool` and
 * frees them before returning; the pool needs the pages for them.
 * Per request (in): prefix_dev (device [P][hidden]), P, max_len, out (host
 * [max_len]); optional planting as in ssb_decode (cont_dev, cont_len, astar,
 * n_astar; SPEC mode only). Per request (out): n_out, rounds (decode
 * launches it took part in), finish_us (completion time from the call's
 * start). */
#define SSB_SERVE_AR 0
#define SSB_SERVE_SPEC 1
typedef struct ssb_request {
  const void* prefix_dev;
  int P, max_len;
  const int32_t* cont_dev;
  int cont_len;
  const int32_t* astar;
  int n_astar;
  int32_t* out;
  int n_out, rounds;
  double finish_us;
} ssb_request;
typedef struct ssb_serve_stats {
  int steps;             /* decode launches */
  int prefills;
  long long tokens;      /* output tokens of all requests, y1 included */
  double total_us, prefill_us, decode_us;
  double mean_running;   /* running requests per decode launch, averaged */
} ssb_serve_stats;
int ssb_serve(ssb_model* m, ssb_pool* pool, ssb_request* reqs, int n_reqs, int max_running, int mode, int B,
              int max_tokens, ssb_serve_stats* stats, void* stream);

/* Teacher-forced causal forward over tokens (host [M], M <= max_rows) at
 * positions p..p+M-1 of the kv. Writes their KV but does not change the
 * kv's committed length. logits_dev: nullable device fp32 [M][vocab].
 * argmax (host [M]) gets the greedy token of every row. top1/top2 (host
 * [M], nullable) get the two largest logits. Used to judge decoded
 * sequences position by position. */
int ssb_forward_tokens(ssb_model* m, ssb_kv* kv, const int32_t* tokens, int M, int p, float* logits_dev,
                       int32_t* argmax, float* top1, float* top2, void* stream);

/* Kernel timing hook for measurement. While a kind is selected, every
 * launch of that kernel kind is issued with hipExtLaunchKernel and a start /
 * stop event pair that the runtime attaches to the dispatch itself, on the
 * stream it is launched on. Rounds and AR steps then run without graph
 * replay. With SSB_PROFILE_IN_GRAPH or'ed into kind, greedy and stochastic
 * rounds (single and batched) and AR steps keep replaying launch graphs
 * instead: in a separate graph per timed kind every launch records the
 * latest end of its workgroups on the device's real-time counter, and a
 * launch of the timed kind counts from the end of the launch before it to
 * its own end (back-to-back graph launches start when the previous one
 * completes, so this is the interval a kernel trace reports for the
 * dispatch); the other calls run eagerly as above.
 * ssb_profile_read returns the summed time and the launch
 * count since the last reset; reset != 0 clears them.
 * kind: one of SSB_K_*, or -1 to stop timing. SSB_K_DOWN is the down
 * projection GEMM; SSB_K_REDUCE its K-split reduce (absent when the down
 * projection is not split); SSB_K_TAIL the fused layer tail that replaces
 * the O, gate|up and down launches of decode windows of at most 48 rows. */
#define SSB_K_QKV 0
#define SSB_K_ATTN 1
#define SSB_K_COMBINE 2
#define SSB_K_O 3
#define SSB_K_GATEUP 4
#define SSB_K_DOWN 5
#define SSB_K_LMHEAD 6
#define SSB_K_ARGMAX 7
#define SSB_K_REDUCE 8
#define SSB_K_TAIL 9   /* the fused layer tail: O, gate|up and down of a decode window of <= 48 rows */
#define SSB_PROFILE_IN_GRAPH 0x100
int ssb_profile_kernel(ssb_model* m, int kind);
int ssb_profile_read(ssb_model* m, double* total_us, long long* launches, int reset);

/* Debug check of the in-place KV overwrite and of rollback (GravityOCR
 * review, Appendix B.2: verify overwrites the draft's window slots, and only
 * causal state survives a round). With SSB_DEBUG_POISON set, every greedy or
 * stochastic round (single, batched, inside decode and serve) writes NaN into
 * every layer's K and V at positions p+1 .. p+B+1 of each request between its
 * draft and verify forwards, and at p+A+2 .. p+B+1 after accept. A correct
 * engine reads none of them before rewriting them, so results are unchanged
 * bit for bit; a stale read surfaces as NaN logits (SSB_EHIP from the round).
 * Rounds then run without graph replay.
 * With SSB_DEBUG_UNFUSED set, decode windows of at most 48 rows run each
 * layer's O, gate|up and down projections as three GEMM launches instead of
 * the fused layer tail (the same per-row arithmetic, so results are bit-
 * identical: a test and measurement switch). Changing it drops the captured
 * launch graphs. flags: any or of SSB_DEBUG_POISON and SSB_DEBUG_UNFUSED;
 * SSB_EINVAL for other bits or a null model. */
#define SSB_DEBUG_POISON 1
#define SSB_DEBUG_UNFUSED 2
int ssb_set_debug(ssb_model* m, int flags);

/* Debug: writes NaN into every layer's K and V at positions [lo, hi) of the
 * kv's pages (a test hook for the poisoning above: poisoning a slot the next
 * round reads makes that round fail with SSB_EHIP; poisoning slots the next
 * window rewrites first changes nothing). SSB_EINVAL if the range is outside
 * the pages the kv holds. Synchronous on stream. */
int ssb_kv_poison(ssb_kv* kv, int lo, int hi, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSB_H */

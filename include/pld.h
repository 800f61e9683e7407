/*
 * pld.h — C ABI of the persistent batch-1 decode library (libpld.so, MI355X / gfx950).
 *
 * One decode step of one MoE transformer layer runs as ONE launch of a persistent
 * cooperative kernel: every workgroup stays resident, and the stages (RMSNorm,
 * projections, attention, output projection + residual, router top-k, experts) are
 * chained by device-side data dependencies (epoch-tagged activation words that the
 * consumers poll) instead of kernel boundaries. This is the
 * "persistent Engine Kernel" of the TileRT article (InferenceX, "Ultra-High
 * Interactivity on NVIDIA GPUs? TileRT on InferenceX", section "But What Exactly is
 * TileRT?": the host launches once and execution stays on the GPU; stages overlap at
 * tile granularity; intermediates move through on-chip memory and L2), rebuilt for
 * gfx950 with HIP. The calls follow that article's decode problem: batch 1, one
 * in-flight request per decode engine, a KV cache prefilled elsewhere and handed over
 * (section "PD Disaggregated Engine with vLLM and TileRT"); input preparation,
 * sampling policy and KV-cache management stay with the caller, as in the vLLM Kimi K3
 * backend article ("A narrow deployment lane"), which also routes unsupported
 * configurations elsewhere — here they are rejected with PLD_E_UNSUPPORTED.
 *
 * Conventions for every call:
 *  - All tensors are caller-owned DEVICE memory (e.g. allocated by torch). The library
 *    keeps non-owning pointers; it never allocates, frees or reallocates device memory.
 *  - Pointers must be 16-byte aligned; reduction dimensions must be multiples of the
 *    16-byte load width (8 bf16 or 16 FP8 elements).
 *  - Linear weights are row-major [out, in] ("rows" are outputs). bf16 weights are raw
 *    bf16 bit patterns. FP8 weights are OCP E4M3FN bytes with one fp32 scale per
 *    128x128 block: scales[ceil(out/128)][ceil(in/128)], W[n,k] = dec(Q[n,k]) *
 *    scales[n/128][k/128] (edge blocks have their own scale).
 *  - Expert weights are stacked per slot: w_gate/w_up [n_experts+n_shared][inter][hidden],
 *    w_down [n_experts+n_shared][hidden][inter]; shared experts come after the routed
 *    ones. FP8 expert scales are stacked the same way.
 *  - Norm gains and router bias are fp32.
 *  - Errors: every call returns a pld_status. Argument errors are returned
 *    synchronously before anything is enqueued. Device-side failures (the watchdog of a
 *    bounded wait) are reported by decode_poll_status after the stream has completed,
 *    and leave the handle in PLD_E_STATE until decode_reset. No C++ exception crosses
 *    the ABI.
 *  - Threading: one handle = one sequence, used from one host thread and one stream at
 *    a time. Launches on one handle must be stream-ordered.
 */
#ifndef PLD_H
#define PLD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLD_ABI_VERSION 1

typedef enum pld_status {
  PLD_OK = 0,
  PLD_E_INVALID = -1,        /* null or misaligned pointer, bad size, bad index */
  PLD_E_UNSUPPORTED = -2,    /* configuration outside the supported set (no fallback) */
  PLD_E_CAPACITY = -3,       /* pos + n_query > max_seq, or workspace too small */
  PLD_E_HIP = -4,            /* a HIP runtime call failed */
  PLD_E_DEVICE_TIMEOUT = -5, /* a device wait passed its deadline; see pld_device_status */
  PLD_E_STATE = -6           /* handle needs decode_reset after a device failure */
} pld_status;

enum { PLD_ATTN_GQA = 0, PLD_ATTN_MLA = 1, PLD_ATTN_KDA = 2 };
enum { PLD_WFMT_BF16 = 0, PLD_WFMT_FP8_BLOCK128 = 1, PLD_WFMT_LUT3 = 2 };
enum { PLD_FFN_DENSE = 0, PLD_FFN_MOE = 1 };
enum { PLD_ROUTER_SOFTMAX_TOPK = 0, PLD_ROUTER_SIGMOID_BIAS = 1 };

/* Layer shape. GQA fields are used when attn_kind == PLD_ATTN_GQA (MHA is
 * n_kv_heads == n_heads); MLA fields when attn_kind == PLD_ATTN_MLA; index_* when
 * index_topk > 0 (MLA only; index_topk at most 8192, larger is PLD_E_UNSUPPORTED).
 * KDA (attn_kind == PLD_ATTN_KDA, the linear attention of the Kimi K3 article, section
 * "FlashKDA Algorithm"): n_heads heads of head_dim key and value channels, a decay
 * projection of rank kda_rank and a causal depthwise convolution of conv_width taps over
 * the q, k and v projections (the compiled layout: head_dim 128, kda_rank 128,
 * conv_width 4, FP8 weights). */
typedef struct pld_config {
  int32_t attn_kind;
  int32_t wfmt;
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads, head_dim;                          /* GQA */
  int32_t q_lora, kv_lora, rope_dim, nope_dim, v_dim;    /* MLA */
  int32_t index_heads, index_dim, index_topk;            /* sparse indexer */
  int32_t ffn_kind;
  int32_t inter;                                         /* dense width or per-expert width */
  int32_t n_experts, top_k, n_shared;
  int32_t router_kind;
  int32_t max_seq;                                       /* cache capacity in rows */
  double eps;                                            /* RMSNorm epsilon */
  double rope_base;                                      /* RoPE base (interleaved pairs) */
  int32_t vocab;                                         /* LM head rows; 0 = no head */
  int32_t kda_rank, conv_width;                          /* KDA */
  int32_t expert_wfmt;       /* 0: experts in wfmt; PLD_WFMT_LUT3: the routed and shared expert matrices
                                (w_gate, w_up, w_down) hold 3-bit indices into one 8-entry E4M3 codebook
                                per 8x64 block, 3.125 bits per weight (the Vera Rubin article, "Lookup
                                Table Weight Decompression in Rubin SM107 Tensor Core"); FP8 layers only.
                                Layout of an [out, in] matrix: data = per row and group of 128 weights 48
                                bytes (plane p = bytes 16p..16p+15 as four little-endian u32, bit j of
                                word d = bit p of the index of weight 32d+j of the group), 3*in/8 bytes
                                per row; scales = the codebook bytes [out/8][in/64][8] (entry e of a
                                block = byte e), cast to const float*. */
  int32_t max_query;         /* 0 or 1: no batched verify; 2..8: the workspace also holds the buffers of
                                decode_verify_batched for up to max_query positions (FP8 MLA MoE layers
                                with an LM head only, else PLD_E_UNSUPPORTED) */
  int32_t max_batch;         /* 0 or 1: one sequence per handle; 2..8: decode_batch runs up to max_batch
                                sequences, and every layer's latent cache holds max_batch sequences of
                                max_seq rows back to back (sequence b's row r at row b * max_seq + r;
                                the single-sequence calls use sequence 0). Same shapes as max_query. */
} pld_config;

typedef struct pld_matrix {
  const void* data;    /* bf16 bits or E4M3FN bytes, [out, in] row-major */
  const float* scales; /* FP8 only: [ceil(out/128)][ceil(in/128)]; NULL for bf16 */
} pld_matrix;

typedef struct pld_layer_weights {
  const float* attn_norm;   /* [hidden] */
  const float* ffn_norm;    /* [hidden] */
  const float* q_norm;      /* MLA: [q_lora] */
  const float* kv_norm;     /* MLA: [kv_lora] */
  pld_matrix wq, wk, wv;    /* GQA: [n_heads*hd, H], [n_kv*hd, H], [n_kv*hd, H] */
  pld_matrix w_dq;          /* MLA: [q_lora, H] */
  pld_matrix w_uq;          /* MLA: [n_heads*(nope+rope), q_lora]; per head nope rows then rope rows */
  pld_matrix w_dkv;         /* MLA: [kv_lora+rope, H]; latent rows then rope rows */
  pld_matrix w_uk;          /* MLA: [n_heads*nope, kv_lora] */
  pld_matrix w_uv;          /* MLA: [n_heads*v_dim, kv_lora] */
  pld_matrix w_qi;          /* indexer: [index_heads*index_dim, q_lora] */
  pld_matrix w_w;           /* indexer head weights: [index_heads, H], always bf16 */
  pld_matrix w_ki;          /* indexer key: [index_dim, H] */
  pld_matrix wo;            /* [H, n_heads*hd] (GQA, KDA) or [H, n_heads*v_dim] (MLA) */
  const void* router;       /* MoE: bf16 [n_experts, H] */
  const float* router_bias; /* sigmoid router: [n_experts] */
  pld_matrix w_gate, w_up;  /* [slots][inter][H] (dense FFN: slots = 1) */
  pld_matrix w_down;        /* [slots][H][inter] */
  /* KDA (q = n_heads*head_dim): wq, wk, wv above are its [q, H] projections, and */
  pld_matrix w_g;           /* output gate [q, H] */
  pld_matrix w_beta;        /* delta-rule strength [n_heads, H] */
  pld_matrix w_adown;       /* decay, low rank [kda_rank, H] */
  pld_matrix w_aup;         /* decay [q, kda_rank] */
  const float* conv_taps;   /* fp32 [3*q][conv_width]: channels q, k, v; the last tap on the current position */
  const float* o_norm;      /* fp32 [head_dim] gain of the per-head output RMSNorm */
} pld_layer_weights;

/* KV cache of one layer (caller-owned, device). Rows 0..pos-1 must hold the prefilled
 * history; decode writes row pos. A KDA layer's "cache" is its state and convolution ring
 * instead: every step reads and rewrites them in place. */
typedef struct pld_kv_cache {
  void* k;              /* GQA: bf16 [n_kv_heads][max_seq][head_dim] */
  void* v;              /* GQA: bf16 [n_kv_heads][max_seq][head_dim] */
  void* latent;         /* MLA: bf16 [max_seq][kv_lora + rope_dim] (c_kv then k_rope) */
  void* index_codes;    /* indexer: E4M3FN [max_seq][index_dim] */
  float* index_scales;  /* indexer: fp32 [max_seq] */
  float* kda_state;     /* KDA: fp32 [n_heads][head_dim (key)][head_dim (value)], advanced in place */
  float* conv_ring;     /* KDA: fp32 [conv_width-1][3*q] projection outputs of the previous positions,
                           slot = position mod (conv_width-1); the current one replaces slot pos mod 3 */
} pld_kv_cache;

/* LM head of a layer stack (only with vocab > 0). */
typedef struct pld_head_weights {
  const void* embed;        /* bf16 [vocab][hidden] */
  const float* final_norm;  /* [hidden] */
  pld_matrix head;          /* [vocab, hidden], FP8 block-scaled or bf16 (same wfmt as the layers) */
} pld_head_weights;

/* Device status read back by decode_poll_status. code 0 = ok. */
typedef struct pld_device_status {
  int32_t code;       /* 0 ok, PLD_E_DEVICE_TIMEOUT when a wait expired */
  int32_t stage;      /* what the expired wait was for: 0 layer input x, 1 q, 2 new k/v row,
                         3 attention partials, 4 attention output o, 5 h2, 6 router logits,
                         7 expert activations m */
  int32_t layer;      /* layer index (within the launch's stack) */
  int32_t token;      /* token index within the launch */
  int32_t wg;         /* workgroup that detected it */
  int32_t reserved[3];
} pld_device_status;

typedef struct pld_persistent_args {
  int32_t start_pos;          /* cache position of the first token */
  int32_t n_tokens;           /* tokens to decode in this launch (greedy loop when a head is present);
                                 must be 1 when n_query > 1 */
  int32_t n_query;            /* 1; >1 = verify n_query positions in one launch (head required) */
  int32_t in_token;           /* >= 0: first input is embed[in_token]; < 0: use in_hidden
                                 (verify: the last accepted token, required) */
  const void* in_hidden;      /* bf16 [hidden] first input when in_token < 0 */
  const int32_t* draft_tokens;/* verify: device int32 [n_query-1], 4-byte aligned; draft j feeds
                                 position start_pos + j + 1. Ids outside [0, vocab) are never
                                 accepted (their embedding row is read at the clamped id). */
  void* out_hidden;           /* bf16 [hidden]: output of the last layer for the last position */
  float* out_logits;          /* fp32 [n_tokens or n_query][vocab], or NULL */
  int32_t* out_tokens;        /* int32 [n_tokens or n_query] greedy tokens, or NULL */
  int32_t* out_accepted;      /* verify: int32 [1] accepted draft count, or NULL */
  double temperature;         /* 0: greedy argmax; > 0: each token is sampled from softmax(logits / T)
                                 (LM head required; finite, >= 0, else PLD_E_INVALID) */
  uint64_t sample_seed;       /* seed of the sampling noise (see decode_layers_persistent) */
} pld_persistent_args;

typedef struct pld_handle pld_handle;

/* Bytes of device workspace decode_layer_init needs for this shape and stack depth
 * (status, handoff buffers, attention partials, RoPE table, layer descriptors).
 * Returns 0 for an invalid or unsupported configuration. */
size_t pld_workspace_bytes(const pld_config* cfg, int32_t n_layers);

/* The same size for a device with n_cus compute units (one workgroup per CU), without
 * querying any device: for planning allocations off the GPU. */
size_t pld_workspace_bytes_for_cus(const pld_config* cfg, int32_t n_layers, int32_t n_cus);

/* Validate the configuration and pointers, build the static per-workgroup schedule
 * (the ahead-of-time scheduling of the TileRT article, section "Why Is TileRT
 * Development Slow?", done here at init), upload the RoPE table and layer
 * descriptors into `workspace`, zero the handoff buffers, and check that the persistent grid
 * can be co-resident. Synchronous. Nothing is allocated on the device.
 *   cfg:       layer shape (copied)
 *   n_layers:  number of layers in `w` and `kv` (>= 1)
 *   w, kv:     host arrays of n_layers descriptors of device pointers (copied)
 *   head:      NULL, or LM head weights when cfg->vocab > 0
 *   workspace: device buffer of at least pld_workspace_bytes(cfg, n_layers) bytes,
 *              owned by the caller, used exclusively by this handle until destroy
 *   out:       receives the handle (host memory owned by the library)
 * Errors: PLD_E_INVALID, PLD_E_UNSUPPORTED, PLD_E_CAPACITY, PLD_E_HIP. */
pld_status decode_layer_init(const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                             const pld_kv_cache* kv, const pld_head_weights* head, void* workspace,
                             size_t ws_bytes, pld_handle** out);

/* decode_layer_init for callers that cannot allocate device memory (code that later runs
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same validation and set-up, but the workspace is the library's own static device array
 * of 32 MiB per GPU (held from the first use on a GPU until the process ends), so no
 * workspace argument is taken, and nothing is allocated on the device or the host.
 *   Returns PLD_E_CAPACITY when pld_workspace_bytes(cfg, n_layers) exceeds 32 MiB (every
 *   single-layer workload of this library fits; so does a 24-layer stack of the FP8 MLA
 *   layer), else the errors of decode_layer_init.
 *   The handle is library storage, one per GPU: every call on a GPU returns the same
 *   handle and re-initialises it (and that GPU's array; the status and handoff buffers are
 *   cleared, the step epoch keeps counting), so an earlier handle of the same GPU now runs
 *   the new configuration. Launches of that handle that overlap with a re-initialisation
 *   or with each other race. decode_layer_destroy on it does nothing. Synchronous; it is
 *   not itself capturable, but the launches on the handle are plain kernel launches.
 *   cfg, n_layers, w, kv, head: as for decode_layer_init; out receives the handle. */
pld_status decode_layer_init_static(const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                                    const pld_kv_cache* kv, const pld_head_weights* head, pld_handle** out);

/* Decode one token through layer `layer` in one launch: RMSNorm -> projections ->
 * RoPE + cache append at row `pos` -> attention over rows 0..pos -> output projection +
 * residual -> RMSNorm -> router top-k -> routed + shared SwiGLU experts -> residual.
 * x_in, x_out: device bf16 [hidden] (may alias). Asynchronous on `stream`.
 * Errors: PLD_E_INVALID (bad layer/pointers), PLD_E_CAPACITY (pos >= max_seq),
 * PLD_E_STATE, PLD_E_HIP. */
pld_status decode_step(pld_handle* h, int32_t layer, const void* x_in, int32_t pos, void* x_out,
                       void* stream);

/* One launch for a whole decode run: for each of a->n_tokens tokens (or the n_query
 * verify positions), every layer of the stack in order, then (with a head) final
 * RMSNorm -> LM head -> token choice -> embedding of the chosen token as the next input.
 * Asynchronous on `stream`.
 * Token choice: temperature 0 takes the greedy argmax (lowest id on ties). temperature T > 0
 * samples softmax(logits / T) by the Gumbel-max rule: token = argmax_i (logit_i / T - log(-log
 * u_i)) in fp64, ties to the lower id, with u_i in (0, 1) from a counter-based SplitMix64
 * stream keyed by (sample_seed, the step's cache position, i): with G = 0x9E3779B97F4A7C15
 * and mix the splitmix64 output mixer, k = mix(seed * G + pos), r = mix(k + (i + 1) * G),
 * u = (2 (r >> 12) + 1) 2^-53. A token thus depends only on its position's logits and the
 * seed; temperature sampling is a serving setting of the vLLM Kimi K3 backend article ("A
 * narrow deployment lane"), which leaves the sampling policy to the caller.
 * Verify (n_query > 1): positions start_pos .. start_pos + n_query - 1 are fed in_token,
 * then the drafts; every position's logits and chosen token are written; out_accepted[0] =
 * the number of leading drafts equal to the token chosen at the position before them
 * (the speculative decoding with a draft of six tokens in the vLLM Kimi K3 backend article;
 * with T > 0 this is the speculative-sampling rule for a deterministic drafter: a draft is
 * kept with probability p(draft), and on rejection the position's sample follows p without
 * the draft, renormalised). Rows of all n_query positions are appended; the caller
 * continues at start_pos + out_accepted[0] + 1 and later launches overwrite the rest.
 * The positions run as sequential steps inside the launch (the plain definition of a
 * causal multi-token verify).
 * Errors: PLD_E_INVALID, PLD_E_UNSUPPORTED (verify without head), PLD_E_CAPACITY,
 * PLD_E_STATE, PLD_E_HIP. */
pld_status decode_layers_persistent(pld_handle* h, const pld_persistent_args* a, void* stream);

/* The same verify with the positions batched: the n_query positions (2 .. cfg->max_query,
 * at most 8) go through every layer together, so each weight matrix is read from HBM once
 * per verify instead of once per position. The vLLM Kimi K3 backend article scores a draft
 * of six tokens in one forward pass (its summary and "Throughput holds across the tested
 * range") and lists shape-aware matmuls among its changes ("Four changes drive the gains").
 * Here the dense projections (W_DQ, W_DKV, W_UQ, W_UV, W_O, the shared experts) and the
 * union of the experts the positions route to run on the matrix cores as skinny GEMMs
 * [rows x K] x [K x n_query]: the FP8 weights are widened to bf16 in registers (exactly),
 * the normalised activations enter as bf16, accumulation is fp32; an expert chosen by
 * several positions is read once for all of them. The router logits stay fp64 from fp32
 * activations and the head stays the fp64 one, so the expert choice and the token choice
 * are decided as in decode_layers_persistent. Attention reads the shared history once per
 * pair of positions; position j sees the new rows of positions 0..j.
 * Arguments as for a verify in decode_layers_persistent (n_tokens must be 1, in_token >= 0
 * and draft_tokens set); out_hidden receives the last position's final hidden state. The
 * results agree with the sequential verify to the rounding of the bf16 activation operands
 * (they are not bit-identical to it).
 * FP8 MLA MoE stacks with an LM head whose handle was created with cfg->max_query >= 2.
 * Errors: PLD_E_UNSUPPORTED (handle without batched verify), PLD_E_INVALID, PLD_E_CAPACITY,
 * PLD_E_STATE, PLD_E_HIP. */
pld_status decode_verify_batched(pld_handle* h, const pld_persistent_args* a, void* stream);

/* Arguments of decode_batch. */
typedef struct pld_batch_args {
  int32_t n_seq;            /* sequences decoded together, 2 .. cfg->max_batch */
  int32_t n_tokens;         /* tokens to decode per sequence (>= 1) */
  int32_t start_pos[8];     /* cache position of each sequence's first token (sequence b's rows
                               0 .. start_pos[b]-1 hold its history) */
  int32_t in_token[8];      /* each sequence's input token, in [0, vocab) */
  float* out_logits;        /* fp32 [n_tokens][n_seq][vocab], or NULL */
  int32_t* out_tokens;      /* int32 [n_tokens][n_seq] chosen tokens (device, 4-byte aligned) */
  void* out_hidden;         /* bf16 [hidden]: the last sequence's final hidden state after the last
                               token, 16-byte aligned */
  double temperature;       /* 0 greedy, > 0 sampled (the rule of decode_layers_persistent, keyed
                               by each sequence's own cache position) */
  uint64_t sample_seed;
} pld_batch_args;

/* Batched decoding of n_seq independent sequences in one launch: every step, the sequences'
 * current tokens go through every layer TOGETHER (each weight read once per step for all
 * of them, on the matrix cores as in decode_verify_batched; the union of the experts the
 * sequences route to is read once), each sequence attends to its own cache and appends its
 * own row, and the head chooses each sequence's next token, which feeds the next step. The
 * vLLM Kimi K3 backend article serves batches of 1 to 64 requests on one node ("A narrow
 * deployment lane") and switches its matmuls to split-K at larger batches ("Four changes
 * drive the gains"); this is the small-batch end of that range on one GPU.
 * Each sequence's tokens equal what decode_layers_persistent gives for it alone, up to the
 * rounding of the bf16 activation operands (not bit-identical).
 * Handles created with cfg->max_batch >= 2 (FP8 MLA MoE stacks with an LM head).
 * Errors: PLD_E_UNSUPPORTED (handle without batch decode), PLD_E_INVALID, PLD_E_CAPACITY
 * (start_pos[b] + n_tokens > max_seq), PLD_E_STATE, PLD_E_HIP. */
pld_status decode_batch(pld_handle* h, const pld_batch_args* a, void* stream);

/* Arguments of decode_speculative. */
typedef struct pld_spec_args {
  int32_t start_pos;     /* cache position of in_token; both caches hold rows 0 .. start_pos-1 */
  int32_t in_token;      /* the last kept token (its rows are not yet in either cache) */
  int32_t n_tokens;      /* tokens to produce */
  int32_t n_draft;       /* drafts proposed per verify, 1 .. 15 */
  double temperature;    /* 0 greedy, > 0 sampled (the rule of decode_layers_persistent) */
  uint64_t sample_seed;
  int32_t* out_tokens;   /* device int32 [n_tokens], 4-byte aligned */
  int32_t* out_stats;    /* host int32 [2] or NULL: verify launches, drafts kept in total */
} pld_spec_args;

/* Speculative decoding with a draft stack (the draft-and-verify loop of the vLLM Kimi K3
 * backend article's speculative decoding, where a cheap drafter proposes tokens that the
 * full model checks in one step). `draft` is a second handle over a shallower stack that
 * shares the target's vocabulary, embedding and LM head (the same device pointers) and
 * has caches of its own holding the same history rows. Each round: one draft launch
 * proposes min(n_draft, left - 1) tokens from the current position, one target verify
 * launch scores them (decode_layers_persistent with n_query = drafts + 1), the leading
 * drafts equal to the target's chosen token are kept together with the target's token after
 * them, and both stacks continue after the last kept token (one extra draft step when all
 * drafts were kept; a plain target step for a last single token). Because a token depends
 * only on its position's logits and the seed, the tokens equal those of plain decoding of
 * the target with the same temperature and seed; the drafts change only the number of
 * launches. Host loop: synchronous on `stream` (one small device-to-host read per round).
 * Rows past the last kept position may hold rejected drafts; later launches overwrite them.
 * Uses 136 bytes of the target's workspace. Errors: PLD_E_INVALID (arguments, handles that
 * do not share the head), PLD_E_CAPACITY (start_pos + n_tokens beyond either cache),
 * PLD_E_STATE, PLD_E_HIP. */
pld_status decode_speculative(pld_handle* target, pld_handle* draft, const pld_spec_args* a, void* stream);

/* Copy the device status word into *out (synchronises the stream of the handle's last
 * launch, nothing else). Returns PLD_OK, or PLD_E_DEVICE_TIMEOUT if the last launch's
 * watchdog fired; the handle then refuses launches (PLD_E_STATE) until decode_reset. */
pld_status decode_poll_status(pld_handle* h, pld_device_status* out);

/* Clear the status and the inter-workgroup handoff buffers so the handle can be used
 * again: waits for the stream of the handle's last launch, clears on that stream and waits
 * again (synchronous). The step epoch keeps counting across resets. */
pld_status decode_reset(pld_handle* h);

/* Free the host-side handle. Device memory stays with the caller. NULL and handles of
 * decode_layer_init_static are ignored. */
void decode_layer_destroy(pld_handle* h);

/* Static description of a status code. */
const char* pld_status_string(pld_status s);

/* Device pointer and size in bytes of a named intermediate in the workspace, as left by
 * the last completed launch (for tests). Plain arrays: "a", "b" (fp32 [hidden]), "f" (fp32
 * [hidden], the FFN output before the residual add), "sel" (int32 [top_k]), "gates" (fp32 [top_k]). LL arrays of 8-byte words whose low 32 bits
 * are the payload and high 32 bits the step epoch: "q", "o", "h2", "m" (fp32 payloads),
 * "x" (bf16 pairs), "logits" (4 words per expert: logit and selection key as fp64,
 * low then high halves), "part" (attention partials), "kv" (GQA: the new k/v row),
 * "amax" (LM head: per-workgroup best logit and token). Batched verify (handles with
 * max_query >= 2; per-position copies, position p at p * (size / 8)): "vx" (bf16 pairs, each
 * layer's output), "vcq", "vckv", "volat", "vh2" (fp32), "vqlat", "vo" (bf16 pairs), and the
 * plain arrays "vsel" (int32 [8][8] top-k experts per position, then fp32 [8][8] gates) and
 * "vf" (fp32 [8][hidden], each position's FFN output before the residual add).
 * Returns PLD_E_INVALID for an unknown name or a buffer the handle does not have. */
pld_status pld_debug_buffer(pld_handle* h, const char* name, void** ptr, size_t* bytes);

/* Launch geometry actually used: number of workgroups and threads per workgroup. */
pld_status pld_launch_shape(pld_handle* h, int32_t* n_wg, int32_t* block);

/* Device trace for profiling inside one launch: while set, every later launch writes, for
 * each (step, workgroup) of its first bytes/(n_wg*56*8) steps (a step is one layer of one
 * token), 56 uint64 wall-clock stamps (hipDeviceAttributeWallClockRate ticks) taken by the
 * workgroup's first thread at fixed points of the step; a slot the step does not pass
 * stays 0. Slots: 0 start, 1 layer input ready, 2 q/k/v (MLA: c_q, c_kv) published,
 * 3/12/13/30 attention phases, 4 attention done, 5 attention output ready, 6 h2
 * published, 7 h2 ready, 8 router logits ready, 16 top-k, 9/18 expert activations
 * published, 10 expert activations ready, 19/20 down projection, 11 layer output
 * published, 32 head input ready, 33 head GEMV done, 34 token chosen (last layer of a
 * token with an LM head); the others mark sub-phases. buffer: device memory of `bytes`
 * bytes, 8-aligned, owned by the caller; NULL turns tracing off. Returns PLD_E_CAPACITY if
 * the buffer cannot hold one step. */
pld_status pld_set_trace(pld_handle* h, void* buffer, size_t bytes);

/* Set the watchdog budget of every bounded device wait, in microseconds (default 2e6). */
pld_status pld_set_watchdog_us(pld_handle* h, int64_t us);

/* Test hooks that force the failure and ordering conditions the vLLM Kimi K3 backend
 * article's kernel audit worries about ("Agent-written kernels face evidence gates":
 * reads hoisted above a synchronisation, bugs that only show under other timings), from
 * the host, with every kernel still exiting normally:
 *   PLD_HOOK_DROP_WG0  the next launch's workgroup 0 leaves at once without publishing
 *                      anything (a producer that never arrives): the other workgroups'
 *                      bounded waits expire, the watchdog records the first, and every
 *                      workgroup exits; the flag clears itself after that launch.
 *   PLD_HOOK_DELAY     every later launch: each workgroup waits a pseudo-random time of up
 *                      to 16 us (a hash of `seed`, workgroup, step and stage) at the start of
 *                      four stages, so workgroups reach every handoff in another order; the
 *                      outputs must not change (every sum has a fixed order).
 * flags = 0 turns the hooks off. Errors: PLD_E_INVALID for unknown flags. */
enum { PLD_HOOK_DROP_WG0 = 1, PLD_HOOK_DELAY = 2 };
pld_status pld_set_test_hooks(pld_handle* h, int32_t flags, uint32_t seed);

#ifdef __cplusplus
}
#endif
#endif /* PLD_H */

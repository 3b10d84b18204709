/*
 * liblsn -- layer-streamed LoRA training over a frozen NF4 decoder base on one
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ or
 * framework types.
 *
 * The method (web pages on the "Soup" fine-tuning CLI):
 *   - "Soup: Fine-Tune an 8B Model on a 4 GB GPU" (lucaberton.com), section
 *     "The Core Idea: Layer Streaming": the frozen weights are held off the
 *     GPU (host memory or a disk) and each decoder layer reaches device
 *     memory, through a copy stream of its own, only when a pass needs it, so
 *     device memory holds about one layer plus the adapter; the held weights
 *     may be NF4; the LoRA adapter is the only trained state; DPO's reference
 *     model is the same base run without the adapter.
 *   - "Show HN: Fine-tune an 8B model on a 4 GB laptop GPU" (elseif.net),
 *     first paragraph: policy log-probs with the adapter on, reference
 *     log-probs with it off, from the same streamed base; results bit-exact
 *     against a non-streamed run.
 *   - axbrief.com article, "Beyond Memory: The Layer Streaming Breakthrough":
 *     streamed results are bit-exact with resident execution.
 *
 * Conventions
 *   - Every call returns lsn_status; nothing throws across the ABI.
 *   - "device pointer" = memory on the context's GPU (the caller allocates it,
 *     e.g. with PyTorch); "host pointer" = ordinary CPU memory, copied before
 *     the call returns and never retained.
 *   - All device work is enqueued on the context's compute stream and the
 *     call returns before it completes.  The library's own copy stream is
 *     ordered against it only through events.  lsn_sync() waits and reports
 *     asynchronous HIP errors.
 *   - The library never allocates device memory: lsn_create carves every
 *     device buffer out of ONE caller-owned workspace of lsn_workspace_bytes().
 *     It owns the pinned host copy of the frozen base (hipHostMalloc) and any
 *     file handle.
 *   - Argument errors return LSN_ERR_INVALID with nothing enqueued.  A HIP
 *     failure returns LSN_ERR_HIP and poisons the context: later calls return
 *     LSN_ERR_STATE.  lsn_last_error() gives a message.
 *   - Weights are stored as W^T = [out, in] row-major (the causal-LM layout),
 *     so a projection is y = x W = x (W^T)^T with x [T, in], y [T, out].
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - A context is not thread-safe; use one per device and per thread.
 */
#ifndef LSN_H
#define LSN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lsn_ctx lsn_ctx;

typedef enum {
  LSN_OK = 0,
  LSN_ERR_INVALID = 1, /* bad argument; nothing enqueued */
  LSN_ERR_NOFIT = 2,   /* workspace (or the configured budget) too small */
  LSN_ERR_HIP = 3,     /* HIP runtime failure; context poisoned */
  LSN_ERR_IO = 4,      /* file source read failure; context poisoned */
  LSN_ERR_STATE = 5    /* call out of order, or context poisoned */
} lsn_status;

/* where the frozen base lives during training */
enum { LSN_RESIDENT = 0, LSN_STREAM_HOST = 1, LSN_STREAM_FILE = 2 };
/* pass kinds: forward visits layers 0..L-1, backward L-1..0 */
enum { LSN_PASS_FWD = 0, LSN_PASS_BWD = 1 };
/* projections of a decoder layer, in record order */
enum { LSN_Q = 0, LSN_K = 1, LSN_V = 2, LSN_O = 3, LSN_GATE = 4, LSN_UP = 5, LSN_DOWN = 6 };

typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t tied_embeddings; /* 1: the LM head is the embedding table */
  float rms_eps, rope_theta;
  int32_t lora_rank;       /* 1..16 */
  float lora_alpha;        /* LoRA scale s = alpha / rank */
  uint32_t lora_targets;   /* bit p set = projection p carries an adapter */
  int32_t max_tokens;      /* upper bound of n_seq * seq_len per pass */
  int32_t max_seq_len;     /* upper bound of seq_len */
  int32_t mode;            /* LSN_RESIDENT | LSN_STREAM_HOST | LSN_STREAM_FILE */
  const char* store_path;  /* LSN_STREAM_FILE: file that holds the layer records */
  uint64_t vram_budget;    /* 0 = none; else lsn_create refuses a larger workspace */
  /* 1 (streamed modes only): the embedding and LM-head tables stay in the
   * library's pinned host memory instead of the workspace; the embedding
   * gather and the head backward's target rows read them over the host link,
   * and each LM-head pass streams W_lm in slot-sized row chunks through the
   * two layer slots (page "Soup: Fine-Tune an 8B Model on a 4 GB GPU", "The
   * Core Idea: Layer Streaming": only the current layer and the adapter
   * need to sit in VRAM).  0: both tables live in the workspace. */
  int32_t head_on_host;
  /* vocabulary rows per LM-head chunk: 0 picks them (about 256 output tiles
   * at max_tokens, at least 16384, and with head_on_host at most one slot of
   * W_lm rows); else a multiple of 8, at most one slot of rows with
   * head_on_host.  The logits buffer holds max_tokens x rows fp32. */
  int32_t head_chunk_rows;
  /* device slots the streamed modes copy layer records into: 0 or 2 = a
   * double buffer (the copy of the next layer overlaps the current one); 3
   * or 4 keep more records resident, so the first layers of a pass that
   * another pass has just left in the slots are reused instead of copied
   * again (2 * (n_slots - 2) fewer record copies per SFT step), at one
   * record of device memory per slot.  Ignored when resident. */
  int32_t n_slots;
  /* 0: a layer call runs all of the pass's tokens as one batch.  Else the
   * layer workspace holds max(layer_tokens, max_seq_len) tokens (at most
   * max_tokens) and each layer call runs its sequences in groups of as many
   * whole sequences as that holds, one group after the other on the same
   * record (a DPO pair: the chosen and then the rejected sequence).  The
   * record is still copied once per layer; the adapter gradients of the
   * groups are added in group order.  Cuts the activation memory of a
   * multi-sequence pass: the pages report streamed DPO below the SFT memory
   * peak ("Show HN: Fine-tune an 8B model on a 4 GB laptop GPU", second
   * paragraph). */
  int32_t layer_tokens;
} lsn_config;

/* ---------------------------------------------------------------------------
 * NF4 host codec (no context).  The pages name the format only ("Soup:
 * Fine-Tune an 8B Model on a 4 GB GPU", "The Core Idea: Layer Streaming":
 * the streamed base optionally quantized to NF4, about four times smaller).
 * Format used: 16 normal-quantile levels with an exact zero, scaled to
 * [-1, 1]; blocks of 64 consecutive elements of the flattened W^T, one fp32
 * absmax per block; code = number of fp32 midpoints strictly below
 * fl32(w / absmax); an all-zero block stores absmax 0 and code 7; two codes
 * per byte, even element in the low nibble (odd n pads a zero nibble).
 * ------------------------------------------------------------------------- */
/* out16: host, 16 floats, ascending (-1 .. 1, entry 7 is 0). */
lsn_status lsn_nf4_codebook(float* out16);
/* w: host [n] fp32 (finite, else LSN_ERR_INVALID); codes: host [(n+1)/2];
 * absmax: host [(n+63)/64].  Multithreaded; deterministic. */
lsn_status lsn_nf4_quantize(const float* w, uint64_t n, uint8_t* codes, float* absmax);
/* host inverse: w[e] = fl32(level[code_e] * absmax[e/64]). */
lsn_status lsn_nf4_dequantize(const uint8_t* codes, const float* absmax, uint64_t n, float* w);

/* ---------------------------------------------------------------------------
 * Device NF4 dequantization (all pointers device).  out_bf16 = 0: fp32
 * output fl32(level * absmax), bit-equal to the host codec; 1: that value
 * rounded to bf16 (what the GEMMs feed the matrix cores).  n % 8 == 0.
 * ------------------------------------------------------------------------- */
lsn_status lsn_nf4_dequant(const uint8_t* codes, const float* absmax, uint64_t n, void* out,
                           int32_t out_bf16, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Single NF4 projection with a LoRA branch, stateless (the frozen linear of
 * "only the adapter trains", page "Soup: Fine-Tune an 8B Model on a 4 GB GPU",
 * "The Core Idea: Layer Streaming"; formula y = x W + s (x A) B).
 * All pointers device.  W^T codes [N*K/2] + absmax [N*K/64] as the codec
 * writes them; X bf16 [M, K]; A fp32 [K, r]; B fp32 [r, N] (A = B = NULL or
 * r = 0: no adapter); Y fp32 [M, N].  K % 16 == 0, N % 8 == 0, r <= 16.
 * scratch: device, >= lsn_nf4_linear_scratch_bytes().
 * bwd: dY bf16 [M, N] -> dX fp32 [M, K] (overwritten), dA fp32 [K, r] and
 * dB fp32 [r, N] (overwritten; may be NULL when r = 0).  The base gets no
 * gradient.
 * ------------------------------------------------------------------------- */
lsn_status lsn_nf4_linear_scratch_bytes(int32_t M, int32_t K, int32_t N, int32_t r,
                                        uint64_t* bytes);
lsn_status lsn_nf4_linear_fwd(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                              int32_t N, const uint16_t* X, const float* A, const float* B,
                              int32_t r, float s, float* Y, void* scratch, uint64_t scratch_bytes,
                              void* hip_stream);
lsn_status lsn_nf4_linear_bwd(const uint8_t* codes, const float* absmax, int32_t M, int32_t K,
                              int32_t N, const uint16_t* X, const float* A, const float* B,
                              int32_t r, float s, const uint16_t* dY, float* dX, float* dA,
                              float* dB, void* scratch, uint64_t scratch_bytes, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward projection as lsn_nf4_linear_fwd, same arguments without the
 * scratch, and the same bits (the same kernels and split-k).  Its scratch
 * is a fixed 64 MiB device array inside the library (allocated by the HIP
 * runtime with the library's code on each device it runs on, held until the
 * process ends); the call allocates nothing.  A shape whose scratch (t and
 * the bf16 adapter operands, the low-rank product's partial sums, and the
 * NF4 GEMM's split-k partial sums: split x (M x N + 1024) fp32, split up to
 * 8 when M x N is small) exceeds 64 MiB returns LSN_ERR_INVALID with the
 * bytes it needs.  Every call on a device shares that device's array: calls
 * that overlap on one device (two streams, two threads) race and corrupt
 * each other's results; calls on one stream are ordered and safe. */
lsn_status lsn_nf4_linear_fwd_noalloc(const uint8_t* codes, const float* absmax, int32_t M,
                                      int32_t K, int32_t N, const uint16_t* X, const float* A,
                                      const float* B, int32_t r, float s, float* Y,
                                      void* hip_stream);

/* ---------------------------------------------------------------------------
 * Context lifecycle.
 * ------------------------------------------------------------------------- */
/* Device bytes the context needs for cfg (records or slots, head tables,
 * adapters and gradients, one layer's activations at max_tokens). */
lsn_status lsn_workspace_bytes(const lsn_config* cfg, uint64_t* bytes);
/* Bytes of one layer record for cfg (codes + absmax + norm gains, 4 KiB
 * aligned): the host store holds n_layers of them, a streamed step copies
 * each one twice.  Used to choose RAM or file storage before lsn_create
 * ("RAM when it fits, NVMe when it does not": page "Soup: Fine-Tune an 8B
 * Model on a 4 GB GPU", "The Core Idea: Layer Streaming"). */
lsn_status lsn_config_record_bytes(const lsn_config* cfg, uint64_t* bytes);
/* dev_ws: device, ws_bytes >= lsn_workspace_bytes (else LSN_ERR_NOFIT, the
 * pre-flight refusal of a run that will not fit: page "Soup: Fine-Tune an 8B
 * Model on a 4 GB GPU", "A Practical Quick Start").  hip_stream: the compute
 * stream (hipStream_t, may be 0).  The context's copy stream is created
 * non-blocking, so it never synchronizes implicitly with the null stream.  The
 * workspace stays owned by the caller and must outlive the context. */
lsn_status lsn_create(const lsn_config* cfg, void* dev_ws, uint64_t ws_bytes, void* hip_stream,
                      lsn_ctx** out);
void lsn_destroy(lsn_ctx* ctx);
/* The message of the context's last error.  With ctx == NULL: the message of
 * the calling thread's last failed call that takes no context (lsn_create,
 * the stateless projection and dequantization calls). */
const char* lsn_last_error(const lsn_ctx* ctx);
lsn_status lsn_sync(lsn_ctx* ctx);
/* bytes of one layer record (NF4 codes + absmax + norm gains), 4 KiB aligned */
lsn_status lsn_record_bytes(const lsn_ctx* ctx, uint64_t* bytes);
/* *direct = 1 when the file source reads its records with O_DIRECT (around
 * the page cache, so each streamed step reads the storage device), 0 when the
 * file system refused O_DIRECT and reads are buffered, or when the context
 * has no file source (page "Soup: Fine-Tune an 8B Model on a 4 GB GPU", "The
 * Core Idea: Layer Streaming": the base may stream from NVMe). */
lsn_status lsn_file_direct_io(const lsn_ctx* ctx, int32_t* direct);

/* ---------------------------------------------------------------------------
 * Frozen base (page "Soup: Fine-Tune an 8B Model on a 4 GB GPU", "The Core
 * Idea: Layer Streaming": the frozen base is kept in CPU RAM or on NVMe).
 * Host pointers; copied into the library's pinned store (and, in
 * LSN_RESIDENT mode, into the device record).  codes[p]/absmax[p] as
 * lsn_nf4_quantize writes them for W_p^T; norms bf16 [hidden].
 * LSN_STREAM_FILE: the record is written to store_path at its offset.
 * Between passes a layer may be loaded again: the call waits for any copy
 * still reading the old record, and the next pass copies the new one.
 * ------------------------------------------------------------------------- */
lsn_status lsn_load_layer_nf4(lsn_ctx* ctx, int32_t layer, const uint8_t* const* codes,
                              const float* const* absmax, const uint16_t* attn_norm_bf16,
                              const uint16_t* mlp_norm_bf16);
/* embed, lm_head: host bf16 [vocab, hidden] (lm_head NULL when tied);
 * final_norm: host bf16 [hidden].  Kept resident on the device. */
lsn_status lsn_load_head(lsn_ctx* ctx, const uint16_t* embed_bf16, const uint16_t* lm_head_bf16,
                         const uint16_t* final_norm_bf16);

/* ---------------------------------------------------------------------------
 * Adapters: fp32 masters and gradients live in the workspace.  Host pointers.
 * A [K, r], B [r, N] of projection proj of layer; proj must be a target.
 * ------------------------------------------------------------------------- */
lsn_status lsn_set_lora(lsn_ctx* ctx, int32_t layer, int32_t proj, const float* A, const float* B);
/* any output may be NULL */
lsn_status lsn_get_lora(lsn_ctx* ctx, int32_t layer, int32_t proj, float* A, float* B, float* dA,
                        float* dB);
/* 0: forward skips every low-rank branch (the DPO reference model, page
 * "Show HN: Fine-tune an 8B model on a 4 GB laptop GPU", first paragraph);
 * 1: branches on.  Backward requires 1 (else LSN_ERR_STATE from lsn_begin_pass
 * and from every lsn_backward_layer). */
lsn_status lsn_set_adapter_enabled(lsn_ctx* ctx, int32_t enabled);
lsn_status lsn_zero_grads(lsn_ctx* ctx);
/* theta -= lr * grad for every adapter matrix (plain SGD). */
lsn_status lsn_sgd_step(lsn_ctx* ctx, float lr);

/* ---------------------------------------------------------------------------
 * A pass over the stack (page "Soup: Fine-Tune an 8B Model on a 4 GB GPU",
 * section "The Core Idea: Layer Streaming", second bullet: on a dedicated
 * stream the base is copied into VRAM one decoder layer at a time, as the
 * forward or the backward pass reaches it).  begin_pass fixes the layer
 * order (FWD 0..L-1, BWD L-1..0) and the pass geometry: n_seq sequences of
 * seq_len tokens each, back to back (T = n_seq*seq_len; seq_len % 8 == 0,
 * seq_len <= max_seq_len, T <= max_tokens, else LSN_ERR_INVALID).  When
 * streaming it starts copying the first layer records into the device slots
 * on the copy stream.  Each forward_layer / backward_layer must name the next
 * layer of the pass (else LSN_ERR_STATE, nothing enqueued); it waits for its
 * record, runs, frees the slot and queues the copy of the next layer that is
 * not in a slot.  A record already in a slot is reused, not copied again.
 * ------------------------------------------------------------------------- */
lsn_status lsn_begin_pass(lsn_ctx* ctx, int32_t kind, int32_t n_seq, int32_t seq_len);
/* The input of the first decoder layer: the embedding row of each token (the
 * pages stream only the decoder layers, same section, first and second
 * bullets; the embedding table stays with the head tables).  tokens: device
 * int32 [T] of the current pass; h0: device fp32 [T, hidden], overwritten.
 * A token outside [0, vocab) gives a NaN row and reads no table row.
 * LSN_ERR_STATE before lsn_load_head or outside a pass. */
lsn_status lsn_embed(lsn_ctx* ctx, const int32_t* tokens, float* h0);
/* One decoder layer of the forward pass on the layer's streamed record (same
 * section: the layer is in VRAM only while the pass needs it).  h_in, h_out:
 * device fp32 [T, hidden] (may alias), caller-owned.  Computes RMSNorm,
 * q/k/v (+LoRA), RoPE, causal GQA attention, o (+LoRA) + residual, RMSNorm,
 * SwiGLU MLP (+LoRA) + residual; low-rank branches follow
 * lsn_set_adapter_enabled.  The caller keeps h_in for the backward pass. */
lsn_status lsn_forward_layer(lsn_ctx* ctx, int32_t layer, const float* h_in, float* h_out);
/* Reference and policy forward of one layer on ONE copy of its record: the
 * layer runs first with every low-rank branch skipped on h_ref_in ->
 * h_ref_out (the DPO reference model: the same base with the adapter off,
 * page "Show HN: Fine-tune an 8B model on a 4 GB laptop GPU", first
 * paragraph), then with the adapter state set by lsn_set_adapter_enabled on
 * h_in -> h_out.  Results are bit-identical to two separate passes; the
 * streamed base is read once instead of twice (that page's second paragraph
 * gives the cost of separate passes: 1.52x the layer reads of SFT).
 * Device fp32 [T, hidden] each; the outputs must not alias the other
 * stream's buffers. */
lsn_status lsn_forward_layer_pair(lsn_ctx* ctx, int32_t layer, const float* h_ref_in,
                                  float* h_ref_out, const float* h_in, float* h_out);
/* One decoder layer of the backward pass (page "Soup: Fine-Tune an 8B Model
 * on a 4 GB GPU", section "The Core Idea: Layer Streaming": the backward pass
 * streams each layer again, and only the adapter trains).  Recomputes the
 * layer from its saved input h_in_saved, then back-propagates:
 * dh_in = d loss / d h_in (may alias dh_out), and adds the adapter
 * gradients of this layer into the context's gradient buffers.  The base
 * gets no gradient.  All device fp32 [T, hidden].  Needs the adapters on
 * (else LSN_ERR_STATE). */
lsn_status lsn_backward_layer(lsn_ctx* ctx, int32_t layer, const float* h_in_saved,
                              const float* dh_out, float* dh_in);

/* ---------------------------------------------------------------------------
 * LM head: the per-token log-probabilities of the training targets (page
 * "Show HN: Fine-tune an 8B model on a 4 GB laptop GPU", first paragraph:
 * the policy log-probs come from a pass with the adapter active, the
 * reference log-probs from a pass of the same base with it switched off).
 * h: device fp32 [T, hidden]; targets: device int32 [T] (a negative target
 * gives logp 0; a target >= vocab gives NaN and reads no table row); logp:
 * device fp32 [T] = log softmax(RMSNorm(h) W_lm^T) at the target, over the
 * vocabulary in chunks (online max / sum).  want_grad_state != 0 also keeps,
 * per position, the expected embedding row E[t] = sum_v softmax_v W_v,
 * accumulated chunk by chunk (rescaled to the running max), for the
 * backward.  lm_head_backward is the derivative of that definition: it must
 * follow an lm_head_logprobs call with want_grad_state on the same h (else
 * LSN_ERR_STATE) and writes dh (device fp32 [T, hidden], overwritten) from
 * dlogp (device fp32 [T]) as dlogp_t (W[y_t] - E[t]) through the final
 * RMSNorm, with no second pass over W_lm.
 * ------------------------------------------------------------------------- */
lsn_status lsn_lm_head_logprobs(lsn_ctx* ctx, const float* h, const int32_t* targets, float* logp,
                                int32_t want_grad_state);
lsn_status lsn_lm_head_backward(lsn_ctx* ctx, const float* h, const int32_t* targets,
                                const float* dlogp, float* dh);

/* ---------------------------------------------------------------------------
 * Losses (device pointers).
 * SFT: loss[0] = -mean of logp over positions with target >= 0;
 *      dlogp = -1/count there, 0 elsewhere.
 * DPO on one pair laid out as two sequences (chosen, rejected) of seq_len:
 *      pc, pr (policy) and rc, rr (reference) = sums of logp over response
 *      targets (positions prompt_len-1 .. seq_len-2 of each sequence);
 *      z = beta((pc - rc) - (pr - rr)); out[0] = -log sigmoid(z), out[1] = z,
 *      out[2..5] = pc, pr, rc, rr; dlogp_pol = -+ beta sigmoid(-z) on the
 *      chosen / rejected response positions, 0 elsewhere.  The reference
 *      log-probs come from the same base with the adapter off (page "Show HN:
 *      Fine-tune an 8B model on a 4 GB laptop GPU", first paragraph).
 * ------------------------------------------------------------------------- */
lsn_status lsn_sft_loss(lsn_ctx* ctx, const float* logp, const int32_t* targets, int32_t n,
                        float* loss, float* dlogp);
lsn_status lsn_dpo_loss(lsn_ctx* ctx, const float* logp_pol, const float* logp_ref,
                        int32_t seq_len, int32_t prompt_len, float beta, float* out6,
                        float* dlogp_pol);

/* Other preference losses over the same streamed base (page "axbrief.com",
 * "The Architecture of Low-VRAM Alignment", and the evermx page: DPO, ORPO,
 * SimPO and KTO run over layer streaming; the pages give no formulas).
 * Same pair layout and response positions as lsn_dpo_loss; n = seq_len -
 * prompt_len response tokens per sequence; mc, mr = pc/n, pr/n.
 *   LSN_LOSS_DPO   as lsn_dpo_loss (param unused)
 *   LSN_LOSS_SIMPO u = beta(mc - mr) - param (param = gamma), loss = -log sig(u)
 *   LSN_LOSS_ORPO  v = lo(mc) - lo(mr), lo(m) = m - log(1 - e^m),
 *                  loss = -mc - param * log sig(v) (param = lambda; beta unused)
 *   LSN_LOSS_KTO   loss = (1 - sig(beta(pc-rc))) + (1 - sig(-beta(pr-rr)))
 *                  (chosen desirable, rejected undesirable, reference point 0)
 * logp_ref (device) is required for DPO and KTO and ignored otherwise.
 * out6 = {loss, z|u|v|pc-rc, pc, pr, rc, rr}; dlogp_pol as for DPO. */
enum { LSN_LOSS_DPO = 0, LSN_LOSS_SIMPO = 1, LSN_LOSS_ORPO = 2, LSN_LOSS_KTO = 3 };
lsn_status lsn_pref_loss(lsn_ctx* ctx, int32_t kind, const float* logp_pol, const float* logp_ref,
                         int32_t seq_len, int32_t prompt_len, float beta, float param,
                         float* out6, float* dlogp_pol);

/* Counters since lsn_create: layer records copied host->device, bytes copied
 * host->device by the scheduler, and workspace bytes carved.  Any may be NULL. */
lsn_status lsn_stats(const lsn_ctx* ctx, uint64_t* layer_loads, uint64_t* bytes_h2d,
                     uint64_t* ws_bytes);
/* Fault injection, for tests of the stream ordering (results must not
 * change: streamed runs are bit-exact against resident ones, page "Show HN:
 * Fine-tune an 8B model on a 4 GB laptop GPU", first paragraph).
 * copy_delay_us: a kernel on the copy stream waits this long before every
 * copy into a slot (a compute that did not wait for its copy would read the
 * slot early); compute_delay_us: a kernel on the compute stream waits this
 * long before every layer's kernels (a copy that did not wait for the slot's
 * last reader would overwrite it early); poison_slots != 0: every slot is
 * filled with 0xFF bytes (NaN fp32, NaN absmax) on the copy stream just
 * before a copy into it.  Delays 0..100000, else LSN_ERR_INVALID. */
lsn_status lsn_set_fault_injection(lsn_ctx* ctx, int32_t copy_delay_us, int32_t compute_delay_us,
                                   int32_t poison_slots);
/* The copy stream (hipStream_t) the scheduler uses, for timing its copies. */
lsn_status lsn_copy_stream(const lsn_ctx* ctx, void** hip_stream);

/* ---------------------------------------------------------------------------
 * Live timing (measurement only; results are unchanged).  on is a mask: bit
 * 0 records a timing event pair on every NF4 GEMM launch (carried by the
 * kernel's own dispatch on the compute stream, so it adds no packet), bit 1
 * an event pair around every layer-record copy (two event packets on the
 * copy stream per copy); 0 stops, other values give LSN_ERR_INVALID.  Any
 * call clears earlier records.  Synchronizes both streams.
 * ------------------------------------------------------------------------- */
lsn_status lsn_set_profiling(lsn_ctx* ctx, int32_t on);
/* Totals over the recorded events.  what = 0: NF4 GEMM launches whose operand
 * forms are (a, b) -- A: 0 bf16 row-major, 1 bf16 transposed, 2 fp32
 * row-major; B: 0 bf16 [N,K], 1 bf16 [K,N], 2 NF4 W^T used as y = x W,
 * 3 NF4 W^T used as dx = dy W^T -- and whose tile id is tile (0: 256x128,
 * 1: 128x128, 2: 64x64, 3: the 256x256 forward NF4 kernel, 4: the 256x256
 * input-gradient NF4 kernel; -1: any);
 * work = algorithmic flops 2*M*N*K per
 * problem (the low-rank extension not counted).  what = 1: record copies;
 * work = bytes.  count = launches, ms = summed event time.  Synchronizes. */
lsn_status lsn_profile_query(lsn_ctx* ctx, int32_t what, int32_t a, int32_t b, int32_t tile,
                             uint64_t* count, double* work, double* ms);

#ifdef __cplusplus
}
#endif
#endif /* LSN_H */

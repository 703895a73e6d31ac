/*
 * mk.h -- C ABI of the MI355X persistent decode megakernel (libmk.so).
 *
 * One autoregressive decode step of a Llama-style decoder runs as a static,
 * fine-grained task graph inside one long-lived HIP kernel (MPK blog
 * translation, "MPK runtime" section and Figure 3; MPK walk-through sections
 * 0.2 and 3.2; Hazy megakernel summary: one kernel per forward pass).
 *
 * Conventions for every call:
 *  - Return value: MK_OK (0) or a negative MK_E* code. No exception crosses the
 *    ABI. mk_last_error() returns a thread-local message for the last failure.
 *  - "device pointer" = memory on the current HIP device (e.g. torch tensor
 *    data_ptr()); "host pointer" = ordinary CPU memory.
 *  - Streams are hipStream_t passed as void* (NULL = the null stream).
 *  - Nothing here allocates or frees caller memory; the library owns only what
 *    its own mk_* objects hold and releases it in mk_free_*.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MK_OK            0
#define MK_EINVAL       (-1)   /* bad argument (shape, NULL, range) */
#define MK_ENOMEM       (-2)   /* device or host allocation failed */
#define MK_EHIP         (-3)   /* a HIP runtime call failed */
#define MK_ETIMEOUT     (-4)   /* device watchdog expired inside the kernel */
#define MK_EUNSUPPORTED (-5)   /* shape/option/device the library does not support */
#define MK_EDEVICE      (-6)   /* device-side argument error (token or position out of range) */

/* decode modes for mk_decode_step */
#define MK_NOALLOC_SCRATCH_BYTES (16u << 20) /* static workspace of mk_generate_noalloc, per GPU */

#define MK_MODE_MEGAKERNEL 0   /* one persistent launch runs the whole step */
#define MK_MODE_OPLAUNCH   1   /* one launch per operator, same task bodies (baseline) */

/* Model shape (MPK walk-through 3.3.1: hidden size, heads, kv heads, head dim,
 * vocab; max_seq_length in the PersistentKernel constructor). tied_embeddings
 * = 1 uses the embedding as LM head. rms_eps is added inside the square root of
 * RMSNorm; rope_theta is the RoPE base (half-split pairs, no scaling).
 * qk_norm = 1: each query and key head vector is RMS-normalised over head_dim
 * with its layer's [head_dim] gain (q_norm / k_norm weights) after the
 * projection and before RoPE (MPK walk-through 3.3.1: attention_layer takes
 * q_norm and k_norm); 0: no such norm (Llama). */
typedef struct mk_model_desc {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t tied_embeddings, max_batch, max_seq;
    float rms_eps, rope_theta;
    int32_t qk_norm;
} mk_model_desc;

/* Task-graph knobs (MPK walk-through 3.3.1: per-layer grid sizes and worker
 * counts). 0 = default; the defaults are a pure function of the desc:
 * num_cus 256, row_block 4, use_mfma 2 when a launch holds more than 4
 * sequences (min(max_batch, 16) > 4) and hidden, n_q_heads * head_dim and ffn
 * are multiples of 64 of at least 256, else 1; qkv_tasks_per_group
 * ceil(num_cus / n_kv_heads), with use_mfma 2 at least one per 16 rows of a
 * group ((n_q_heads / n_kv_heads + 2) * head_dim rows); gu_tasks = d_tasks = num_cus; o_tasks num_cus,
 * or ceil(num_cus / 2) with use_mfma 1 when the O projection's weights
 * (hidden * n_q_heads * head_dim bf16) are under 64 KiB per num_cus task; lm_tasks
 * num_cus (use_mfma 1) or max(num_cus, ceil(vocab / 128)) (use_mfma 2);
 * attn_chunks max(1, min(num_cus / (min(max_batch, 4) * n_kv_heads),
 * max_seq / 1024)). Every task count is then capped at the number of
 * row_block-row blocks of its operator's rows. */
typedef struct mk_graph_opts {
    int32_t num_cus;             /* compute units = workgroups of the persistent kernel */
    int32_t qkv_tasks_per_group; /* QKV tasks per kv head group */
    int32_t o_tasks, gu_tasks, d_tasks, lm_tasks;
    int32_t attn_chunks;         /* attention position chunks per (kv group, sequence) */
    int32_t row_block;           /* rows per matvec block (task row ranges are whole blocks) */
    int32_t use_mfma;            /* matvec bodies: 1 vector ALU (at most 4 sequences per launch),
                                    2 matrix cores (v_mfma, at most 16 sequences per launch; hidden,
                                    Hq*head_dim and ffn multiples of 64, at least 256);
                                    0 = 2 when a launch would hold more than 4 sequences and the
                                    shape allows it, else 1 */
} mk_graph_opts;

typedef struct mk_graph mk_graph;   /* host-only task graph */
typedef struct mk_model mk_model;   /* graph + packed weights + device state */

/* Per-layer weights: device pointers to bf16, HF layout [out, in] row-major.
 * wq [Hq*D, H], wk/wv [Hkv*D, H], wo [H, Hq*D], wg/wu [F, H], wd [H, F],
 * g_attn/g_mlp [H] (RMSNorm gains); q_norm/k_norm [D] (per-head q/k RMSNorm
 * gains, read only when the desc has qk_norm = 1, else may be NULL). */
typedef struct mk_layer_weights {
    const void *wq, *wk, *wv, *wo, *wg, *wu, *wd, *g_attn, *g_mlp;
    const void *q_norm, *k_norm;
} mk_layer_weights;

/* All model tensors (MPK walk-through 3.3.1: attach_input of every weight and
 * of the per-layer k_cache / v_cache). embed [V, H] bf16; lm_head [V, H] bf16 or
 * NULL when tied; g_final [H] bf16; layers = HOST array of n_layers entries.
 * k_cache / v_cache: bf16 [L][max_batch][Hkv][max_seq][D], caller-owned decode
 * state that must stay alive and unmoved while the model is used; keys are
 * stored after RoPE. */
typedef struct mk_weights {
    const void *embed, *lm_head, *g_final;
    const mk_layer_weights *layers;
    void *k_cache, *v_cache;
} mk_weights;

/* Split each operator of one decode step into per-compute-unit tasks joined by
 * events with trigger thresholds, and place them round-robin on per-unit queues
 * (MPK blog translation, "MPK compiler" section and Figure 2; MPK walk-through
 * 3.2 task-graph generation: dependency analysis, event generation, TaskDesc /
 * EventDesc). Host only; touches no device. *out receives a new graph the
 * caller frees with mk_free_graph. opts may be NULL (all defaults).
 * Errors: MK_EINVAL for an inconsistent shape (Hq not a multiple of Hkv, odd
 * head_dim, K dims not multiples of 8, qk_norm not 0 or 1, ...), MK_ENOMEM. */
int mk_build_task_graph(const mk_model_desc *desc, const mk_graph_opts *opts, mk_graph **out);

/* Canonical little-endian bytes of the graph (header, tasks, events, queues):
 * the compiled form of the task graph that the runtime executes (MPK blog
 * translation, "MPK compiler" section: the compiler's output is the task graph
 * the runtime consumes; MPK walk-through 3.2: TaskDesc / EventDesc arrays).
 * The layout is this library's own, version 5 (magic, version, desc, resolved
 * options, then each task's type, layer, sequence, kv group, chunk, row range,
 * dependent and triggering event and compute unit, each event's threshold and
 * dependents, each unit's queue), so that two builders of the same
 * specification can be compared byte for byte. Writes at most cap bytes into
 * buf (buf may be NULL with cap 0 to query) and always stores the full length
 * in *len. MK_EINVAL if buf is too small or g is NULL. */
int mk_graph_serialize(const mk_graph *g, uint8_t *buf, size_t cap, size_t *len);

/* Counts and the resolved (default-filled) options of a graph. Any output
 * pointer may be NULL. */
int mk_graph_info(const mk_graph *g, int32_t *n_tasks, int32_t *n_events, mk_graph_opts *resolved);

void mk_free_graph(mk_graph *g);

/* Bind a graph to the current HIP device: pack the weights into the library's
 * tile-major copy (QKV rows grouped per kv head and gate/up rows interleaved per
 * block, as fuse_tensors does in MPK walk-through 3.3.1), upload task
 * descriptors, per-unit queues, event thresholds and counters, build the RoPE
 * cos/sin tables, and allocate the activation workspace (MPK walk-through 3.2,
 * runtime initialisation). Weight pointers may be freed after this returns; the
 * KV cache may not. Work is enqueued on `stream` and completed before return.
 * *out receives a model the caller frees with mk_free_model (after its work
 * has finished). The graph may be freed afterwards.
 * One launch stages at most batch_per_launch sequences (mk_model_info): the
 * largest count up to 4 whose staging slots leave LDS room for weight rings of
 * at least 4 items per stream wave. max_batch may exceed it (up to 256); a
 * model whose max_batch exceeds batch_per_launch runs, on each group of
 * sequences, the graph these options give for a batch_per_launch-sequence desc
 * (mk_model_info's n_tasks counts that graph's tasks).
 * Errors: MK_EINVAL (NULL pointer, a NULL q_norm/k_norm with qk_norm = 1),
 * MK_EUNSUPPORTED (fewer resident compute
 * units than num_cus, shape the library does not support), MK_ENOMEM, MK_EHIP. */
int mk_load_weights(const mk_graph *g, const mk_weights *w, void *stream, mk_model **out);

/* One decode step for `batch` (1..max_batch) sequences (MPK walk-through
 * 3.3.1, the per-step model: embedding, per layer RMSNorm + QKV, attention with
 * the KV cache, O projection + residual, RMSNorm + gate/up, SiLU, down
 * projection + residual, final RMSNorm, LM head, argmax; MPK blog translation,
 * "MPK runtime" section: the step's task graph run by per-unit workers that
 * wait on and trigger events): feed d_tokens[b] at
 * position d_pos[b], write K/V there, attend over 0..d_pos[b], and write the
 * greedy next token to d_next[b] and (if d_logits != NULL) the fp32 logits to
 * d_logits [batch, V] row-major. All four arrays are device pointers (int32 /
 * fp32). mode MK_MODE_MEGAKERNEL = one persistent launch; MK_MODE_OPLAUNCH = one
 * launch per operator with the same task bodies. A batch above the model's
 * batch_per_launch runs as consecutive launches over groups of that many
 * sequences (sequences never interact), each group's outputs at its own rows.
 * Asynchronous on `stream`;
 * argument errors return synchronously. Device-side errors (token >= V,
 * position >= max_seq, watchdog) are recorded in the model's status word,
 * which only mk_check reads and reports: a later call still returns MK_OK.
 * After a watchdog expiry the abort word stays raised until mk_check has
 * reported it, so launches made in between leave at their first wait and
 * write no outputs; the call after mk_check resets the counters. */
int mk_decode_step(mk_model *m, const int32_t *d_tokens, const int32_t *d_pos, int32_t batch,
                   float *d_logits, int32_t *d_next, int32_t mode, void *stream);

/* n_steps greedy decode steps inside ONE persistent launch (MPK walk-through
 * 0.2: the CPU launches once; the step counter and token buffer live on the
 * device). Step k feeds, for every sequence b, d_tokens0[b] (k = 0) or the
 * token chosen at step k-1, at position d_pos0[b] + k. Chosen tokens go to
 * d_out_tokens [n_steps, batch] (int32, device); if d_last_logits != NULL the
 * fp32 logits of the final step go there [batch, V]. A batch above
 * batch_per_launch runs group by group, as for mk_decode_step (each group's
 * n_steps in one launch). Asynchronous on `stream`; errors as for
 * mk_decode_step. */
int mk_generate(mk_model *m, const int32_t *d_tokens0, const int32_t *d_pos0, int32_t batch,
                int32_t n_steps, int32_t *d_out_tokens, float *d_last_logits, void *stream);

/* mk_generate for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, outputs and errors as mk_generate, and the same kernels, so the
 * same tokens, logits and KV-cache entries bit for bit. The launch's scratch
 * (event counters, abort flag, activations, attention and LM partials, token
 * buffer) lives in one static device array of MK_NOALLOC_SCRATCH_BYTES (16 MiB)
 * per GPU, which that GPU holds until the process ends, instead of in the
 * model's own workspace; this call allocates and frees nothing and records no
 * memset (a fill kernel clears the counters at the start of every launch). The
 * array's address on a device is resolved once, by the first mk_load_weights
 * on that device. Every call on one GPU shares the array and finds it as the
 * last call left it: calls that overlap on one GPU (other streams, other
 * threads) race; order them on one stream. The model's status word still
 * reports device errors (mk_check). Errors: as mk_generate; MK_EINVAL also
 * when one launch of this model needs more scratch than the array holds (the
 * message gives both sizes; the Llama-3.2-1B and Llama-3-8B shapes need about
 * 2.7 and 5.3 MiB at one sequence per launch, 12.1 MiB at four) or
 * n_steps is too large for the event counters; MK_EHIP if the array's address
 * was not resolved on the current device. */
int mk_generate_noalloc(mk_model *m, const int32_t *d_tokens0, const int32_t *d_pos0, int32_t batch,
                        int32_t n_steps, int32_t *d_out_tokens, float *d_last_logits, void *stream);

/* Prefill: the n_tokens prompt tokens d_tokens (device int32) of sequence
 * `seq` at positions pos0 .. pos0 + n_tokens - 1, as columns of one graph
 * step per group of batch_per_launch consecutive tokens (16 on the
 * matrix-core bodies) instead of one step per token (MPK blog translation,
 * Figure 1 workload: a prompt then generation; MPK walk-through 3.2: the
 * prompt is placed in the token buffer before the kernel runs). Every column
 * runs the whole decoder for its position: the projections and the MLP as
 * one batched matvec over the columns, attention over the sequence's cached
 * positions before the group plus the group's own positions up to the
 * column's (causal), its key and value appended to the sequence's caches.
 * Writes the greedy next token of every position to d_next[n_tokens] and, if
 * d_logits != NULL, the fp32 logits of every position to d_logits
 * [n_tokens, V] (device). Positions below pos0 must hold the sequence's
 * cache entries already (a previous prefill or decode). Asynchronous on
 * `stream`; MK_EINVAL for a NULL pointer, seq outside 0..max_batch-1,
 * n_tokens < 1 or pos0 + n_tokens > max_seq; device errors as for
 * mk_decode_step. */
int mk_prefill(mk_model *m, const int32_t *d_tokens, int32_t n_tokens, int32_t seq, int32_t pos0, float *d_logits,
               int32_t *d_next, void *stream);

/* Synchronise `stream`, then read and clear the model's device status word
 * (this error reporting is the library's own: argument errors the kernel
 * sees and its watchdog, which bounds every wait so that a missing event ends
 * the kernel instead of hanging it, set bits in a device word that this call
 * reports).
 * Returns MK_OK, MK_EDEVICE (token or position out of range was seen; the
 * offending task was skipped), or MK_ETIMEOUT (a wait exceeded the watchdog;
 * every wave left the kernel). After MK_ETIMEOUT the event counters are reset
 * on the next call. */
int mk_check(mk_model *m, void *stream);

/* Watchdog bound for every wait inside the persistent kernel, in
 * milliseconds (default 2000). 0 restores the default. */
int mk_set_watchdog_ms(mk_model *m, int32_t ms);

/* Fault injection for testing the watchdog: the task with global id
 * `task_id` (in every step of later megakernel calls) finishes without adding
 * to its triggering event, so its dependents wait until the watchdog expires
 * and every wave leaves the kernel. -1 disables. MK_EINVAL if out of range. */
int mk_debug_drop_signal(mk_model *m, int32_t task_id);

/* Optional per-task timeline (MPK walk-through 3.3.1: profiler_tensor).
 * d_buf: device buffer of `bytes` bytes receiving, for each executed task of
 * the last megakernel call, 12 x uint64 {t_event, t_staged, t_computed,
 * t_signal, w0, w1, w2, w3, f0, f1, f2, f3} in 100 MHz constant-clock ticks: when its
 * dependent event was seen complete, when its inputs were staged, when its
 * compute finished and when its epilogue finished (just before it counts its
 * triggering event); for a task with weight or KV units, w_s holds stream
 * wave s's start (high 32 bits) and end (low 32 bits) of its piece, as the
 * low 32 bits of the same clock, and f_s when its first item had landed;
 * slot = step * n_tasks + task id. The task's compute unit is the one its queue
 * names. Written only when the buffer holds n_steps * n_tasks slots; NULL
 * disables. MK_EINVAL if bytes is too small for one step. */
int mk_set_profile_buffer(mk_model *m, void *d_buf, size_t bytes);

/* Optional wait accounting of the megakernel's waves (diagnostics). d_buf:
 * zeroed device buffer of at least num_cus * 6 * 16 uint64 words; later
 * megakernel calls add, for workgroup c and wave v, into words
 * [(c * 6 + v) * 16 + j] (times in 100 MHz ticks, j4: the wave's lifetime):
 *   wave 0 (stager):  j0 waiting for a free staging slot, j1 waiting for the
 *                     dependent event, j2 staging, j3 tasks;
 *   wave 1 (retirer): j0 waiting for staging, j1 waiting for the stream
 *                     waves, j2 epilogue, j3 tasks;
 *   waves 2-5 (stream): j0 waiting for a KV step to open, j2 waiting for
 *                     staging, j3 items.
 * NULL disables. */
int mk_set_wait_counters(mk_model *m, void *d_buf, size_t bytes);

/* Facts about a loaded model (each pointer may be NULL):
 *   packed_weight_bytes  device bytes of the packed weight copy (padding
 *                        included);
 *   num_cus, n_tasks     workgroups of the persistent launch, tasks per step;
 *   ring_slots           2 KiB items each stream wave keeps in flight (its
 *                        register ring);
 *   lds_bytes            dynamic LDS per workgroup;
 *   batch_per_launch     the most sequences one launch handles (larger calls
 *                        run in groups of this size).
 * MK_EINVAL for a NULL model. */
int mk_model_info(const mk_model *m, uint64_t *packed_weight_bytes, int32_t *num_cus,
                  int32_t *n_tasks, int32_t *ring_slots, int32_t *lds_bytes,
                  int32_t *batch_per_launch);

void mk_free_model(mk_model *m);

const char *mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */

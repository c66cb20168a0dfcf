/*
 * oda.h -- C ABI of the On-Demand Attention (ODA) decode hot path on MI355X.
 *
 * The method (picx.dev summary of "On-Demand Attention: Language Models Know
 * When to Recall", section "Local-First Decoding"): at decode position t every
 * step first attends the Local access set
 *     S^L_t = {1..min(s,t)} U {max(1,t-w+1)..t}      (s sinks, recent window w)
 * then a recall score q_t decides, on the device, whether the same step is
 * recomputed with Full attention over S^F_t = {1..t}: Full iff q_t > theta
 * (theta = 0 by default); otherwise the Local result is accepted.  Section
 * "Efficient Execution" of the same page names the runtime pieces rebuilt
 * here: a persistent ring KV workspace serving Local, fused KV commits across
 * layers, and GPU-side conditional execution of the Full pass.
 *
 * Conventions for every function below
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *     buffer and the stream; the library keeps no state between calls, never
 *     allocates, never synchronises, and launches only kernels (no memset or
 *     memcpy nodes), so every call may be recorded into a HIP graph.
 *   - Element type of K and V (caches, rings, k_cur/v_cur, k_new/v_new, prefill
 *     sources) is oda_dims.kv_dtype.  Queries are of the same type for bf16
 *     and f32, and bf16 when K/V are FP8 E4M3.  Stored K and V values are
 *     multiplied by oda_dims.k_scale / v_scale (per-tensor dequantisation
 *     scales, any dtype).  Outputs and lse are always f32; accumulation is f32.
 *   - seq_len[b] is the number of committed positions of request b.  During a
 *     step the token being decoded is at position t = seq_len[b] + 1 and its
 *     K/V come from the k_cur/v_cur (or k_new/v_new) arguments, not from the
 *     caches.  seq_len[b] < 0 marks an inactive request slot: no kernel reads
 *     or writes anything for it.
 *   - Host-detectable argument errors return a negative status before any
 *     launch.  Conditions only the device can see (a context beyond the block
 *     table's capacity, a block id outside [0, num_blocks)) skip the affected
 *     request and set a bit in the workspace error word (ODA_DEVERR_*).
 *   - A workspace must not be shared by calls that may run concurrently.
 */
#ifndef ODA_H_
#define ODA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as HIP's hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t* oda_stream;

typedef enum {
  ODA_OK = 0,
  ODA_ERR_INVALID_ARG = -1,  /* a pointer, size or index is wrong            */
  ODA_ERR_UNSUPPORTED = -2,  /* valid but not built (head_dim, group, dtype)  */
  ODA_ERR_HIP = -3,          /* a kernel launch failed                        */
  ODA_ERR_WORKSPACE = -4     /* workspace missing or smaller than required    */
} oda_status;

/* ODA_FP8_E4M3: one byte per element in the OCP OFP8 E4M3 encoding (bias 7,
 * no infinities, largest finite 448).  Quantising the stored KV is the
 * complementary technique of the kongchang.com Declarative Attention page,
 * section "The KV Cache Compression Technology Ecosystem"; the codes are
 * produced by the caller (the projection that makes K/V), the library only
 * stores, moves and dequantises them. */
typedef enum { ODA_BF16 = 0, ODA_F32 = 1, ODA_FP8_E4M3 = 2 } oda_dtype;

/* Layer kinds.  GATED layers have distinct Local (sinks + window, served from
 * the ring) and Full (whole paged cache) access sets.  SLIDING layers (hybrid
 * backbones) read the same recent window in both modes, from their own ring,
 * and keep no paged cache. */
typedef enum { ODA_LAYER_GATED = 0, ODA_LAYER_SLIDING = 1 } oda_layer_kind;

enum { ODA_MAX_LAYERS = 256, ODA_MAX_BATCH = 4096 };

/* Bits of the device error word (first 4 bytes of the workspace).
 * ODA_DEVERR_MERGE_WAIT: in a launch small enough for all its workgroups to be
 * resident at once, the workgroup that merges a (request, KV head) gave up
 * waiting (about a second) for the other splits, e.g. because other work held
 * the compute units; that pass's outputs are not written and the workspace
 * must be prepared again (oda_workspace_init) before further use. */
enum { ODA_DEVERR_CAPACITY = 1, ODA_DEVERR_BLOCK_ID = 2, ODA_DEVERR_OUT_CAPACITY = 4, ODA_DEVERR_MERGE_WAIT = 8 };

/* Accounting counters, int64 per request (see oda_gate). */
enum {
  ODA_ACCT_STEPS = 0,        /* decode steps taken                           */
  ODA_ACCT_FULL_CALLS,       /* steps whose gate fired                       */
  ODA_ACCT_F_LOCAL,          /* sum of F_Local                               */
  ODA_ACCT_F_FULL_TAKEN,     /* sum of a_t * F_Full(t)                       */
  ODA_ACCT_F_FULL_ALWAYS,    /* sum of F_Full(t) (the always-Full cost)      */
  ODA_ACCT_DELTA_F,          /* sum of (1-a_t) F_Full - F_Local - F_Recall   */
  ODA_ACCT_KV_BYTES,         /* K/V bytes the taken passes attend            */
  ODA_ACCT_F_RECALL,         /* sum of F_Recall                              */
  ODA_ACCT_N
};

typedef struct {
  int32_t num_layers;          /* L, 1..ODA_MAX_LAYERS                                   */
  int32_t num_q_heads;         /* Hq                                                     */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0; query head h reads KV head h/(Hq/Hkv);
                                  built for groups Hq/Hkv of 1, 2 and 4, and 8 for
                                  bf16, FP8 and f32 with d = 64 (else ODA_ERR_UNSUPPORTED) */
  int32_t head_dim;            /* d: 64 or 128                                           */
  int32_t sink;                /* s >= 0 of gated layers                                 */
  int32_t window;              /* w >= 1 of gated layers; gated ring has s+w slots       */
  int32_t sw_window;           /* window of sliding layers (>= 1 when any exist)         */
  int32_t block_size;          /* paged block in positions, a power of two (16)          */
  int32_t max_batch;           /* request slots the caches and tables are sized for      */
  int32_t max_blocks_per_seq;  /* columns of block_table                                 */
  int32_t kv_dtype;            /* oda_dtype                                              */
  int32_t focus;               /* 0: a fired gated layer reads S^F_t = {1..t};
                                  1: it reads S^L_t U [a, b) (focus region per request)  */
  int32_t full_splits;         /* split-K partitions per (request, KV head) of a Full
                                  or focus pass; 0 = library default                     */
  int32_t local_splits;        /* same for ring passes; 0 = default                      */
  float   softmax_scale;       /* 0 -> 1/sqrt(head_dim)                                  */
  float   k_scale;             /* K = k_scale * stored value; 0 -> 1                     */
  float   v_scale;             /* V = v_scale * stored value; 0 -> 1                     */
  int32_t reserved0;           /* must be 0                                              */
  int64_t recall_flops;        /* F_Recall charged per request per step (accounting)     */
  const uint8_t* layer_kind;   /* host [num_layers] of oda_layer_kind; NULL = all GATED  */
} oda_dims;

/* Let Lg / Ls be the numbers of gated / sliding layers.  A layer's cache index
 * is its rank among the layers of its kind.  All arrays are dense, row-major. */
typedef struct {
  void* k_cache;               /* [Lg][Hkv][num_blocks][block_size][d]  paged history   */
  void* v_cache;               /*   (position p of request b: block block_table[b][(p-1)/bs],
                                     row (p-1) % bs)                                     */
  void* k_ring;                /* [Lg][max_batch][Hkv][s+w][d]  Local ring workspace     */
  void* v_ring;                /*   slot of position p: p-1 if p <= s, else s+(p-s-1) mod w */
  void* k_swring;              /* [Ls][max_batch][Hkv][sw][d]   sliding-layer rings,     */
  void* v_swring;              /*   slot (p-1) mod sw; NULL when Ls == 0                 */
  int32_t* ring_pos;           /* [max_batch][s+w]  position held by each slot, 0 = none */
  int32_t* swring_pos;         /* [max_batch][sw]   same for sliding rings (NULL if Ls == 0) */
  const int32_t* block_table;  /* [max_batch][max_blocks_per_seq] physical block ids    */
  int32_t* seq_len;            /* [max_batch] committed positions; < 0 = inactive slot   */
  const int64_t* focus_range;  /* [max_batch][2] (a, b): 1-based, half-open; read only
                                  when dims.focus != 0                                   */
  int64_t num_blocks;          /* physical blocks per layer in k_cache / v_cache         */
} oda_kv;

/* Host.  Bytes of workspace the calls below need (the first 256 bytes hold
 * the device error word).  The layout depends on the dims alone: it is sized
 * for any batch up to dims->max_batch, so calls with different batches can
 * share one prepared workspace.  `batch` is only validated.  0 on invalid
 * dims or batch. */
size_t oda_workspace_size(const oda_dims* dims, int32_t batch);

/* Prepares the workspace (small kernels; call once after allocating it): zeroes
 * the error word, the ticket words, the tail-tile counters and the barrier
 * words of the one-launch Full section, and marks every split-partial slot
 * empty.  Between launches the tickets and counters read
 * zero and the slots read empty: each launch's merging workgroup finds the
 * other splits' partials by a ticket (any launch size) or by re-reading slots
 * until none is empty (launches whose workgroups are all resident at once),
 * and leaves all of them as it found them. */
oda_status oda_workspace_init(const oda_dims* dims, int32_t batch, void* workspace,
                              size_t workspace_bytes, oda_stream stream);

/* After prefill: writes positions 1..seq_len[b] of layer `layer` from a dense
 * source [batch][src_rows][Hkv][d] (row p-1 = position p) into the paged cache
 * (gated layer) and into the layer's ring (the slots a one-by-one commit of
 * those positions would leave), and sets ring_pos / swring_pos.  Needs
 * seq_len[b] <= src_rows. */
oda_status oda_prefill_kv(const oda_dims* dims, const oda_kv* kv, int32_t batch, int32_t layer,
                          const void* k_src, const void* v_src, int64_t src_rows,
                          void* workspace, size_t workspace_bytes, oda_stream stream);

/* Rebuilds every gated layer's ring (and ring_pos) from the paged cache for
 * the committed positions 1..seq_len[b].  The ring is the persistent Local KV
 * workspace of the picx.dev summary, section "Efficient Execution"; it holds
 * the s initial positions and the last w positions that S^L_t reads
 * (section "Local-First Decoding", access-set equation). */
oda_status oda_ring_init(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                         void* workspace, size_t workspace_bytes, oda_stream stream);

/* The fused cross-layer KV commit ("Efficient Execution"): one launch writes
 * the token at position t = seq_len[b]+1 of every layer -- k_new/v_new
 * [L][batch][Hkv][d] -- into the paged cache (gated layers) and the ring slot
 * of t (all layers), records t in ring_pos / swring_pos, then sets
 * seq_len[b] = t. */
oda_status oda_commit_kv(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                         const void* k_new, const void* v_new,
                         void* workspace, size_t workspace_bytes, oda_stream stream);

/* The Local pass of one layer for every active request (picx.dev summary,
 * section "Local-First Decoding": every step first runs the Local access mode,
 * F^L over S^L_t; the ring it reads is the one of section "Efficient
 * Execution"): softmax attention of q [batch][Hq][d] over S^L_t (gated layer:
 * sinks + window, from the ring; sliding layer: its window) where position t
 * is k_cur/v_cur [batch][Hkv][d].  Writes out [batch][Hq][d] and lse
 * [batch][Hq] (natural log; nullable). */
oda_status oda_decode_local(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t batch,
                            const void* q, const void* k_cur, const void* v_cur,
                            float* out, float* lse,
                            void* workspace, size_t workspace_bytes, oda_stream stream);

/* The gate plus the Full pass of one layer (picx.dev summary, section
 * "Local-First Decoding": if q_t > theta the step is recomputed with the Full
 * access set S^F_t = {1..t}, otherwise the Local result is accepted; the
 * decision stays on the device as in section "Efficient Execution").  A
 * request fires iff recall_score[b] > theta (strict; NaN never fires;
 * inactive slots never fire).  Fired requests, compacted in ascending order, attend S^F_t
 * (or S^L_t U [a,b) when dims.focus; sliding layers: their window) over the
 * paged cache with position t from k_cur/v_cur, and their rows of out / lse
 * are overwritten; rows of requests that did not fire are left as they are
 * (the accepted Local result).  call_list [batch] (ascending request ids,
 * then -1) and call_count [1] are written when not NULL. */
oda_status oda_decode_full_gated(const oda_dims* dims, const oda_kv* kv, int32_t layer,
                                 int32_t batch, const void* q, const void* k_cur,
                                 const void* v_cur, const float* recall_score, float theta,
                                 float* out, float* lse, int32_t* call_list, int32_t* call_count,
                                 void* workspace, size_t workspace_bytes, oda_stream stream);

/* The gate on its own, with the per-step accounting of the "Computational
 * Savings" section (dF = (1-a) F_Full - F_Local - F_Recall, F = 4*Hq*d per
 * attended position per layer).  Writes call_list / call_count (nullable);
 * adds the decisions to full_calls [batch] and the step's figures to
 * counters [batch][ODA_ACCT_N] (both nullable). */
oda_status oda_gate(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                    const float* recall_score, float theta, int32_t* call_list,
                    int32_t* call_count, int64_t* full_calls, int64_t* counters,
                    oda_stream stream);

/* One whole decode step for every active request, in the order of the
 * picx.dev summary, section "Local-First Decoding" (Local first, then the
 * recall-score gate, then Full only where q_t > theta), run as section
 * "Efficient Execution" describes (device-side conditional Full pass, fused
 * cross-layer KV commit; learnaivisually explainer, runtime paragraph: the
 * recalled step still pays the Local attempt): the Local pass of every layer,
 * the gate (with accounting), the Full pass of every layer for the fired
 * requests, then the fused commit.  When every layer is gated and a layer's
 * Full pass fits the chip in one round of workgroups, the Full passes of all
 * layers are one launch: it ends at once when no request fired, and otherwise
 * runs the layers in order, each after the previous layer's merge (a barrier
 * of the whole grid); otherwise each layer has its own launch.  q_local / q_full
 * [L][batch][Hq][d] (q_full NULL: reuse q_local), k_new / v_new
 * [L][batch][Hkv][d], out [L][batch][Hq][d] (the accepted result), lse
 * [L][batch][Hq] (nullable).  Capture it once into a HIP graph and replay it
 * to run the step without any host round trip. */
oda_status oda_step(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                    const void* q_local, const void* q_full, const void* k_new,
                    const void* v_new, const float* recall_score, float theta,
                    float* out, float* lse, int32_t* call_list, int32_t* call_count,
                    int64_t* full_calls, int64_t* counters,
                    void* workspace, size_t workspace_bytes, oda_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): oda_step
 * with no caller workspace.  Its workspace is a static device array of
 * ODA_STATIC_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends; the call allocates nothing and calls no allocating routine.
 * Returns ODA_ERR_WORKSPACE before any launch when the workspace this dims and
 * batch need (oda_workspace_size) exceed that size.  Every call on a GPU
 * shares that GPU's array and starts with one small kernel that clears the
 * words which must read zero, so calls that may overlap on one GPU (other
 * streams or threads) race and must not be made.  Device-side errors skip the
 * affected request as in oda_step but are not reported (the error word lives
 * in the array).  Every pass merges its split partials by ticket, so outputs
 * may differ from oda_step's in the last bits.  Other arguments and results
 * as for oda_step. */
enum { ODA_STATIC_SCRATCH_BYTES = 4 << 20 };
oda_status oda_step_static(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                           const void* q_local, const void* q_full, const void* k_new,
                           const void* v_new, const float* recall_score, float theta,
                           float* out, float* lse, int32_t* call_list, int32_t* call_count,
                           int64_t* full_calls, int64_t* counters, oda_stream stream);

/* The access sets of the picx.dev summary, section "Local-First Decoding"
 * (S^L_t = {1..min(s,t)} U {max(1,t-w+1)..t}, S^F_t = {1..t}; focus and
 * sliding variants as for oda_decode_full_gated): the positions layer `layer`
 * would attend for request b in the given mode (0 Local, 1 Full) at
 * t = seq_len[b]+1, derived by the same device index code the attention
 * kernels use: *count is set to the set size and the
 * members are written, in no particular order, to positions [capacity].
 * Sets ODA_DEVERR_OUT_CAPACITY if capacity is too small. */
oda_status oda_access_set(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t b,
                          int32_t mode, int32_t* positions, int64_t capacity, int64_t* count,
                          void* workspace, size_t workspace_bytes, oda_stream stream);

/* Input staging for replayed graphs: for i < n copies bytes[i] bytes from
 * src[i] + k*bytes[i] to dst[i], where k = step_counter[0] mod num_steps, then
 * advances step_counter[0] by one.  step_counter points to two device int64:
 * the step index and a word the kernel uses to find its last workgroup (zero
 * before the first call; the kernel leaves it zero).  src, dst and bytes are
 * HOST arrays of n <= 8 entries (their values are baked into the launch); the
 * buffers they point to are device memory and every bytes[i] must be a
 * multiple of 16. */
oda_status oda_stage_step(int32_t n, const void* const* src, void* const* dst,
                          const int64_t* bytes, int64_t* step_counter, int64_t num_steps,
                          oda_stream stream);

/* step_counter[0] += 1 (one tiny kernel). */
oda_status oda_advance_counter(int64_t* step_counter, oda_stream stream);

/* Host.  Host-resident paged history (zhichai.net Declarative Attention page,
 * section "System-2 KV Cache Offloading": KV that the local mode does not
 * need may live in CPU memory and be read only when global attention is
 * declared).  The paged caches of oda_kv may be pinned host memory: only the
 * rings must be in HBM, and the Full pass then reads the history over the host
 * link, only for the requests whose gate fired.  Given a pointer into pinned
 * host memory (hipHostMalloc, or a pinned torch tensor), writes the address at
 * which kernels reach it to *device_ptr; ODA_ERR_INVALID_ARG if the memory is
 * not pinned host memory, ODA_ERR_HIP if the runtime call fails. */
oda_status oda_host_kv_pointer(void* host_ptr, void** device_ptr);

/* Recall-head stand-in.  The recall score is q_t = R_psi(h_{t-1}, E(x_t), h^L_t)
 * (picx.dev summary, "Local-First Decoding"): a small trained module reading
 * the previous hidden state, the current token's embedding and the hidden
 * state the Local pass produced; on Qwen3-1.7B it holds 28,325,889 parameters
 * (learnaivisually explainer, glossary).  The pages do not give its layers;
 * this stand-in is one hidden ReLU layer:
 *     x = [h_{t-1}; E(x_t); h^L_t]   (in_dim values, bf16)
 *     q = w2 . max(W1 x + b1, 0) + b2
 * All pointers are device pointers; the caller owns them. */
typedef struct {
  int32_t in_dim;              /* length of x, a multiple of 8, <= 32768          */
  int32_t hidden;              /* hidden units, >= 1                              */
  const void* w1;              /* bf16 [hidden][in_dim], 16-byte aligned           */
  const float* b1;             /* [hidden]                                        */
  const float* w2;             /* [hidden]                                        */
  float b2;
  int32_t reserved0;           /* must be 0                                       */
} oda_recall_head;

/* Host.  Bytes of the recall head's own workspace for `batch` requests (its
 * per-workgroup partial sums and a ticket word); 0 on invalid arguments. */
size_t oda_recall_workspace_size(const oda_recall_head* head, int32_t batch);

/* Recall scores of `batch` requests: x bf16 [batch][in_dim] (16-byte aligned)
 * -> scores [batch] f32.  One kernel; its last workgroup adds the partial sums.
 * The workspace must be zeroed once after allocation (oda_recall_workspace_init). */
oda_status oda_recall_scores(const oda_recall_head* head, int32_t batch, const void* x, float* scores,
                             void* head_workspace, size_t head_workspace_bytes, oda_stream stream);

/* Zeroes the recall head's workspace (a small kernel). */
oda_status oda_recall_workspace_init(const oda_recall_head* head, int32_t batch, void* head_workspace,
                                     size_t head_workspace_bytes, oda_stream stream);

/* oda_step with the recall score computed on the device between the Local
 * passes and the gate, as "Local-First Decoding" orders them: Local pass of
 * every layer, recall head over head_x [batch][in_dim] (writing recall_score
 * [batch], which the gate then reads), gate, Full pass of every layer for the
 * fired requests, fused commit.  Other arguments as for oda_step. */
oda_status oda_step_recall(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                           const void* q_local, const void* q_full, const void* k_new,
                           const void* v_new, const oda_recall_head* head, const void* head_x,
                           float* recall_score, float theta, float* out, float* lse,
                           int32_t* call_list, int32_t* call_count, int64_t* full_calls,
                           int64_t* counters, void* workspace, size_t workspace_bytes,
                           void* head_workspace, size_t head_workspace_bytes, oda_stream stream);

/* Test support: the failure path of the Local pass's merge.  Runs
 * oda_decode_local's pass (same arguments) with split `withheld_split` of
 * every (request, KV head) leaving without storing its partial, and the
 * merging workgroup giving up after `spin_limit` re-reads of the partial slots
 * instead of about a second's worth.  Every workgroup exits normally; the
 * merging ones find the withheld partial missing, set ODA_DEVERR_MERGE_WAIT
 * in the workspace error word and write no output (a request whose Local set
 * spans fewer than withheld_split + 2 splits merges normally: the withheld
 * split is then its merging split or has no rows).  The workspace must then
 * be prepared again (oda_workspace_init).  Built for bf16 K/V with GQA
 * groups of 1 and 2; ODA_ERR_UNSUPPORTED for other shapes, when the pass
 * would merge by ticket (more workgroups than compute units) or when
 * withheld_split is not below the last split.  Not for production use. */
oda_status oda_test_merge_wait(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t batch,
                               const void* q, const void* k_cur, const void* v_cur, float* out,
                               float* lse, int32_t withheld_split, int32_t spin_limit,
                               void* workspace, size_t workspace_bytes, oda_stream stream);

/* Host.  Human-readable status name. */
const char* oda_status_string(oda_status status);

#ifdef __cplusplus
}
#endif

#endif /* ODA_H_ */

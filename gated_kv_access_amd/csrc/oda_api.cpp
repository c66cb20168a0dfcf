// oda_api.cpp -- the extern "C" entry points declared in include/oda.h:
// argument validation, planning (split counts, workspace carve-up) and the
// order of launches of one decode step.  Validation runs before any HIP call,
// so argument errors are reported on a machine without a GPU.
//
// Step order follows the picx.dev summary of "On-Demand Attention", section
// "Local-First Decoding": Local pass of every layer, then the recall-score
// gate, then (for requests whose score exceeds theta) the Full recomputation
// of every layer; section "Efficient Execution": one fused commit of the new
// token's K/V for all layers.
#include <math.h>
#include <string.h>

#include "oda_internal.h"

using oda::Plan;
using oda::WsLayout;

namespace {

constexpr int32_t kComputeUnits = 256;        // MI355X: one 8-wave workgroup fills a CU
constexpr int32_t kFullRowsPerSplit = 16384;  // beyond this, more rounds of workgroups
constexpr int32_t kMaxSplits = 512;           // bounds the workspace's partials per (request, head)
constexpr int32_t kSplitRowUnit = 16;         // split ranges are whole units of this many rows (kernel side too)

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Validates dims and derives the plan; ODA_OK or the error to return.
oda_status make_plan(const oda_dims* d, Plan* p) {
  if (!d || !p) return ODA_ERR_INVALID_ARG;
  memset(p, 0, sizeof *p);
  if (d->num_layers < 1 || d->num_layers > ODA_MAX_LAYERS) return ODA_ERR_INVALID_ARG;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1) return ODA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return ODA_ERR_INVALID_ARG;
  if (d->head_dim < 1 || d->kv_dtype < ODA_BF16 || d->kv_dtype > ODA_FP8_E4M3) return ODA_ERR_INVALID_ARG;
  if (d->sink < 0 || d->max_batch < 1 || d->max_batch > ODA_MAX_BATCH) return ODA_ERR_INVALID_ARG;
  if (d->full_splits < 0 || d->local_splits < 0 || d->reserved0 != 0) return ODA_ERR_INVALID_ARG;
  if (!(d->softmax_scale >= 0.f) || isinf(d->softmax_scale)) return ODA_ERR_INVALID_ARG;
  if (!(d->k_scale >= 0.f) || isinf(d->k_scale) || !(d->v_scale >= 0.f) || isinf(d->v_scale))
    return ODA_ERR_INVALID_ARG;
  if (d->recall_flops < 0 || (d->focus != 0 && d->focus != 1)) return ODA_ERR_INVALID_ARG;
  p->L = d->num_layers;
  p->Hq = d->num_q_heads;
  p->Hkv = d->num_kv_heads;
  p->D = d->head_dim;
  p->G = d->num_q_heads / d->num_kv_heads;
  p->dtype = d->kv_dtype;
  p->esize = d->kv_dtype == ODA_F32 ? 4 : (d->kv_dtype == ODA_BF16 ? 2 : 1);
  p->q_esize = d->kv_dtype == ODA_F32 ? 4 : 2;
  p->sink = d->sink;
  p->window = d->window;
  p->sw_window = d->sw_window;
  p->focus = d->focus;
  p->max_batch = d->max_batch;
  p->max_blocks = d->max_blocks_per_seq;
  p->block_size = d->block_size;
  p->recall_flops = d->recall_flops;
  int16_t ng = 0, ns = 0;
  for (int l = 0; l < p->L; ++l) {
    const uint8_t k = d->layer_kind ? d->layer_kind[l] : (uint8_t)ODA_LAYER_GATED;
    if (k != ODA_LAYER_GATED && k != ODA_LAYER_SLIDING) return ODA_ERR_INVALID_ARG;
    p->kind[l] = k;
    p->kidx[l] = k == ODA_LAYER_GATED ? ng++ : ns++;
  }
  p->Lg = ng;
  p->Ls = ns;
  if (p->Lg > 0) {
    if (d->window < 1 || !is_pow2(d->block_size) || d->max_blocks_per_seq < 1) return ODA_ERR_INVALID_ARG;
    if ((int64_t)d->max_blocks_per_seq * d->block_size > (int64_t)1 << 30) return ODA_ERR_INVALID_ARG;
    if ((int64_t)d->sink + d->window > (int64_t)1 << 24) return ODA_ERR_INVALID_ARG;
  }
  if (p->Ls > 0 && (d->sw_window < 1 || d->sw_window > (1 << 24))) return ODA_ERR_INVALID_ARG;
  // Built variants: d in {64, 128}, group in {1, 2, 4}; group 8 for bf16 and
  // FP8, and for f32 with d = 64.
  if (p->D != 64 && p->D != 128) return ODA_ERR_UNSUPPORTED;
  if (p->G != 1 && p->G != 2 && p->G != 4 && p->G != 8) return ODA_ERR_UNSUPPORTED;
  if (p->G == 8 && p->dtype == ODA_F32 && p->D != 64) return ODA_ERR_UNSUPPORTED;
  p->ring_slots = p->Lg > 0 ? p->sink + p->window : 0;
  p->block_shift = 0;
  if (p->Lg > 0)
    while ((1 << p->block_shift) < p->block_size) ++p->block_shift;
  const float scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf((float)p->D);
  const float k_scale = d->k_scale > 0.f ? d->k_scale : 1.f;
  p->scale_log2 = scale * k_scale * 1.44269504088896340736f;
  p->v_scale = d->v_scale > 0.f ? d->v_scale : 1.f;
  p->tile_rows = oda::tile_rows_for(p->dtype, p->D, oda::kSrcPaged, p->G);
  return ODA_OK;
}

// Split counts depend only on dims and batch, so the workspace size does too.
void choose_splits(const oda_dims* d, int32_t batch, Plan* p) {
  const int32_t tile = p->tile_rows;
  const int32_t b = batch > 0 ? batch : 1;
  if (p->Lg > 0) {
    const int64_t max_ctx = (int64_t)p->max_blocks * p->block_size;
    const int32_t tiles = ceil_div(max_ctx + 1, tile);  // + 1: the current token is a row too
    int32_t f = d->full_splits;
    if (f <= 0) {
      // Whole rounds of kComputeUnits workgroups: `round` splits per (request,
      // KV head) fill the chip once; long contexts take several rounds so that
      // requests of different lengths balance through dynamic dispatch.
      const int64_t pairs = (int64_t)b * p->Hkv;
      const int32_t round = pairs >= kComputeUnits ? 1 : (int32_t)(kComputeUnits / pairs);
      f = ceil_div(max_ctx, kFullRowsPerSplit);
      f = ceil_div(f, round) * round;
      if (f > tiles) f = tiles;
    }
    const int32_t units = ceil_div(max_ctx + 1, kSplitRowUnit);
    if (f > units) f = units;
    if (f > kMaxSplits) f = kMaxSplits;
    p->full_splits = f < 1 ? 1 : f;
    // Ring passes: a single round of workgroups.  While the (request, KV head)
    // pairs leave the chip unfilled, each pair spreads over ceil(256 / pairs)
    // workgroups, which then hold less than a tile (the kernel skips the empty
    // passes, so each SIMD reduces fewer rows); at larger batches each
    // workgroup takes several tiles, so that no workgroup's fixed cost is paid
    // twice per CU.
    const int32_t runits = ceil_div(p->ring_slots + 1, kSplitRowUnit);
    const int64_t pairs = (int64_t)b * p->Hkv;
    const int32_t round = pairs >= kComputeUnits ? 1 : (int32_t)ceil_div(kComputeUnits, pairs);
    int32_t l = d->local_splits > 0 ? d->local_splits : round;
    if (l > runits) l = runits;
    if (l > kMaxSplits) l = kMaxSplits;
    p->local_splits = l < 1 ? 1 : l;
  }
  if (p->Ls > 0) {
    const int32_t sunits = ceil_div(p->sw_window + 1, kSplitRowUnit);
    const int64_t pairs = (int64_t)b * p->Hkv;
    const int32_t round = pairs >= kComputeUnits ? 1 : (int32_t)ceil_div(kComputeUnits, pairs);
    int32_t s = d->local_splits > 0 ? d->local_splits : round;
    if (s > sunits) s = sunits;
    if (s > kMaxSplits) s = kMaxSplits;
    p->sw_splits = s < 1 ? 1 : s;
  }
}

// Partial-slot rows (request, query head, split) that a call with any batch
// up to max_batch uses.  Below 256 / Hkv requests the split counts change with
// the batch; above it they are constant, so the product grows with the batch.
int64_t max_partial_rows(const oda_dims* d, const Plan& p0) {
  int64_t best = 0;
  auto at = [&](int32_t b) {
    Plan q = p0;
    choose_splits(d, b, &q);
    int32_t ms = q.full_splits;
    if (q.local_splits > ms) ms = q.local_splits;
    if (q.sw_splits > ms) ms = q.sw_splits;
    if ((int64_t)b * ms > best) best = (int64_t)b * ms;
  };
  const int32_t lim = p0.max_batch < 256 ? p0.max_batch : 256;
  for (int32_t b = 1; b <= lim; ++b) at(b);
  at(p0.max_batch);
  return best * p0.Hq;
}

// The workspace layout depends on the dims alone, not on a call's batch: its
// words are sized for max_batch requests and its partial slots for the
// largest set any batch up to max_batch uses, so calls with different batches
// can share one prepared workspace (a slot always lies in the area that was
// marked empty, never on a counter word of another batch's layout).
WsLayout layout(const oda_dims* d, const Plan& p) {
  WsLayout w{};
  const int32_t b = p.max_batch > 0 ? p.max_batch : 1;
  const int64_t rows = max_partial_rows(d, p);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.err_off = 0;
  w.count_off = 4;
  w.list_off = oda::kWsHeader;
  w.order_off = up(w.list_off + sizeof(int32_t) * (size_t)b);
  w.len_off = up(w.order_off + sizeof(int32_t) * (size_t)b);
  w.ticket_off = up(w.len_off + sizeof(int32_t) * (size_t)b);
  w.claim_off = up(w.ticket_off + sizeof(int32_t) * (size_t)b * p.Hkv);
  // one tail-pool counter per (request, KV head), each on its own 256-byte line
  w.commit_ticket_off = up(w.claim_off + sizeof(int32_t) * oda::kCounterStride * (size_t)b * p.Hkv);
  // grid barrier of the one-launch Full section: count, generation, broken flag, a line each
  w.barrier_off = up(w.commit_ticket_off + sizeof(int32_t) * (size_t)b);
  w.part_o_off = up(w.barrier_off + 3 * 256);
  w.part_ml_off = up(w.part_o_off + sizeof(float) * (size_t)rows * p.D);
  const size_t ml_copies = p.D >= 64 ? (size_t)p.D / 64 : 1;  // one (m, l) per merging wave
  w.total = up(w.part_ml_off + sizeof(float) * 2 * ml_copies * (size_t)rows);
  return w;
}

struct Ctx {
  Plan plan;
  WsLayout ws;
  char* base;
  uint32_t* err;
  bool ticket_only = false;  // merge by ticket in every pass (the static scratch holds no empty-slot marks)
};

oda_status prepare(const oda_dims* dims, int32_t batch, void* workspace, size_t ws_bytes, Ctx* c,
                   bool need_ws = true) {
  oda_status st = make_plan(dims, &c->plan);
  if (st != ODA_OK) return st;
  if (batch < 0 || batch > c->plan.max_batch) return ODA_ERR_INVALID_ARG;
  choose_splits(dims, batch, &c->plan);
  c->ws = layout(dims, c->plan);
  if (need_ws) {
    if (!workspace || ws_bytes < c->ws.total) return ODA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return ODA_ERR_WORKSPACE;
  }
  c->base = static_cast<char*>(workspace);
  c->err = workspace ? reinterpret_cast<uint32_t*>(c->base + c->ws.err_off) : nullptr;
  return ODA_OK;
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

oda_status check_kv(const Plan& p, const oda_kv* kv, bool need_gated_cache, bool need_rings) {
  if (!kv || !kv->seq_len) return ODA_ERR_INVALID_ARG;
  if (need_gated_cache && p.Lg > 0) {
    if (!kv->k_cache || !kv->v_cache || !kv->block_table || kv->num_blocks < 1) return ODA_ERR_INVALID_ARG;
    if (!aligned16(kv->k_cache) || !aligned16(kv->v_cache)) return ODA_ERR_INVALID_ARG;
  }
  if (need_rings) {
    if (p.Lg > 0 && (!kv->k_ring || !kv->v_ring || !kv->ring_pos)) return ODA_ERR_INVALID_ARG;
    if (p.Ls > 0 && (!kv->k_swring || !kv->v_swring || !kv->swring_pos)) return ODA_ERR_INVALID_ARG;
    if (p.Lg > 0 && (!aligned16(kv->k_ring) || !aligned16(kv->v_ring))) return ODA_ERR_INVALID_ARG;
    if (p.Ls > 0 && (!aligned16(kv->k_swring) || !aligned16(kv->v_swring))) return ODA_ERR_INVALID_ARG;
  }
  if (p.focus && p.Lg > 0 && !kv->focus_range) return ODA_ERR_INVALID_ARG;
  return ODA_OK;
}

oda_status hip_status(int rc) { return rc == 0 ? ODA_OK : ODA_ERR_HIP; }

// Attention pass of one layer.  gate: kGateAll (Local pass of every active
// request), kGateList (Full pass of the step's compacted list) or kGateBallot
// (Full pass that compacts score > theta itself).
oda::AttnParams make_pass(const Ctx& c, const oda_kv* kv, int32_t layer, int32_t batch, int32_t gate,
                          const void* q, const void* k_cur, const void* v_cur, float* out, float* lse,
                          const int32_t* call_list, const int32_t* call_count, const int32_t* call_len,
                          const float* score, float theta, int32_t* list_out, int32_t* count_out) {
  const Plan& p = c.plan;
  const bool gated = p.kind[layer] == ODA_LAYER_GATED;
  const bool full = gate != oda::kGateAll;
  oda::AttnParams a{};
  a.rows.source = (gated && full) ? oda::kSrcPaged : oda::kSrcRing;
  a.rows.focus = p.focus;
  a.rows.sink = gated ? p.sink : 0;
  a.rows.window = gated ? p.window : p.sw_window;
  a.rows.ring_slots = gated ? p.ring_slots : p.sw_window;
  a.gate_mode = gate;
  a.batch = batch;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.splits = a.rows.source == oda::kSrcPaged ? p.full_splits : (gated ? p.local_splits : p.sw_splits);
  a.max_blocks = p.max_blocks;
  a.block_shift = p.block_shift;
  a.capacity = p.max_blocks * p.block_size;
  a.num_blocks = kv->num_blocks;
  const int64_t row_bytes = (int64_t)p.D * p.esize;
  const int64_t rank = p.kidx[layer];
  if (a.rows.source == oda::kSrcPaged) {
    const int64_t layer_bytes = kv->num_blocks * p.Hkv * p.block_size * row_bytes;
    a.k_base = static_cast<const char*>(kv->k_cache) + rank * layer_bytes;
    a.v_base = static_cast<const char*>(kv->v_cache) + rank * layer_bytes;
  } else {
    const int64_t layer_bytes = (int64_t)p.max_batch * p.Hkv * a.rows.ring_slots * row_bytes;
    a.k_base = static_cast<const char*>(gated ? kv->k_ring : kv->k_swring) + rank * layer_bytes;
    a.v_base = static_cast<const char*>(gated ? kv->v_ring : kv->v_swring) + rank * layer_bytes;
  }
  a.block_table = kv->block_table;
  a.seq_len = kv->seq_len;
  a.focus_range = kv->focus_range;
  a.call_list = call_list;
  a.call_count = call_count;
  a.call_len = call_len;
  a.score = score;
  a.theta = theta;
  a.call_list_out = list_out;
  a.call_count_out = count_out;
  a.q = q;
  a.k_cur = k_cur;
  a.v_cur = v_cur;
  a.out = out;
  a.lse = lse;
  a.part_o = reinterpret_cast<float*>(c.base + c.ws.part_o_off);
  a.part_ml = reinterpret_cast<float*>(c.base + c.ws.part_ml_off);
  a.tickets = reinterpret_cast<int32_t*>(c.base + c.ws.ticket_off);
  // Polling needs every workgroup of the launch resident at once (the merging
  // workgroup waits for the others): one per compute unit at most.  Such a
  // launch also balances its tail through the pool of tail tiles; larger ones
  // already balance through the dispatch of later workgroups.  FP8 passes of
  // GQA groups of 4 and 8 (MFMA) keep static splits: with the pool they measured
  // about 1 us slower per launch at 128K, where it saves 1 us at group 2.
  const bool one_round = (int64_t)a.splits * p.Hkv * batch <= kComputeUnits;
  a.merge_mode = one_round && !c.ticket_only ? oda::kMergePoll : oda::kMergeTicket;
  const bool pool = one_round && !(p.dtype == ODA_FP8_E4M3 && p.G >= 4);
  a.claims = pool ? reinterpret_cast<int32_t*>(c.base + c.ws.claim_off) : nullptr;
  a.err = c.err;
  a.scale_log2 = p.scale_log2;
  a.v_scale = p.v_scale;
  return a;
}

oda_status run_pass(const Ctx& c, const oda_kv* kv, int32_t layer, int32_t batch, int32_t gate,
                    const void* q, const void* k_cur, const void* v_cur, float* out, float* lse,
                    const int32_t* call_list, const int32_t* call_count, const int32_t* call_len,
                    const float* score, float theta, int32_t* list_out, int32_t* count_out,
                    oda_stream s) {
  const oda::AttnParams a = make_pass(c, kv, layer, batch, gate, q, k_cur, v_cur, out, lse, call_list, call_count,
                                      call_len, score, theta, list_out, count_out);
  return hip_status(oda::launch_attention(c.plan, a, batch, s));
}

oda_status check_head(const oda_recall_head* h) {
  if (!h || !h->w1 || !h->b1 || !h->w2 || h->reserved0 != 0) return ODA_ERR_INVALID_ARG;
  if (h->in_dim < 8 || h->in_dim > 32768 || h->in_dim % 8 != 0) return ODA_ERR_INVALID_ARG;
  if (h->hidden < 1 || h->hidden > (1 << 24) || !aligned16(h->w1) || isnan(h->b2)) return ODA_ERR_INVALID_ARG;
  return ODA_OK;
}

oda_status check_head_ws(const oda_recall_head* h, int32_t batch, void* ws, size_t ws_bytes) {
  oda_status st = check_head(h);
  if (st != ODA_OK) return st;
  if (batch < 0 || batch > ODA_MAX_BATCH) return ODA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < oda::recall_workspace_bytes(h->hidden, batch > 0 ? batch : 1)) return ODA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return ODA_ERR_WORKSPACE;
  return ODA_OK;
}

// One decode step: Local pass of every layer; the recall head when one is
// given (writing recall_score); the gate; the Full pass of every layer for the
// fired requests; the fused commit.
oda_status check_step(const Ctx& c, const oda_kv* kv, const void* q_local, const void* q_full,
                      const void* k_new, const void* v_new, const float* recall_score, float theta,
                      const float* out) {
  if (!q_local || !k_new || !v_new || !recall_score || !out || isnan(theta)) return ODA_ERR_INVALID_ARG;
  if (!aligned16(q_local) || (q_full && !aligned16(q_full)) || !aligned16(k_new) || !aligned16(v_new))
    return ODA_ERR_INVALID_ARG;
  return check_kv(c.plan, kv, true, true);
}

oda_status run_step(const Ctx& c, const oda_kv* kv, int32_t batch, const void* q_local, const void* q_full,
                    const void* k_new, const void* v_new, const oda_recall_head* head, const void* head_x,
                    void* head_ws, float* recall_score, float theta, float* out, float* lse,
                    int32_t* call_list, int32_t* call_count, int64_t* full_calls, int64_t* counters,
                    oda_stream stream) {
  oda_status st = check_step(c, kv, q_local, q_full, k_new, v_new, recall_score, theta, out);
  if (st != ODA_OK) return st;
  if (batch == 0) return ODA_OK;
  const Plan& p = c.plan;
  const int64_t q_layer = (int64_t)batch * p.Hq * p.D * p.q_esize;
  const int64_t kv_layer = (int64_t)batch * p.Hkv * p.D * p.esize;
  const int64_t o_layer = (int64_t)batch * p.Hq * p.D;
  const int64_t l_layer = (int64_t)batch * p.Hq;
  const void* qf = q_full ? q_full : q_local;
  auto at = [](const void* base, int64_t off) { return static_cast<const char*>(base) + off; };
  // 1) Local pass, every layer.
  for (int32_t l = 0; l < p.L; ++l) {
    st = run_pass(c, kv, l, batch, oda::kGateAll, at(q_local, l * q_layer), at(k_new, l * kv_layer),
                  at(v_new, l * kv_layer), out + l * o_layer, lse ? lse + l * l_layer : nullptr,
                  nullptr, nullptr, nullptr, nullptr, 0.f, nullptr, nullptr, stream);
    if (st != ODA_OK) return st;
  }
  // 2) Recall score from the decoding state, on the device.
  if (head) {
    if (oda::launch_recall(*head, batch, head_x, recall_score, head_ws, stream)) return ODA_ERR_HIP;
  }
  // 3) Gate: compaction of the fired requests, counters.
  int32_t* list = call_list ? call_list : reinterpret_cast<int32_t*>(c.base + c.ws.list_off);
  int32_t* count = call_count ? call_count : reinterpret_cast<int32_t*>(c.base + c.ws.count_off);
  int32_t* order = reinterpret_cast<int32_t*>(c.base + c.ws.order_off);
  int32_t* lens = reinterpret_cast<int32_t*>(c.base + c.ws.len_off);
  int rc = oda::launch_gate(p, *kv, batch, recall_score, theta, list, count, order, lens, full_calls, counters,
                            stream);
  if (rc) return ODA_ERR_HIP;
  // 4) Full recomputation of every layer for the fired requests, dispatched
  //    longest first.  When every layer is gated and a layer's workgroups fit
  //    the chip at once, the whole section is one launch: nothing runs when
  //    nothing fired, and otherwise the layers follow each other inside it.
  const oda::AttnParams a0 = make_pass(c, kv, 0, batch, oda::kGateList, qf, k_new, v_new, out, lse, order, count,
                                       lens, nullptr, 0.f, nullptr, nullptr);
  const int64_t groups = (int64_t)a0.splits * p.Hkv * batch;
  const int cus = oda::compute_units();
  if (p.Ls == 0 && cus > 0 && groups <= cus && groups <= kComputeUnits) {
    oda::RegionParams r{};
    r.layers = p.L;
    r.groups = (uint32_t)groups;
    r.cache_layer_bytes = kv->num_blocks * p.Hkv * p.block_size * (int64_t)p.D * p.esize;
    r.q_layer_bytes = q_layer;
    r.kv_layer_bytes = kv_layer;
    r.o_layer = o_layer;
    r.l_layer = l_layer;
    r.bar_count = reinterpret_cast<uint32_t*>(c.base + c.ws.barrier_off);
    r.bar_gen = reinterpret_cast<uint32_t*>(c.base + c.ws.barrier_off + 256);
    r.bar_broken = reinterpret_cast<uint32_t*>(c.base + c.ws.barrier_off + 512);
    r.err = c.err;
    if (oda::launch_full_section(p, a0, r, batch, stream)) return ODA_ERR_HIP;
  } else {
    for (int32_t l = 0; l < p.L; ++l) {
      st = run_pass(c, kv, l, batch, oda::kGateList, at(qf, l * q_layer), at(k_new, l * kv_layer),
                    at(v_new, l * kv_layer), out + l * o_layer, lse ? lse + l * l_layer : nullptr,
                    order, count, lens, nullptr, 0.f, nullptr, nullptr, stream);
      if (st != ODA_OK) return st;
    }
  }
  // 5) Fused commit of position t for all layers.
  return hip_status(oda::launch_commit(p, *kv, batch, k_new, v_new,
                                       reinterpret_cast<int32_t*>(c.base + c.ws.commit_ticket_off), c.err, stream));
}

}  // namespace

extern "C" {

size_t oda_workspace_size(const oda_dims* dims, int32_t batch) {
  Ctx c;
  if (prepare(dims, batch, nullptr, 0, &c, false) != ODA_OK) return 0;
  return c.ws.total;
}

oda_status oda_workspace_init(const oda_dims* dims, int32_t batch, void* workspace, size_t bytes,
                              oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, bytes, &c);
  if (st != ODA_OK) return st;
  return hip_status(oda::launch_workspace_init(workspace, c.ws.part_o_off, c.ws.total, stream));
}

oda_status oda_prefill_kv(const oda_dims* dims, const oda_kv* kv, int32_t batch, int32_t layer,
                          const void* k_src, const void* v_src, int64_t src_rows, void* workspace,
                          size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (layer < 0 || layer >= c.plan.L || !k_src || !v_src || src_rows < 0) return ODA_ERR_INVALID_ARG;
  if (!aligned16(k_src) || !aligned16(v_src)) return ODA_ERR_INVALID_ARG;
  const bool gated = c.plan.kind[layer] == ODA_LAYER_GATED;
  st = check_kv(c.plan, kv, gated, true);
  if (st != ODA_OK) return st;
  return hip_status(oda::launch_prefill(c.plan, *kv, batch, layer, k_src, v_src, src_rows, c.err, stream));
}

oda_status oda_ring_init(const oda_dims* dims, const oda_kv* kv, int32_t batch, void* workspace,
                         size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  st = check_kv(c.plan, kv, true, true);
  if (st != ODA_OK) return st;
  return hip_status(oda::launch_ring_init(c.plan, *kv, batch, c.err, stream));
}

oda_status oda_commit_kv(const oda_dims* dims, const oda_kv* kv, int32_t batch, const void* k_new,
                         const void* v_new, void* workspace, size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return ODA_ERR_INVALID_ARG;
  st = check_kv(c.plan, kv, true, true);
  if (st != ODA_OK) return st;
  return hip_status(oda::launch_commit(c.plan, *kv, batch, k_new, v_new,
                                       reinterpret_cast<int32_t*>(c.base + c.ws.commit_ticket_off), c.err, stream));
}

oda_status oda_decode_local(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t batch,
                            const void* q, const void* k_cur, const void* v_cur, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (layer < 0 || layer >= c.plan.L || !q || !k_cur || !v_cur || !out) return ODA_ERR_INVALID_ARG;
  if (!aligned16(q)) return ODA_ERR_INVALID_ARG;
  st = check_kv(c.plan, kv, false, true);
  if (st != ODA_OK) return st;
  return run_pass(c, kv, layer, batch, oda::kGateAll, q, k_cur, v_cur, out, lse, nullptr, nullptr, nullptr,
                  nullptr, 0.f, nullptr, nullptr, stream);
}

oda_status oda_test_merge_wait(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t batch,
                               const void* q, const void* k_cur, const void* v_cur, float* out, float* lse,
                               int32_t withheld_split, int32_t spin_limit, void* workspace,
                               size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (layer < 0 || layer >= c.plan.L || !q || !k_cur || !v_cur || !out) return ODA_ERR_INVALID_ARG;
  if (!aligned16(q) || spin_limit < 0 || withheld_split < 0) return ODA_ERR_INVALID_ARG;
  st = check_kv(c.plan, kv, false, true);
  if (st != ODA_OK) return st;
  if (batch == 0) return ODA_OK;
  const oda::AttnParams a = make_pass(c, kv, layer, batch, oda::kGateAll, q, k_cur, v_cur, out, lse, nullptr,
                                      nullptr, nullptr, nullptr, 0.f, nullptr, nullptr);
  if (a.merge_mode != oda::kMergePoll || withheld_split + 1 >= a.splits) return ODA_ERR_UNSUPPORTED;
  if (c.plan.dtype != ODA_BF16 || c.plan.G > 2) return ODA_ERR_UNSUPPORTED;
  return hip_status(oda::launch_attention_merge_wait(c.plan, a, batch, withheld_split, spin_limit, stream));
}

oda_status oda_decode_full_gated(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t batch,
                                 const void* q, const void* k_cur, const void* v_cur,
                                 const float* recall_score, float theta, float* out, float* lse,
                                 int32_t* call_list, int32_t* call_count, void* workspace,
                                 size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (layer < 0 || layer >= c.plan.L || !q || !k_cur || !v_cur || !out || !recall_score)
    return ODA_ERR_INVALID_ARG;
  if (!aligned16(q) || isnan(theta)) return ODA_ERR_INVALID_ARG;
  const bool gated = c.plan.kind[layer] == ODA_LAYER_GATED;
  st = check_kv(c.plan, kv, gated, !gated);
  if (st != ODA_OK) return st;
  return run_pass(c, kv, layer, batch, oda::kGateBallot, q, k_cur, v_cur, out, lse, nullptr, nullptr,
                  nullptr, recall_score, theta, call_list, call_count, stream);
}

oda_status oda_gate(const oda_dims* dims, const oda_kv* kv, int32_t batch, const float* recall_score,
                    float theta, int32_t* call_list, int32_t* call_count, int64_t* full_calls,
                    int64_t* counters, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, nullptr, 0, &c, false);
  if (st != ODA_OK) return st;
  if (!recall_score || isnan(theta) || !kv || !kv->seq_len) return ODA_ERR_INVALID_ARG;
  if (c.plan.focus && c.plan.Lg > 0 && counters && !kv->focus_range) return ODA_ERR_INVALID_ARG;
  return hip_status(oda::launch_gate(c.plan, *kv, batch, recall_score, theta, call_list, call_count,
                                     nullptr, nullptr, full_calls, counters, stream));
}

oda_status oda_step(const oda_dims* dims, const oda_kv* kv, int32_t batch, const void* q_local,
                    const void* q_full, const void* k_new, const void* v_new,
                    const float* recall_score, float theta, float* out, float* lse,
                    int32_t* call_list, int32_t* call_count, int64_t* full_calls, int64_t* counters,
                    void* workspace, size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (!recall_score) return ODA_ERR_INVALID_ARG;
  return run_step(c, kv, batch, q_local, q_full, k_new, v_new, nullptr, nullptr, nullptr,
                  const_cast<float*>(recall_score), theta, out, lse, call_list, call_count, full_calls, counters,
                  stream);
}

oda_status oda_step_static(const oda_dims* dims, const oda_kv* kv, int32_t batch, const void* q_local,
                           const void* q_full, const void* k_new, const void* v_new,
                           const float* recall_score, float theta, float* out, float* lse,
                           int32_t* call_list, int32_t* call_count, int64_t* full_calls, int64_t* counters,
                           oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, nullptr, 0, &c, false);
  if (st != ODA_OK) return st;
  if (c.ws.total > oda::kStaticScratchBytes) return ODA_ERR_WORKSPACE;
  st = check_step(c, kv, q_local, q_full, k_new, v_new, recall_score, theta, out);
  if (st != ODA_OK) return st;
  if (batch == 0) return ODA_OK;
  void* scr = nullptr;
  if (oda::static_scratch(&scr) != 0) return ODA_ERR_HIP;
  c.base = static_cast<char*>(scr);
  c.err = reinterpret_cast<uint32_t*>(c.base + c.ws.err_off);
  c.ticket_only = true;
  // The scratch keeps whatever the last call on this GPU left: the words that
  // must read zero (error word, call list and count, tickets, tail-tile
  // counters, commit tickets) are cleared by a kernel, not a memset, so the
  // call may be captured into a graph.  Ticket merges read partials only
  // after every split has stored its own, so the partial slots need no
  // preparation.
  if (oda::launch_clear(scr, c.ws.part_o_off, stream)) return ODA_ERR_HIP;
  return run_step(c, kv, batch, q_local, q_full, k_new, v_new, nullptr, nullptr, nullptr,
                  const_cast<float*>(recall_score), theta, out, lse, call_list, call_count, full_calls, counters,
                  stream);
}

size_t oda_recall_workspace_size(const oda_recall_head* head, int32_t batch) {
  if (check_head(head) != ODA_OK || batch < 0 || batch > ODA_MAX_BATCH) return 0;
  return oda::recall_workspace_bytes(head->hidden, batch > 0 ? batch : 1);
}

oda_status oda_recall_workspace_init(const oda_recall_head* head, int32_t batch, void* head_workspace,
                                     size_t head_workspace_bytes, oda_stream stream) {
  oda_status st = check_head_ws(head, batch, head_workspace, head_workspace_bytes);
  if (st != ODA_OK) return st;
  return hip_status(oda::launch_clear(head_workspace, oda_recall_workspace_size(head, batch), stream));
}

oda_status oda_recall_scores(const oda_recall_head* head, int32_t batch, const void* x, float* scores,
                             void* head_workspace, size_t head_workspace_bytes, oda_stream stream) {
  oda_status st = check_head_ws(head, batch, head_workspace, head_workspace_bytes);
  if (st != ODA_OK) return st;
  if (!x || !aligned16(x) || !scores) return ODA_ERR_INVALID_ARG;
  return hip_status(oda::launch_recall(*head, batch, x, scores, head_workspace, stream));
}

oda_status oda_step_recall(const oda_dims* dims, const oda_kv* kv, int32_t batch,
                           const void* q_local, const void* q_full, const void* k_new,
                           const void* v_new, const oda_recall_head* head, const void* head_x,
                           float* recall_score, float theta, float* out, float* lse,
                           int32_t* call_list, int32_t* call_count, int64_t* full_calls,
                           int64_t* counters, void* workspace, size_t workspace_bytes,
                           void* head_workspace, size_t head_workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, batch, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  st = check_head_ws(head, batch, head_workspace, head_workspace_bytes);
  if (st != ODA_OK) return st;
  if (!head_x || !aligned16(head_x) || !recall_score) return ODA_ERR_INVALID_ARG;
  return run_step(c, kv, batch, q_local, q_full, k_new, v_new, head, head_x, head_workspace, recall_score, theta,
                  out, lse, call_list, call_count, full_calls, counters, stream);
}

oda_status oda_access_set(const oda_dims* dims, const oda_kv* kv, int32_t layer, int32_t b,
                          int32_t mode, int32_t* positions, int64_t capacity, int64_t* count,
                          void* workspace, size_t workspace_bytes, oda_stream stream) {
  Ctx c;
  oda_status st = prepare(dims, 0, workspace, workspace_bytes, &c);
  if (st != ODA_OK) return st;
  if (layer < 0 || layer >= c.plan.L || b < 0 || b >= c.plan.max_batch) return ODA_ERR_INVALID_ARG;
  if ((mode != 0 && mode != 1) || !positions || capacity < 1 || !count) return ODA_ERR_INVALID_ARG;
  if (!kv || !kv->seq_len) return ODA_ERR_INVALID_ARG;
  if (c.plan.focus && c.plan.kind[layer] == ODA_LAYER_GATED && mode == 1 && !kv->focus_range)
    return ODA_ERR_INVALID_ARG;
  return hip_status(oda::launch_access_set(c.plan, *kv, layer, b, mode, positions, capacity, count,
                                           c.err, stream));
}

oda_status oda_stage_step(int32_t n, const void* const* src, void* const* dst, const int64_t* bytes,
                          int64_t* step_counter, int64_t num_steps, oda_stream stream) {
  if (n < 1 || n > 8 || !src || !dst || !bytes || !step_counter || num_steps < 1) return ODA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    if (!src[i] || !dst[i] || bytes[i] < 16 || bytes[i] % 16 != 0) return ODA_ERR_INVALID_ARG;
    if (!aligned16(src[i]) || !aligned16(dst[i])) return ODA_ERR_INVALID_ARG;
  }
  return hip_status(oda::launch_stage(n, src, dst, bytes, step_counter, num_steps, stream));
}

oda_status oda_advance_counter(int64_t* step_counter, oda_stream stream) {
  if (!step_counter) return ODA_ERR_INVALID_ARG;
  return hip_status(oda::launch_advance(step_counter, stream));
}

oda_status oda_host_kv_pointer(void* host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr) return ODA_ERR_INVALID_ARG;
  const int rc = oda::host_device_pointer(host_ptr, device_ptr);
  return rc == 0 ? ODA_OK : (rc == 1 ? ODA_ERR_INVALID_ARG : ODA_ERR_HIP);
}

const char* oda_status_string(oda_status status) {
  switch (status) {
    case ODA_OK: return "ODA_OK";
    case ODA_ERR_INVALID_ARG: return "ODA_ERR_INVALID_ARG";
    case ODA_ERR_UNSUPPORTED: return "ODA_ERR_UNSUPPORTED";
    case ODA_ERR_HIP: return "ODA_ERR_HIP";
    case ODA_ERR_WORKSPACE: return "ODA_ERR_WORKSPACE";
  }
  return "ODA_UNKNOWN_STATUS";
}

}  // extern "C"

// oda_internal.h -- plan and kernel-parameter structs shared by the host API
// (oda_api.cpp) and the kernels (oda_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "oda.h"

namespace oda {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 8;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr size_t kWsHeader = 256;  // error word, call count, spare
// Device-scope atomics on words that share a cache line are served one after
// another: counters that many workgroups add to sit this many words apart.
constexpr int32_t kCounterStride = 64;

// Attention passes read their rows either from a ring (Local passes and all
// passes of sliding layers) or from the paged cache (Full / focus passes).
enum Source : int32_t { kSrcRing = 0, kSrcPaged = 1 };

// Everything the host derives once from oda_dims.
struct Plan {
  int32_t L, Hq, Hkv, D, G, dtype, esize, q_esize;  // esize: K/V bytes; q_esize: query bytes
  int32_t sink, window, sw_window, ring_slots;  // ring_slots = sink + window
  int32_t block_size, block_shift, max_batch, max_blocks;
  int32_t focus;
  int32_t Lg, Ls;
  uint8_t kind[ODA_MAX_LAYERS];
  int16_t kidx[ODA_MAX_LAYERS];  // rank of the layer among layers of its kind
  int32_t full_splits, local_splits, sw_splits;
  int32_t tile_rows;  // rows one workgroup consumes per iteration of a paged pass
  float scale_log2;   // softmax scale * k_scale * log2(e)
  float v_scale;
  int64_t recall_flops;
};

// Workspace carve-up for `batch` requests.
struct WsLayout {
  size_t err_off, count_off, list_off, order_off, len_off, ticket_off, claim_off, commit_ticket_off, barrier_off,
      part_o_off, part_ml_off, total;
};

// Which rows a pass scans and how they map to positions.
struct RowSpec {
  int32_t source;        // Source
  int32_t focus;         // paged source only: rows are S^L_t U [a,b) minus t
  int32_t sink, window;  // ring mapping (sliding rings: sink 0, window sw)
  int32_t ring_slots;
};

// Which requests a pass serves.
enum GateMode : int32_t {
  kGateAll = 0,     // every active request (Local passes): blockIdx.z is the request id
  kGateList = 1,    // the compacted list written by the step's gate kernel
  kGateBallot = 2,  // the pass compacts score > theta itself (standalone gated call)
};

// How the workgroup that merges a (request, KV head) is found.
enum MergeMode : int32_t {
  kMergeTicket = 0,  // the last to take a ticket (any launch size)
  kMergePoll = 1,    // the highest split, reading the others' partial slots
                     // until none is empty (every workgroup of the launch
                     // resident at once)
};

// Re-reads of the partial slots the merging workgroup of a polling pass makes
// (about a second) before it gives up.
constexpr int32_t kMergeSpinLimit = 1 << 20;

// One attention pass of one layer: split-K partials, then one workgroup of
// each (request, KV head) merges them.
struct AttnParams {
  RowSpec rows;
  int32_t gate_mode;
  int32_t batch, Hq, Hkv, splits;
  int32_t max_blocks, block_shift, capacity;  // capacity = max_blocks * block_size
  int64_t num_blocks;
  const void* k_base;  // ring of this layer: [max_batch][Hkv][slots][d]; or the cache layer base
  const void* v_base;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* call_list;   // kGateList
  const int32_t* call_count;
  const int32_t* call_len;    // kGateList: committed length of each listed request (same order as call_list)
  const int64_t* focus_range;
  const float* score;         // kGateBallot
  float theta;
  int32_t* call_list_out;     // kGateBallot: optional outputs
  int32_t* call_count_out;
  const void* q;              // [batch][Hq][d]
  const void* k_cur;          // [batch][Hkv][d]  the token at position t
  const void* v_cur;
  float* out;                 // [batch][Hq][d]
  float* lse;                 // [batch][Hq] or NULL
  float* part_o;              // [batch][Hq][splits][d]
  float* part_ml;             // [batch][Hq][splits][d / 64][2]  (one copy per merging wave)
  int32_t* tickets;           // [batch][Hkv], zero between launches
  int32_t* claims;            // [batch][Hkv] x kCounterStride, zero between launches: pool tiles taken
  int32_t merge_mode;         // MergeMode
  uint32_t* err;
  float scale_log2;           // softmax scale * k_scale * log2(e)
  float v_scale;              // applied to the merged output
};

// The Full section of a step in one launch: layer l of `layers` (all gated)
// reads the cache, queries, current token and outputs at l strides from
// those of layer 0 in AttnParams; the layers are separated by a barrier of
// the whole grid.
struct RegionParams {
  int32_t layers;
  uint32_t groups;             // workgroups of the launch
  int64_t cache_layer_bytes;   // paged cache, K and V alike
  int64_t q_layer_bytes;
  int64_t kv_layer_bytes;      // the current token's K / V
  int64_t o_layer, l_layer;    // floats
  uint32_t* bar_count;         // workspace words, each on its own 256-byte line,
  uint32_t* bar_gen;           // zero (count, broken) when the launch starts
  uint32_t* bar_broken;
  uint32_t* err;
};

// Launchers (oda_kernels.hip).  Each returns hipGetLastError() as an int.
int launch_attention(const Plan& p, const AttnParams& a, int32_t batch, oda_stream s);
// A ring pass (bf16, GQA groups 1 and 2) whose split `withheld` stores no
// partial and whose merging workgroups give up after `spin_limit` re-reads:
// the test of the merge's failure path.  Other shapes: hipErrorInvalidValue.
int launch_attention_merge_wait(const Plan& p, const AttnParams& a, int32_t batch, int32_t withheld,
                                int32_t spin_limit, oda_stream s);
int launch_full_section(const Plan& p, const AttnParams& a, const RegionParams& r, int32_t batch, oda_stream s);
// Compute units of the current device (0 if the runtime cannot tell).
int compute_units();
// call_list (ascending; needed when disp_list is given) and call_count are the
// compacted decisions; disp_list / disp_len (nullable) the fired requests and
// their committed lengths in the Full passes' dispatch order (longest first).
int launch_gate(const Plan& p, const oda_kv& kv, int32_t batch, const float* score, float theta,
                int32_t* call_list, int32_t* call_count, int32_t* disp_list, int32_t* disp_len,
                int64_t* full_calls, int64_t* counters, oda_stream s);
int launch_commit(const Plan& p, const oda_kv& kv, int32_t batch, const void* k_new,
                  const void* v_new, int32_t* tickets, uint32_t* err, oda_stream s);
int launch_prefill(const Plan& p, const oda_kv& kv, int32_t batch, int32_t layer,
                   const void* k_src, const void* v_src, int64_t src_rows, uint32_t* err,
                   oda_stream s);
int launch_ring_init(const Plan& p, const oda_kv& kv, int32_t batch, uint32_t* err, oda_stream s);
int launch_access_set(const Plan& p, const oda_kv& kv, int32_t layer, int32_t b, int32_t mode,
                      int32_t* positions, int64_t capacity, int64_t* count, uint32_t* err,
                      oda_stream s);
int launch_clear(void* ptr, size_t bytes, oda_stream s);
// Zeroes workspace bytes [0, partials_off) and marks the split partials at
// [partials_off, total) empty.
int launch_workspace_init(void* ws, size_t partials_off, size_t total, oda_stream s);
int launch_stage(int32_t n, const void* const* src, void* const* dst, const int64_t* bytes,
                 int64_t* counter, int64_t num_steps, oda_stream s);
int launch_advance(int64_t* counter, oda_stream s);
// Recall head: number of workgroups for `hidden` units, the head workspace
// size, and the launch.
int recall_groups(int32_t hidden);
size_t recall_workspace_bytes(int32_t hidden, int32_t batch);
int launch_recall(const oda_recall_head& h, int32_t batch, const void* x, float* scores, void* ws,
                  oda_stream s);
// Device address of pinned host memory: 0, 1 (not pinned host memory) or 2 (runtime error).
int host_device_pointer(void* host_ptr, void** device_ptr);
// Bytes of the static scratch that oda_step_static uses as its workspace.
constexpr size_t kStaticScratchBytes = ODA_STATIC_SCRATCH_BYTES;
// Device address of this GPU's copy of that scratch (taken once per device,
// with the device current): 0, or 1 (no current device) / 2 (runtime error).
int static_scratch(void** ptr);
// Rows per workgroup iteration for the attention kernel built for (dtype, d, source, group).
int tile_rows_for(int32_t dtype, int32_t head_dim, int32_t source, int32_t group);

}  // namespace oda

// Internal kernel-argument structs and launchers of libamdoscar (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oscar {

struct AppendArgs {
  const uint16_t* k_new;   // bf16 [batch][Hkv][128]
  const uint16_t* v_new;
  const int32_t* seq_slot; // nullable
  const int32_t* position; // [batch]
  uint16_t* sink_k; uint16_t* sink_v;
  uint16_t* recent_k; uint16_t* recent_v;
  uint8_t* hist;
  const int32_t* page_table;
  const float* rot_k; const float* rot_v;
  const float* clip_k; const float* clip_v;
  int rot_kv_stride;       // elements from one KV head's R to the next (0: shared)
  int clip_kv_stride;      // likewise for the clip thresholds
  int code_bits;           // 2: INT2 history blocks, 4: INT4
  int hkv;
  int max_pages;
};

struct DemoteArgs {
  const uint16_t* src_k; const uint16_t* src_v;        // bf16 [batch][src_tokens][Hkv][128]
  const float* src_k_f32; const float* src_v_f32;      // or fp32 rotated, same shape
  int src_tokens;     // tokens per batch entry in the source
  int src_tok0;       // source index of the first demoted token
  int n_tokens;       // tokens to demote per entry (when length == nullptr)
  const int32_t* length;      // nullable: count = max(0, length[b] - 320)
  const int32_t* hist_start;  // nullable: 0
  const int32_t* seq_slot;    // nullable
  const float* rot_k; const float* rot_v;
  const float* clip_k; const float* clip_v;
  int rot_kv_stride;  // elements from one KV head's R to the next (0: shared)
  int clip_kv_stride;
  int code_bits;      // 2: INT2 history blocks, 4: INT4
  uint8_t* hist;
  const int32_t* page_table;
  int max_pages;
  int hkv;
  int batch;          // set by the launcher
  int unit_tiles;     // set by the launcher: work units (runs of history pages) per (sequence, KV head)
};

struct PrefillArgs {
  const uint16_t* src_k; const uint16_t* src_v;   // bf16 [batch][max_len][Hkv][128]
  const int32_t* length;
  const int32_t* seq_slot;
  uint16_t* sink_k; uint16_t* sink_v;
  uint16_t* recent_k; uint16_t* recent_v;
  int max_len;
  int hkv;
};

struct DecodeArgs {
  const uint16_t* q;          // bf16 [batch][q_tokens][Hq][128]
  float* out;                 // fp32 [batch][q_tokens][Hq][128]
  const int32_t* seq_slot;    // nullable
  const int32_t* seq_len;     // [batch]; the cached tokens are seq_len[b] + len_offset
  int len_offset;             // 0, or 1 when seq_len holds the step's positions
  const uint16_t* sink_k; const uint16_t* sink_v;
  const uint16_t* recent_k; const uint16_t* recent_v;
  const uint8_t* hist;
  const int32_t* page_table;
  const float* rot_k; const float* rot_v;
  int rot_kv_stride;          // elements from one KV head's R to the next (0: shared)
  const float* clip_k; const float* clip_v;   // the fused step's demotion
  int clip_kv_stride;
  int code_bits;              // 2: INT2 history blocks, 4: INT4
  float* partials;            // workspace: [batch*Hkv][n_splits][G][132]
  int hkv;
  int max_pages;
  int n_hist_splits;          // history splits per (sequence, KV head)
  int pages_per_split;        // a multiple of the wave step (4 pages)
  int n_tile_splits;          // BF16 sink/recent splits per (sequence, KV head)
  int tile_tokens;            // BF16 tokens per tile split (tile_tokens_for(G))
  int tiles_last;             // 1: on each XCD the tile splits after the history splits
  int n_groups_total;         // batch * Hkv * n_colgroups
  int grid_per_xcd;
  // Query columns.  A sequence has q_tokens queries (its last q_tokens
  // positions) and a KV head g_model query heads: q_tokens * g_model
  // "virtual heads" (t, h), numbered t * g_model + h, in n_colgroups groups
  // of G (the kernel's template parameter) columns each.
  int q_tokens;
  int g_model;
  int n_colgroups;
  // nullable (the fused step): the token appended this step, bf16
  // [batch][Hkv][128], not yet in its sink or ring slot.  The tile splits
  // read position n - 1 from here.  From position 320 on, the history split
  // that owns the newest history token demotes the token leaving the ring,
  // writes the new one into its ring slot and attends to the demoted token
  // itself; before that, tile split 0 writes the new token into its slot.
  const uint16_t* k_new; const uint16_t* v_new;
};

struct DecodeBf16Args {
  const uint16_t* q;
  float* out;
  const int32_t* seq_slot;
  const int32_t* seq_len;
  const uint16_t* kv;         // [num_pages][Hkv][2][16][128]
  const int32_t* page_table;
  float* partials;
  int hkv;
  int max_pages;
  int n_splits;
  int pages_per_split;
  int n_groups_total;         // batch * Hkv * n_colgroups
  int q_tokens;               // query columns as in DecodeArgs
  int g_model;
  int n_colgroups;
  int grid_per_xcd;
};

// Log-sum-exp merge of the decode partials, one workgroup per query head.
struct MergeArgs {
  const float* partials;      // [batch*Hkv*n_colgroups][n_splits_total][group][132]
  const int32_t* seq_len;     // [batch]; the cached tokens are seq_len[b] + len_offset
  int len_offset;
  const float* rot;           // R_V for the rotated (history) records; unused when tiered == 0
  int rot_kv_stride;          // elements from one KV head's R_V to the next (0: shared)
  float* out;                 // fp32 [batch][q_tokens][Hq][128]
  int hkv;
  int group;                  // columns per record group
  int q_tokens;               // queries per sequence (virtual heads as in DecodeArgs)
  int g_model;                // query heads per KV head
  int n_colgroups;
  int n_splits_total;         // record slots per (sequence, KV head)
  int n_plain_slots;          // slots before the first rotated record (INT2: tile splits; BF16: all)
  int pages_per_split;
  int tiered;                 // 1: INT2 tiers (plain tile splits + rotated history); 0: BF16 pages
  int tile_tokens;            // INT2 tiers: BF16 tokens per tile split
};

// Decode split geometry, shared by the workspace-size query and the launch.
struct DecodePlan {
  int n_hist_splits;
  int pages_per_split;
  int n_tile_splits;
  int tile_tokens;            // BF16 tokens per tile split
  bool tiles_last;            // more than one round of workgroups: tile splits dispatched last
  int n_splits_total;         // hist + tile
  int n_work;                 // batch * Hkv * n_splits_total
  int grid;                   // padded to a multiple of 8 (one slice per XCD)
  size_t partial_floats;
  size_t workspace_bytes;
  bool ok;                    // false: the context needs more splits than the merge holds
};

// INT2 decode: a history split covers at most this many pages (each of the
// four waves keeps the page ids of its share in one 64-lane register)
constexpr int kMaxPagesPerSplit = 256;

// Workgroups a decode launch may fill with its splits: two per compute unit
// (256 CUs), for oscar_decode and for the fused step alike.  Larger batches
// than this can split exceed it (every group keeps at least one history split).
constexpr int kDecodeSplitTarget = 512;

// group: columns per work item (1, 2, 4, 8 or 16); n_colgroups column groups
// per (sequence, KV head)
DecodePlan plan_decode(int batch, int hkv, int group, int n_colgroups, int max_seq_len,
                       int target = kDecodeSplitTarget);
DecodePlan plan_decode_bf16(int batch, int hkv, int group, int n_colgroups, int max_seq_len);

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t st);
hipError_t launch_demote(const DemoteArgs& a, int batch, int max_count, bool rotated, hipStream_t st);
hipError_t launch_prefill_route(const PrefillArgs& a, int batch, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int group, int grid, hipStream_t st);
hipError_t launch_decode_bf16(const DecodeBf16Args& a, int group, int grid, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, int n_heads, hipStream_t st);

}  // namespace oscar

// Arguments shared by the two block-sparse attention kernels (internal).
#pragma once

#include "common.h"

namespace bsa {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int N, n_valid, nqb, nkb;
  Blocks qb, kb;
  const int32_t* tile_base;   // variable query blocks: [BH][nqb + 1] tile prefix
  const int32_t* order;       // uniform query blocks: [BH][nqb] processing order
  int tiles;                  // tiles per (b, h)
  int bh;                     // B * H
  const int32_t* kv_count;
  const int32_t* kv_index;
  int kv_stride;
  float sl2;                  // scale * log2(e)
  float* lse;                 // null, or [BH][N] natural-log row normaliser of the scaled scores
  // Split over key segments (uniform blocks, long rows): every non-empty
  // (query block I, key segment s) pair is an item; see split_plan_kernel.
  const int32_t* items;       // [BH][max_items][4] {I, list offset, count, s}; per head the
                              // items that are not their query block's last come first
  const int32_t* item_base;   // [BH + 1] prefix of the launch's item counts of the heads in head_order
  const int32_t* item_first;  // null: the launch runs every head's first items; else [BH]
                              // their number, and the launch runs the last item of each query block
  const int32_t* head_order;  // [BH] head at each position of the item sequence
  const int32_t* nseg;        // [BH][nqb] non-empty segments of each query block
  const int32_t* slot_of;     // [BH][nqb][nsegs] item index of (I, s), or -1
  float* part;                // [BH][max_items] partial results (kSplitSlotFloats each)
  int max_items, nsegs;
};

// fp32 words of one partial result of a 64-row tile at d = 128: the O^T
// accumulators of both waves as held in registers, then each lane's reference
// row max (log2 units) and partial row sum.
constexpr int kSplitSlotFloats = 2 * 4 * 16 * 64 + 2 * 2 * 64;

// One-wave kernel (attn_fwd_1w.hip): uniform 64-token blocks, d = 128,
// a.order set; `grid` workgroups of one wave.
hipError_t launch_attn_fwd_1w(const AttnArgs& a, int grid, hipStream_t s);

// Longest-first processing order of n rows per head (attn_fwd.hip): order[bh][i]
// lists the rows by descending count (clamped to [0, cap]). Returns false when
// the counting sort does not fit in LDS (then nothing is launched).
bool launch_qorder(const int32_t* counts, int BH, int n, int cap, int32_t* order, hipStream_t s);

}  // namespace bsa

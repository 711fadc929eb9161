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
};

// One-wave kernel (attn_fwd_1w.hip): uniform 64-token blocks, d = 128,
// a.order set; `grid` workgroups of one wave.
hipError_t launch_attn_fwd_1w(const AttnArgs& a, int grid, hipStream_t s);

// Longest-first processing order of n rows per head (attn_fwd.hip): order[bh][i]
// lists the rows by descending count (clamped to [0, cap]). Returns false when
// the counting sort does not fit in LDS (then nothing is launched).
bool launch_qorder(const int32_t* counts, int BH, int n, int cap, int32_t* order, hipStream_t s);

}  // namespace bsa

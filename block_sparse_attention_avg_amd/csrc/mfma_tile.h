// MFMA tile helpers shared by the attention-gradient, tile-statistics and
// k-means assignment kernels: 64-row bf16 tiles staged in LDS by
// direct-to-LDS buffer loads with XOR-swizzled 16-byte pieces, the row
// operand read, the transposed operand read (LDS transpose read, rows in the
// order of the 32 x 32 accumulator layout), and the accumulator-to-rows
// store.
#pragma once

#include "lds_tile.h"

namespace bsa {
namespace {

// Tile geometry: 64 rows of D bf16, row-major in LDS with swizzled 16-byte
// pieces; the NW waves of a workgroup share its loads (wave w loads rows
// 64w/NW .. 64(w+1)/NW - 1).
template <int D, int NW = 2>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int BYTES = 64 * ROWB;
  static constexpr int NI = BYTES / 1024 / NW;     // direct-to-LDS loads per wave
  static constexpr int RPI = 1024 / ROWB;          // rows per load
  static constexpr int PPR = ROWB / 16;            // 16-byte pieces per row
};

// Lane offsets of a wave's share of a 64-row tile load.
template <int D, int NW = 2>
__device__ __forceinline__ void tile_offsets(int wave, int lane, uint32_t* off) {
  using T = Tile<D, NW>;
#pragma unroll
  for (int i = 0; i < T::NI; ++i) {
    const int r = (wave * T::NI + i) * T::RPI + lane / T::PPR;
    off[i] = r * T::ROWB + (((lane % T::PPR) ^ swz_compact<D>(r & 15)) << 4);
  }
}
// Rows [r0, r0 + n) of a head into `dst`; rows >= n read as zeros. r0 and n
// are the same on every lane: taking them from the first lane keeps the
// descriptor in scalar registers (one the compiler must treat as divergent
// turns every load into a loop over the distinct descriptors).
template <int D, int NW = 2>
__device__ __forceinline__ void tile_load(const uint16_t* head, int r0, int n, lds_u8* dst, int wave,
                                          const uint32_t* off) {
  using T = Tile<D, NW>;
  r0 = __builtin_amdgcn_readfirstlane(r0);
  n = __builtin_amdgcn_readfirstlane(max(n, 0));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head + (size_t)r0 * D, (uint32_t)n * T::ROWB);
#pragma unroll
  for (int i = 0; i < T::NI; ++i) dma16(rs, dst + (wave * T::NI + i) * 1024, off[i]);
}
// Row operand: lane supplies row (32 g + l32), channels 16 c + 8 half .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_read(const lds_u8* t, int g, int c, int l32, int half) {
  const int off = (32 * g + l32) * Tile<D>::ROWB + (((2 * c + half) ^ swz_compact<D>(l32 & 15)) << 4);
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(t + off);
}
// Transposed operand through the LDS transpose read: lane receives channel
// 32 dg + l32 of rows 32 g + 16 hh + (8 t + 4 half + 0..3, t = 0, 1): the row
// order of the accumulator layout (see the forward).
template <int D>
struct TrOffsets {
  // offset of channel group dg = 0, row half t = 0; the others follow from
  // it: channel group dg flips the piece bits 4 dg (byte bits dg << 6), and
  // the row half t = 1 lies 8 rows further, its swizzle differing by the
  // constant swz(8) ^ swz(0)
  int base;
  __device__ __forceinline__ TrOffsets(int lane) {
    const int half = lane >> 5, g16 = (lane >> 4) & 1, sj = (lane & 15) >> 2, sq = lane & 3;
    const int row = 4 * half + sj;
    const int piece = 2 * g16 + (sq >> 1);
    base = row * Tile<D>::ROWB + ((piece ^ swz_compact<D>(row)) << 4) + ((sq & 1) << 3);
  }
  __device__ __forceinline__ int at(int dg, int t) const {
    const int kFlip = (swz_compact<D>(8) ^ swz_compact<D>(0)) << 4;   // rows r and r + 8 (r < 8)
    const int o = base ^ (dg << 6);
    return t ? (o ^ kFlip) + 8 * Tile<D>::ROWB : o;
  }
};
template <int D>
__device__ __forceinline__ bf16x8 tr_read(const lds_u8* t, const TrOffsets<D>& o, int g, int hh, int dg) {
  const lds_u8* b = t + (32 * g + 16 * hh) * Tile<D>::ROWB;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + o.at(dg, 0)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + o.at(dg, 1)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Accumulator element r of a 32 x 32 tile: row 8 (r / 4) + 4 half + (r & 3).
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// 64 x D accumulator tile (transposed: channels x rows, 32 rows per wave) ->
// bf16 rows [r0, r0 + n) of `out`, staged through `stage` (a free tile). All
// NT threads of the workgroup take part; only waves with `active` hold rows
// (row half `wave`).
template <int D, int NT = 128>
__device__ __forceinline__ void store_rows(const f32x16* acc, float mul, lds_u8* stage, uint16_t* out, int r0,
                                           int n, int wave, int lane, bool active = true) {
  using T = Tile<D>;
  const int half = lane >> 5, l32 = lane & 31;
  const int orow = 32 * wave + l32;
  const int fo = swz_compact<D>(orow & 15);
  if (active) {
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const u32x2 w = {pack2(acc[dg][4 * j4 + 0] * mul, acc[dg][4 * j4 + 1] * mul),
                         pack2(acc[dg][4 * j4 + 2] * mul, acc[dg][4 * j4 + 3] * mul)};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
            stage + orow * T::ROWB + (((4 * dg + j4) ^ fo) << 4) + 8 * half) = w;
      }
  }
  wg_barrier();
#pragma unroll
  for (int r = 0; r < T::BYTES / 16 / NT; ++r) {
    const int u = threadIdx.x + NT * r;
    const int row = u / T::PPR, p = u % T::PPR;
    if (row < n)
      *reinterpret_cast<u32x4*>(out + (size_t)(r0 + row) * D + p * 8) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              stage + row * T::ROWB + ((p ^ swz_compact<D>(row & 15)) << 4));
  }
}

}  // namespace
}  // namespace bsa

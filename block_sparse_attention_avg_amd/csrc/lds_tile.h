// LDS tile helpers shared by the gfx950 kernels of libbsa (internal): raw
// buffer descriptors and direct-to-LDS loads, the waits and barriers of the
// load pipelines, the swizzle of 16-byte pieces inside a tile row, bf16
// packing and the reductions over the two halves of a wave.
#pragma once

#include "attn.h"

namespace bsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
// Read-only for the whole kernel: uniform loads through it become scalar loads.
typedef __attribute__((address_space(4))) const int32_t cint;

constexpr float kLog2e = 1.4426950408889634f;

// Swizzle of the 16-byte piece index inside a 64-row tile row (LDS position
// p of row r holds data piece p ^ swz(r)). At d = 128 a row is 256 bytes, one
// full sweep of the 64 four-byte LDS banks, so a piece index is a bank
// group. Row operand reads (16 bytes per lane, 16 lanes per LDS cycle) cover
// 16 consecutive rows at one data piece: swz is a permutation of 0..15 over
// any 16 aligned rows. Transposed reads (8 bytes per lane, 32 lanes per
// cycle) cover 4 consecutive rows x 4 consecutive data pieces: those rows'
// swz values differ in bits 2-3, so the 16 (row, piece) pairs land in 16
// distinct bank groups. Rows r and r + 8 (r < 8) differ by the constant
// swz(8) ^ swz(0), which the transposed-read offsets rely on.
template <int D>
__host__ __device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}
// The layout of the tiles of the gradient, tile-statistics and k-means
// kernels (bits r0, r1, r2, r3 -> 1, 2, 0, 3 at d = 128): also a
// permutation over 16 rows, with rows r and r + 8 differing by 8, but its
// transposed reads meet 2-way conflicts. It stays there because its offset
// arithmetic keeps the gradient kernel's register spills smaller (84 against
// 116 bytes of scratch per lane; 4.25 against 4.70 ms at the 480p layer).
template <int D>
__host__ __device__ __forceinline__ int swz_compact(int r) {
  if constexpr (D == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
  else return (r >> 1) & 7;
}

// Raw buffer descriptor over `bytes` bytes from `base` (gfx9 word 3: 32-bit
// data format); loads at lane offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS (dst is the wave's
// 1 KiB destination; lane l lands at dst + 16 l).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// s_waitcnt lgkmcnt(0) (vmcnt, expcnt unconstrained).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

// Workgroup barrier for the LDS pipelines: this wave's LDS accesses complete
// before it arrives (so no other wave can refill a tile under a read still in
// the LDS queue), compiler-level ordering of memory accesses on both sides,
// but no wait on in-flight direct-to-LDS loads (those are waited explicitly).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t pack2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
}

// max / sum over lanes l and l^32 (the two wave halves hold the same query)
__device__ __forceinline__ float halves_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Per-lane operand reads of the forward's 64-row K and V tiles (row-major,
// 16-byte pieces permuted by swz<D>), shared by its two- and one-wave
// kernels. K operand of S^T = K Q^T: row 32 kb + l32, piece 2 cc + half.
// V^T operand through the transpose read: lane (16-lane group g, slot
// 4 j + q) addresses key row 32 kb + 16 hh + 8 t + 4 half + j, channels
// 32 dg + 16 (g & 1) + 4 q .. +3, so it receives channel 32 dg + l32 of keys
// 32 kb + 16 hh + 8 t + 4 half + 0..3: the P^T slot order.
template <int D>
struct KvOperands {
  static constexpr int ROWB = D * 2;
  int l32, half, fk;
  int voff[D / 32][2];
  __device__ __forceinline__ explicit KvOperands(int lane) {
    l32 = lane & 31;
    half = lane >> 5;
    fk = swz<D>(l32 & 15);
    const int g16 = (lane >> 4) & 1, sj = (lane & 15) >> 2, sq = lane & 3;
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = 8 * t + 4 * half + sj;   // + 32 kb + 16 hh (a multiple of 16)
        const int piece = 4 * dg + 2 * g16 + (sq >> 1);
        voff[dg][t] = row * ROWB + ((piece ^ swz<D>(row & 15)) << 4) + ((sq & 1) << 3);
      }
  }
  // K operand of S^T step j (k-step cc = j / 2, key half kb = j % 2)
  __device__ __forceinline__ bf16x8 k(const lds_u8* Kp, int j) const {
    const int cc = j >> 1, kb = j & 1;
    const int off = (32 * kb + l32) * ROWB + (((2 * cc + half) ^ fk) << 4);
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(Kp + off);
  }
  // V^T operand of PV step j (key half kb, 16-key group hh, channel group dg)
  __device__ __forceinline__ bf16x8 v(const lds_u8* Vp, int j) const {
    const int kb = j / (2 * (D / 32)), hh = (j / (D / 32)) & 1, dg = j % (D / 32);
    const int base = (32 * kb + 16 * hh) * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vp + base + voff[dg][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vp + base + voff[dg][1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

}  // namespace
}  // namespace bsa

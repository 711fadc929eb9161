// Internal helpers shared by the gfx950 kernels of libbsa (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 (raw 16-bit storage) -> fp32: exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Device-side view of a block descriptor (uniform blocks when start == nullptr).
struct Blocks {
  const int32_t* start;
  const int32_t* len;
  int32_t nblocks;
  int32_t per_head;
  int32_t max_len;   // descriptors: 1..64 = no block is longer (caller's bound), else 0
  int32_t block;     // uniform block size
  int32_t n_valid;   // uniform: blocks cover [0, n_valid)

  // The descriptors are read-only while a kernel runs: reading them through
  // the constant address space lets a wave-uniform lookup become a scalar
  // load, which no wait on the vector loads in flight has to cover.
  __device__ __forceinline__ void get(int bh, int i, int& s, int& n) const {
    if (start) {
      typedef __attribute__((address_space(4))) const int32_t c32;
      const size_t o = per_head ? (size_t)bh * nblocks + i : (size_t)i;
      s = ((c32*)start)[o];
      n = ((c32*)len)[o];
    } else {
      s = i * block;
      n = min(block, n_valid - s);
    }
  }
};

// Per-block sizes seen by the select kernel. bias != 0: cluster sizes n_J
// (centroid rule: log n_J added to the logits, per head); bias == 0: block
// lengths (a block with no tokens takes no part). In both, a size <= 0
// excludes a key block and empties a query row.
struct Sizes {
  const int32_t* q;     // null, or [nqb] / [BH][nqb]
  const int32_t* k;     // null, or [nkb] / [BH][nkb]
  int q_per_head, k_per_head;
  int bias;
  __device__ __forceinline__ const int32_t* krow(int bh, int nkb) const {
    return k ? k + (k_per_head ? (size_t)bh * nkb : 0) : nullptr;
  }
  __device__ __forceinline__ bool q_empty(int bh, int nqb, int row) const {
    return q && q[(q_per_head ? (size_t)bh * nqb : 0) + row] <= 0;
  }
};

struct Window {
  int nt, ny, nx, rt, ry, rx;
  int enabled;
  __device__ __forceinline__ bool inside(int I, int J) const {
    const int xI = I % nx, yI = (I / nx) % ny, tI = I / (nx * ny);
    const int xJ = J % nx, yJ = (J / nx) % ny, tJ = J / (nx * ny);
    return abs(tI - tJ) <= rt && abs(yI - yJ) <= ry && abs(xI - xJ) <= rx;
  }
};

// Wave-wide reductions over 64 lanes (values identical in every lane after).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
// Inclusive prefix sum over lanes.
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    unsigned long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Completes this wave's outstanding LDS operations so other lanes of the same
// wave can read what it wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace bsa

// Kernel launchers (defined in the .hip files, called by api.cpp after the
// arguments were validated). They return a hipError_t.
namespace bsa {
hipError_t launch_pool(const uint16_t* x, int BH, int N, int d, const Blocks& blk, float* out,
                       hipStream_t s);
// Q and K pooled in one launch (x1 == nullptr: x0 only).
hipError_t launch_pool2(const uint16_t* x0, const Blocks& blk0, float* out0, const uint16_t* x1,
                        const Blocks& blk1, float* out1, int BH, int N, int d, hipStream_t s);
hipError_t launch_select(const float* qbar, const float* kbar, int BH, int nqb, int nkb, int d,
                         const Sizes& sizes, float thr, float scale,
                         const Window& win, int32_t* kv_count, int32_t* kv_index, int kv_stride,
                         hipStream_t s);
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int BH, int N, int d, int n_valid, const Blocks& qb, const Blocks& kb,
                           const int32_t* kv_count, const int32_t* kv_index, int kv_stride,
                           float scale, int32_t* tile_ws, size_t ws_bytes, float* lse, hipStream_t s);
// Workspace bytes of the forward with every path available (the order table,
// plus the split path's tables and partial results for long uniform rows).
size_t attn_fwd_ws_bytes(int BH, int nqb, int nkb, int d);
hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const uint16_t* dout, const float* lse, int BH, int N, int d, int n_valid,
                           const Blocks& qb, const Blocks& kb, const int32_t* kv_count, const int32_t* kv_index,
                           int kv_stride, float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws,
                           hipStream_t s);
size_t attn_bwd_workspace(int BH, int N, int nqb, int nkb);
hipError_t launch_permute(const uint16_t* x, uint16_t* y, const int32_t* perm, int BH, int N,
                          int d, int per_head, bool inverse, hipStream_t s);
hipError_t launch_tile_stats(const uint16_t* q, const uint16_t* k, const float* lse, int BH, int N, int d,
                             int n_valid, float scale, float* tmax, float* tsum, float* tmin, hipStream_t s);
hipError_t launch_mask_recall(const float* tmax, const float* tsum, const int32_t* kv_count,
                              const int32_t* kv_index, int kv_stride, size_t rows, int nkb, float* oracle_recall,
                              float* mass_recall, hipStream_t s);
hipError_t launch_check_mask(const int32_t* kv_count, const int32_t* kv_index, size_t rows, int nkb, int kv_stride,
                             int32_t* bad, hipStream_t s);
hipError_t launch_kmeans(const uint16_t* x, int BH, int N, int d, int n_valid, int C, int iters,
                         const float* uniforms, float* centroids, int32_t* assign,
                         int32_t* sizes, int32_t* changes, int tol, void* ws, hipStream_t s);
size_t kmeans_ws_bytes(int BH, int N, int C, int d);
hipError_t launch_cluster_order(const int32_t* assign, int BH, int N, int n_valid, int C,
                                int32_t* perm, int32_t* start, int32_t* len, void* ws,
                                hipStream_t s);
size_t cluster_order_ws_bytes(int BH, int N, int C);
}  // namespace bsa

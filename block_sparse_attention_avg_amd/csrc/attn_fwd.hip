// Block-sparse flash-attention forward (NABLA summary, Metodologia section 2,
// "Espansione": only the kept N x N tiles are computed; Sparse VideoGen2
// summary, Metodologia C.2: contiguous queries are computed densely while key
// and value rows of the kept blocks are gathered sparsely, so variable-size
// blocks waste no padding on the key side).
//
// Work item: one 64-row query tile of one head, 2 waves (wave w owns query
// rows 32w..32w+31). The kept key blocks of the tile's query block are walked
// in ascending order as a stream of key rows cut into 64-row chunks; with
// uniform 64-token blocks a chunk is exactly one key block.
//
// Per chunk, K (row-major) and V (transposed to [d][key]) are staged in LDS by
// all 128 threads; the next chunk's global loads are issued before the
// current chunk's math so they overlap it. Each wave then computes
//   S^T = K Q^T           bf16 MFMA 32x32x16, Q^T held in registers as the
//                         B operand for the whole tile,
// which leaves every lane holding 32 key scores of a single query, so the
// online-softmax max/sum are lane-local except for one exchange with the lane
// holding that query's other 32 keys. P^T is rounded to bf16 in registers and
// fed straight back as the B operand of
//   O^T += V^T P^T        bf16 MFMA 32x32x16,
// which works because the transposed V tile is written to LDS with its key
// order permuted to match the accumulator layout of S^T (no shuffles of P).
// The softmax runs in the log2 domain in fp32 (running max m, running sum l);
// O is divided by l once at the end, staged through LDS and stored as bf16
// rows.
#include "common.h"

#include <math.h>

namespace bsa {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int N, n_valid, nqb, nkb;
  Blocks qb, kb;
  const int32_t* tile_base;   // variable query blocks: [BH][nqb + 1] tile prefix
  int tiles;                  // grid tiles per (b, h)
  const int32_t* kv_count;
  const int32_t* kv_index;
  int kv_stride;
  float sl2;                  // scale * log2(e)
};

namespace {

__device__ __forceinline__ uint32_t bf16_of(const uint4& w, int e) {
  const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (e & 1) ? (x >> 16) : (x & 0xffffu);
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  uint4 u;
  u.x = pack_bf16x2(p[0], p[1]);
  u.y = pack_bf16x2(p[2], p[3]);
  u.z = pack_bf16x2(p[4], p[5]);
  u.w = pack_bf16x2(p[6], p[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// Position of key offset o (0..63) inside a transposed V row: within each group
// of 16 keys, offsets (a, g, b) = (bit 3, bit 2, bits 1:0) are stored at
// (g, a, b), which is the order in which a lane of the S^T accumulator holds
// its keys when the accumulator is reused as the PV B operand.
__device__ __forceinline__ int vpos(int o) {
  return (o & ~0xC) | ((o & 4) << 1) | ((o & 8) >> 1);
}

}  // namespace

template <int D, bool QVAR, bool KVAR>
__global__ __launch_bounds__(128) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = D + 8;        // K tile row stride (elements)
  constexpr int VS = 64 + 8;       // V^T tile row stride (elements)
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int NK = 64 * CPR / 128;   // K chunks per thread
  constexpr int NV = 16 * CPR / 128;   // V key-quad units per thread
  __shared__ __align__(16) uint16_t Ks[64 * KS];
  __shared__ __align__(16) uint16_t Vt[D * VS];
  __shared__ int tok[2][64];
  __shared__ int chunk_rows[2];

  // Flat id -> (head, tile): consecutive workgroups are dealt round-robin to
  // the 8 XCDs; remap so each XCD works on a contiguous range of tiles (one or
  // two heads), which keeps a head's K/V hot in that XCD's L2.
  int L = blockIdx.x;
  {
    const int total = gridDim.x, per = total >> 3, rem = total & 7;
    const int x = L & 7, i = L >> 3;
    L = x * per + min(x, rem) + i;
  }
  const int bh = L / a.tiles;
  const int tile = L - bh * a.tiles;

  int I, qs, ql;
  if (!QVAR) {
    I = tile;
    a.qb.get(bh, I, qs, ql);
  } else {
    const int32_t* tb = a.tile_base + (size_t)bh * (a.nqb + 1);
    if (tile >= tb[a.nqb]) return;
    int lo = 0, hi = a.nqb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tb[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    I = lo;
    int s0, n0;
    a.qb.get(bh, I, s0, n0);
    const int sub = tile - tb[I];
    qs = s0 + 64 * sub;
    ql = min(64, n0 - 64 * sub);
  }
  if (ql <= 0) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const size_t head_off = (size_t)bh * a.N * D;
  const uint16_t* qh = a.q + head_off;
  const uint16_t* kh = a.k + head_off;
  const uint16_t* vh = a.v + head_off;

  // Q^T as MFMA B operand: lane supplies Q[row][16c + 8*half .. +7].
  bf16x8 qf[D / 16];
  {
    const int qr = 32 * wave + l32;
    const bool ok = qr < ql;
    const uint16_t* src = qh + (size_t)(qs + (ok ? qr : 0)) * D + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(src + 16 * c) : make_uint4(0, 0, 0, 0);
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dg][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const size_t qrow = (size_t)bh * a.nqb + I;
  const int cnt = a.kv_count[qrow];
  const int32_t* list = a.kv_index + qrow * a.kv_stride;

  uint4 kreg[NK];
  uint4 vreg[NV][4];

  // ---- chunk addressing
  // Uniform: chunk c = key block list[c], rows [64*J, 64*J + kl).
  // Variable: rows come from tok[buf][r] (token index), r < chunk_rows[buf].
  auto load_chunk = [&](int row_base, int kl, const int* tk) {
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const int u = tid + 128 * r;
      const int row = u / CPR, col = u % CPR;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row < kl) {
        const int t = KVAR ? tk[row] : row_base + row;
        w = *reinterpret_cast<const uint4*>(kh + (size_t)t * D + col * 8);
      }
      kreg[r] = w;
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int u = tid + 128 * r;
      const int kq = u / CPR, col = u % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (row < kl) {
          const int t = KVAR ? tk[row] : row_base + row;
          w = *reinterpret_cast<const uint4*>(vh + (size_t)t * D + col * 8);
        }
        vreg[r][e] = w;
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const int u = tid + 128 * r;
      const int row = u / CPR, col = u % CPR;
      *reinterpret_cast<uint4*>(&Ks[row * KS + col * 8]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int u = tid + 128 * r;
      const int kq = u / CPR, col = u % CPR;
      const int pos = vpos(4 * kq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = bf16_of(vreg[r][0], e) | (bf16_of(vreg[r][1], e) << 16);
        w.y = bf16_of(vreg[r][2], e) | (bf16_of(vreg[r][3], e) << 16);
        *reinterpret_cast<uint2*>(&Vt[(col * 8 + e) * VS + pos]) = w;
      }
    }
  };

  auto compute_chunk = [&](int kl) {
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&Ks[(32 * kb + l32) * KS + 16 * c + 8 * half]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], sacc[kb], 0, 0, 0);
      }
    }
    // sacc[kb][r] = S[query 32*wave + l32][key 32kb + 8(r/4) + 4*half + r%4]
    if (kl < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kl) sacc[kb][r] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc * a.sl2);
    const float alpha = exp2f(m_run - m_new);
    float p[2][16];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kb][r] = exp2f(fmaf(sacc[kb][r], a.sl2, -m_new));
        rs += p[kb][r];
      }
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dg][r] *= alpha;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pf[kb][hh] = pack8(&p[kb][8 * hh]);
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              &Vt[(32 * dg + l32) * VS + 32 * kb + 16 * hh + 8 * half]);
          oacc[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kb][hh], oacc[dg], 0, 0, 0);
        }
  };

  if (!KVAR) {
    int kl_next = 0;
    if (cnt > 0) {
      int ks;
      a.kb.get(bh, list[0], ks, kl_next);
      load_chunk(ks, kl_next, nullptr);
    }
    for (int c = 0; c < cnt; ++c) {
      const int kl = kl_next;
      __syncthreads();
      store_chunk();
      __syncthreads();
      if (c + 1 < cnt) {
        int ks;
        a.kb.get(bh, list[c + 1], ks, kl_next);
        load_chunk(ks, kl_next, nullptr);
      }
      compute_chunk(kl);
    }
  } else {
    // Cursor over the stream of kept key rows: list entry e, offset off.
    // Wave 0 produces the token indices of the next chunk into tok[buf].
    int e = 0, off = 0;
    auto next_chunk = [&](int buf) {
      // wave 0 only; skips entries until at least one row is available
      int rows = 0;
      while (rows == 0 && e < cnt) {
        const int ent = e + lane;
        int ks = 0, n = 0;
        if (ent < cnt) a.kb.get(bh, list[ent], ks, n);
        int incl = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        const int total = __shfl(incl, 63);
        rows = min(64, total - off);
        // row `lane` sits at stream position off + lane: first entry with incl > pos
        const int pos = off + lane;
        int lo = 0, hi = 64;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (__shfl(incl, mid & 63) > pos) hi = mid; else lo = mid + 1;
        }
        const int src = lo & 63;
        const int excl_src = __shfl(incl, src) - __shfl(n, src);
        const int ks_src = __shfl(ks, src);
        if (lane < rows) tok[buf][lane] = ks_src + (pos - excl_src);
        // advance the cursor past the rows consumed
        const int pend = off + rows;
        int lo2 = 0, hi2 = 64;
        while (lo2 < hi2) {
          const int mid = (lo2 + hi2) >> 1;
          if (__shfl(incl, mid & 63) > pend) hi2 = mid; else lo2 = mid + 1;
        }
        if (lo2 >= 64) {
          e += 64;
          off = pend - total;
        } else {
          off = pend - (__shfl(incl, lo2) - __shfl(n, lo2));
          e += lo2;
        }
      }
      if (lane == 0) chunk_rows[buf] = rows;
    };
    if (wave == 0) next_chunk(0);
    __syncthreads();
    int buf = 0;
    int kl = chunk_rows[0];
    if (kl > 0) load_chunk(0, kl, tok[0]);
    while (kl > 0) {
      __syncthreads();
      store_chunk();
      if (wave == 0) next_chunk(buf ^ 1);
      __syncthreads();
      const int kl_next = chunk_rows[buf ^ 1];
      if (kl_next > 0) load_chunk(0, kl_next, tok[buf ^ 1]);
      compute_chunk(kl);
      kl = kl_next;
      buf ^= 1;
    }
  }

  // ---- epilogue: O = O^T / l, staged through LDS, stored as bf16 rows
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  __syncthreads();
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      uint2 w;
      w.x = pack_bf16x2(oacc[dg][4 * j4 + 0] * inv, oacc[dg][4 * j4 + 1] * inv);
      w.y = pack_bf16x2(oacc[dg][4 * j4 + 2] * inv, oacc[dg][4 * j4 + 3] * inv);
      *reinterpret_cast<uint2*>(&Ks[(32 * wave + l32) * KS + 32 * dg + 8 * j4 + 4 * half]) = w;
    }
  __syncthreads();
  uint16_t* oh = a.o + head_off;
#pragma unroll
  for (int r = 0; r < NK; ++r) {
    const int u = tid + 128 * r;
    const int row = u / CPR, col = u % CPR;
    if (row < ql)
      *reinterpret_cast<uint4*>(oh + (size_t)(qs + row) * D + col * 8) =
          *reinterpret_cast<const uint4*>(&Ks[row * KS + col * 8]);
  }
}

// Tile prefix over query blocks of any length: tb[bh][I] = sum_{I'<I} ceil(len/64).
__global__ __launch_bounds__(256) void tile_base_kernel(Blocks qb, int32_t* __restrict__ tb) {
  __shared__ int part[256];
  const int bh = blockIdx.x;
  const int n = qb.nblocks;
  const int per = (n + 255) / 256;
  const int i0 = threadIdx.x * per;
  int sum = 0;
  for (int i = i0; i < min(n, i0 + per); ++i) {
    int s, l;
    qb.get(bh, i, s, l);
    sum += (max(l, 0) + 63) / 64;
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int v = part[t];
      part[t] = run;
      run += v;
    }
  }
  __syncthreads();
  int run = part[threadIdx.x];
  int32_t* out = tb + (size_t)bh * (n + 1);
  for (int i = i0; i < min(n, i0 + per); ++i) {
    out[i] = run;
    int s, l;
    qb.get(bh, i, s, l);
    run += (max(l, 0) + 63) / 64;
  }
  if (threadIdx.x == 255) out[n] = run;
}

__global__ __launch_bounds__(256) void zero_rows_kernel(uint4* __restrict__ o, int N, int n_valid,
                                                        int cpr, size_t total) {
  const size_t per_head = (size_t)(N - n_valid) * cpr;
  for (size_t u = blockIdx.x * (size_t)256 + threadIdx.x; u < total; u += (size_t)gridDim.x * 256) {
    const size_t bh = u / per_head, rem = u % per_head;
    o[(bh * N + n_valid) * cpr + rem] = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int BH, int N, int d, int n_valid, const Blocks& qb, const Blocks& kb,
                           const int32_t* kv_count, const int32_t* kv_index, int kv_stride,
                           float scale, int32_t* tile_ws, hipStream_t s) {
  if (BH == 0) return hipSuccess;
  if (n_valid < N) {
    const int cpr = d / 8;
    const size_t total = (size_t)BH * (N - n_valid) * cpr;
    const size_t want = (total + 255) / 256;
    const int grid = (int)(want < 4096 ? want : 4096);
    zero_rows_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<uint4*>(o), N, n_valid, cpr, total);
  }
  if (qb.nblocks == 0) return hipGetLastError();
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.N = N; a.n_valid = n_valid; a.nqb = qb.nblocks; a.nkb = kb.nblocks;
  a.qb = qb; a.kb = kb;
  a.kv_count = kv_count; a.kv_index = kv_index; a.kv_stride = kv_stride;
  a.sl2 = scale * 1.4426950408889634f;
  // Uniform 64-token query blocks need no tiling table; key blocks that are not
  // uniform 64-token blocks are gathered row by row.
  const bool qvar = qb.start != nullptr;
  const bool kvar = kb.start != nullptr;
  a.tile_base = tile_ws;
  if (qvar) {
    tile_base_kernel<<<BH, 256, 0, s>>>(qb, tile_ws);
    a.tiles = (N + 63) / 64 + qb.nblocks;
  } else {
    a.tiles = qb.nblocks;
  }
  const long long grid = (long long)BH * a.tiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
#define BSA_ATTN(DD, QV, KV) attn_fwd_kernel<DD, QV, KV><<<(int)grid, 128, 0, s>>>(a)
  if (d == 128) {
    if (qvar && kvar) BSA_ATTN(128, true, true);
    else if (qvar) BSA_ATTN(128, true, false);
    else if (kvar) BSA_ATTN(128, false, true);
    else BSA_ATTN(128, false, false);
  } else {
    if (qvar && kvar) BSA_ATTN(64, true, true);
    else if (qvar) BSA_ATTN(64, true, false);
    else if (kvar) BSA_ATTN(64, false, true);
    else BSA_ATTN(64, false, false);
  }
#undef BSA_ATTN
  return hipGetLastError();
}

}  // namespace bsa

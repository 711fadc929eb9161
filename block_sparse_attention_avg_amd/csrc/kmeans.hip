// k-means of query / key vectors and the cluster-contiguous order (Sparse
// VideoGen2 summary, Metodologia A, "Clustering" and "Permutazione").
//
// Seeding is k-means++ (each new centre drawn with probability proportional
// to D^2, by inverse CDF over token order with a caller-supplied uniform).
// One launch per seeding round: every workgroup owns 256 tokens, keeps their
// D^2 in a double buffer and publishes its partial sum; at the start of the
// next round one wave of every workgroup re-derives the drawn index from
// those partials with the same fixed-order wave scans (over the chunk
// partials, then over the chosen chunk's D^2; no grid barrier) while the
// other four start reading their token rows; the first workgroup records the
// centre, and all update D^2 against it (centre through scalar loads).
//
// Warm start (Sparse VideoGen2 summary, Metodologia C.1: the previous
// denoising step's centroids initialise k-means): seeding is skipped and the
// Lloyd rounds start from the caller's centroids. Each round counts the tokens
// whose assignment changed (per head, integer atomics, so exact); after the
// first round that moves at most `tol` tokens, every kernel of the later
// rounds of that head returns at once. With tol = 0 that round moved nothing,
// the clustering is a fixed point and the result is bit-identical to running
// the remaining rounds.
//
// Lloyd rounds: assignment on the matrix cores (the nearest centroid by
// |c|^2 - 2 x.c, x.c from an exact three-way bf16 split of the centroids,
// see assign_kernel); the update is a
// stable counting sort by cluster (per-chunk histograms, a per-head scan, an
// in-chunk stable rank) followed by a per-cluster mean over the cluster's
// tokens in ascending token order. Every reduction has a fixed order, so
// results are bit-reproducible. The same sort produces the
// cluster-contiguous permutation.
#include "mfma_tile.h"

#include <math.h>

namespace bsa {

namespace {
constexpr int kChunk = 256;   // tokens per workgroup

struct KmWs {
  float* d2;        // [2][BH][N]
  float* part;      // [2][BH][nchunk]
  int32_t* off;     // [BH][nchunk][C]
  int32_t* order;   // [BH][N]   tokens sorted by cluster
  int32_t* start;   // [BH][C]
  int32_t* size;    // [BH][C]
};

// Early exit of a warm-start round: head bh has stopped when the previous
// round moved at most `tol` tokens (changes[bh][it-1] <= tol).
struct Stop {
  const int32_t* changes;   // null (cold start), or [BH][iters]
  int it, iters, tol;
  __device__ __forceinline__ bool operator()(int bh) const {
    return changes && it >= 1 && changes[(size_t)bh * iters + it - 1] <= tol;
  }
};

__device__ __forceinline__ float load_x(const uint16_t* row, int dd) {
  return __uint_as_float((uint32_t)row[dd] << 16);
}

// Inclusive scan of one value per lane over the wave (fixed order).
__device__ __forceinline__ float wave_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float up = __shfl_up(v, o);
    if (lane >= o) v += up;
  }
  return v;
}

// Inverse-CDF draw of the next centre by one wave: the first token whose
// running sum of D^2 (chunk partials in order, then the chunk's tokens)
// exceeds u * total, every sum a fixed-order wave scan. Rounding can leave
// the target past the last sum: then the last chunk is taken, and in the
// chunk the last token with positive D^2 (the last token if none). With
// no positive D^2 at all the draw is floor(u * n). Every lane returns the
// same token.
__device__ int kpp_draw_wave(const float* pp, const float* d2p, int nchunk, int n, float u) {
  constexpr int kCache = 8;                        // chunk partials held in registers: 512 chunks
  const int lane = threadIdx.x & 63;
  float pv[kCache];
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = 64 * j + lane;
    pv[j] = c < nchunk ? pp[c] : 0.f;
  }
  auto part = [&](int j) {
    const int c = 64 * j + lane;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kCache; ++q)
      if (q == j) v = pv[q];
    return j < kCache ? v : (c < nchunk ? pp[c] : 0.f);
  };
  const int slabs = (nchunk + 63) / 64;
  float total = 0.f;
  for (int j = 0; j < slabs; ++j) total += __shfl(wave_scan(part(j)), 63);
  if (!(total > 0.f)) return min((int)floor((double)u * (double)n), n - 1);
  const float target = u * total;
  int ch = -1;
  float before = 0.f, carry = 0.f, last_before = 0.f;
  for (int j = 0; j < slabs; ++j) {
    const float v = part(j);
    const float incl = wave_scan(v);
    const int c = 64 * j + lane;
    const unsigned long long hit = __ballot(c < nchunk && carry + incl > target);
    if (c == nchunk - 1) last_before = carry + incl - v;
    if (hit) {
      const int f = __builtin_ctzll(hit);
      ch = 64 * j + f;
      before = carry + __shfl(incl - v, f);
      break;
    }
    carry += __shfl(incl, 63);
  }
  if (ch < 0) {
    ch = nchunk - 1;
    before = __shfl(last_before, (nchunk - 1) & 63);
  }
  // the token inside the chunk: four slabs of 64
  float dv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = ch * kChunk + 64 * j + lane;
    dv[j] = i < n ? d2p[i] : 0.f;
  }
  int last_pos = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = ch * kChunk + 64 * j + lane;
    const float incl = wave_scan(dv[j]);
    const unsigned long long hit = __ballot(i < n && before + incl > target);
    if (hit) return ch * kChunk + 64 * j + __builtin_ctzll(hit);
    const unsigned long long pos = __ballot(i < n && dv[j] > 0.f);
    if (pos) last_pos = ch * kChunk + 64 * j + 63 - __builtin_clzll(pos);
    before += __shfl(incl, 63);
  }
  return last_pos >= 0 ? last_pos : min(n, (ch + 1) * kChunk) - 1;
}

}  // namespace

// One seeding round. Five waves per workgroup: waves 0-3 own the chunk's 256
// tokens, wave 4 draws the round's centre from the previous round's D^2. The
// token waves issue the first half of their rows' 16-byte pieces and their
// previous D^2 before the draw is known, so those reads overlap it (each
// wave waits only on its own loads); after the workgroup barrier they read
// the rest of the row and the centre (wave-uniform: scalar loads), update
// D^2 (min with the previous unless first) and sum it over the chunk in a
// fixed order (a butterfly per wave, then the four wave totals). The first
// workgroup records the centre.
template <int D>
__global__ __launch_bounds__(320) void kpp_round_kernel(const uint16_t* __restrict__ x, int N,
                                                        int n, int C, int r,
                                                        const float* __restrict__ uni,
                                                        float* __restrict__ cent, KmWs ws,
                                                        int BH) {
  constexpr int P = D / 8, PH = P / 2;             // 16-byte pieces per row, pieces read early
  __shared__ int sidx;
  __shared__ float wsum[4];
  const int bh = blockIdx.y;
  const int nchunk = gridDim.x;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const uint16_t* xh = x + (size_t)bh * N * D;
  const int prev = (r + 1) & 1, next = r & 1;
  const float* d2p = ws.d2 + ((size_t)prev * BH + bh) * N;
  float* d2n = ws.d2 + ((size_t)next * BH + bh) * N;
  const float* pp = ws.part + ((size_t)prev * BH + bh) * nchunk;
  float* pn = ws.part + ((size_t)next * BH + bh) * nchunk;
  const int i = blockIdx.x * kChunk + t;
  const bool tok = wave < 4 && i < n;

  uint4 xa[P];
  float dprev = 0.f;
  if (wave == 4) {
    const float u = uni[(size_t)bh * C + r];
    const int idx = r == 0 ? min((int)floor((double)u * (double)n), n - 1) : kpp_draw_wave(pp, d2p, nchunk, n, u);
    if (lane == 0) sidx = idx;
  } else if (tok) {
    const uint4* xr = reinterpret_cast<const uint4*>(xh + (size_t)i * D);
#pragma unroll
    for (int k = 0; k < PH; ++k) xa[k] = xr[k];
    if (r > 0) dprev = d2p[i];
  }
  __syncthreads();
  const int cidx = __builtin_amdgcn_readfirstlane(min(max(sidx, 0), n - 1));
  if (blockIdx.x == 0 && t < D)
    cent[((size_t)bh * C + r) * D + t] = load_x(xh + (size_t)cidx * D, t);
  float v = 0.f;
  if (tok) {
    const uint4* xr = reinterpret_cast<const uint4*>(xh + (size_t)i * D);
    const uint4* cr = reinterpret_cast<const uint4*>(xh + (size_t)cidx * D);
#pragma unroll
    for (int k = PH; k < P; ++k) xa[k] = xr[k];
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const uint4 w = xa[k], c = cr[k];
      const uint32_t xs[4] = {w.x, w.y, w.z, w.w}, cs[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t0 = bf16_lo(xs[e]) - bf16_lo(cs[e]);
        const float t1 = bf16_hi(xs[e]) - bf16_hi(cs[e]);
        acc = fmaf(t0, t0, acc);
        acc = fmaf(t1, t1, acc);
      }
    }
    v = r == 0 ? acc : fminf(acc, dprev);
    d2n[i] = v;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  if (lane == 0 && wave < 4) wsum[wave] = v;
  __syncthreads();
  if (t == 0) pn[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// Assignment on the matrix cores. The nearest centroid minimises
// |c|^2 - 2 x.c (|x|^2 is common to all centroids). Tokens are bf16, so each
// x.c is computed exactly up to fp32 accumulation from a three-way bf16 split
// c = c1 + c2 + c3 of the fp32 centroid (each remainder is exact in fp32 and
// the last fits bf16): three bf16 MFMA 32x32x16 products into one fp32
// accumulator, smallest part first.
//
// A workgroup of 4 waves owns 256 tokens, 64 per wave as two 32-token groups
// whose rows stay in registers as the B operand. Centroids go through LDS in
// chunks of 32: the workgroup reads the fp32 rows, splits them, stores the
// three bf16 parts in swizzled 32-row tiles and |c|^2 (fixed-order sums, the
// same in every workgroup); the parts are the A operand, shared by both
// token groups. A lane holds 16 centroid scores of one token; it keeps the
// first minimum in centroid order, and the two lane halves merge at the end
// (equal scores go to the lower index). Three waves per SIMD (at most 168
// registers; left alone the compiler takes 154 + 32 accumulation registers
// and fits two).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void assign_kernel(const uint16_t* __restrict__ x, int N, int n,
                                                     int C, const float* __restrict__ cent,
                                                     int32_t* __restrict__ assign, Stop stop,
                                                     int32_t* __restrict__ changes) {
  constexpr int ROWB = D * 2, PART = 32 * ROWB;
  constexpr int CPT = D / 8;                       // channels per thread in the chunk load
  __shared__ __align__(16) unsigned char parts[3 * PART];
  __shared__ __align__(16) float nrm[32];
  const int bh = blockIdx.y;
  if (stop(bh)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * kChunk + 64 * wave;

  bf16x8 xf[2][D / 16];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int i = tok0 + 32 * g + l32;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      xf[g][c] = i < n ? *reinterpret_cast<const bf16x8*>(x + ((size_t)bh * N + i) * D + 16 * c + 8 * half)
                       : bf16x8{};
  }

  // chunk loader: thread t takes centroid row t / 8, channels CPT * (t % 8) ..
  const int lr = tid >> 3, ls = tid & 7;
  const float* cb = cent + (size_t)bh * C * D;
  float cv[CPT];
  auto fetch = [&](int c0) {
    const bool ok = c0 + lr < C;
    const float4* src = reinterpret_cast<const float4*>(cb + (size_t)(ok ? c0 + lr : 0) * D + CPT * ls);
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) {
      const float4 w = ok ? src[j] : float4{0.f, 0.f, 0.f, 0.f};
      cv[4 * j + 0] = w.x; cv[4 * j + 1] = w.y; cv[4 * j + 2] = w.z; cv[4 * j + 3] = w.w;
    }
  };
  auto stage = [&](int c0) {
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) sq = fmaf(cv[j], cv[j], sq);
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    sq += __shfl_xor(sq, 4);
    if (ls == 0) nrm[lr] = c0 + lr < C ? sq : INFINITY;
#pragma unroll
    for (int pc = 0; pc < CPT / 8; ++pc) {
      u32x4 w[3];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r0 = cv[8 * pc + 2 * e], r1 = cv[8 * pc + 2 * e + 1];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const uint32_t b = pack2(r0, r1);
          w[p][e] = b;
          r0 -= __uint_as_float(b << 16);
          r1 -= __uint_as_float(b & 0xffff0000u);
        }
      }
      const int piece = (CPT / 8) * ls + pc;
      const int off = lr * ROWB + ((piece ^ swz_compact<D>(lr & 15)) << 4);
#pragma unroll
      for (int p = 0; p < 3; ++p)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((lds_u8*)parts + p * PART + off) = w[p];
    }
  };

  float best[2] = {INFINITY, INFINITY};
  int bi[2] = {0, 0};
  fetch(0);
  for (int c0 = 0; c0 < C; c0 += 32) {
    __syncthreads();                               // the previous chunk's reads are done
    stage(c0);
    __syncthreads();
    if (c0 + 32 < C) fetch(c0 + 32);
    f32x16 acc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[g][r] = 0.f;
#pragma unroll
    for (int p = 2; p >= 0; --p)
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 a = row_read<D>((const lds_u8*)parts + p * PART, 0, c, l32, half);
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[g][c], acc[g], 0, 0, 0);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 nr = *reinterpret_cast<const float4*>(nrm + 8 * j + 4 * half);
      const float nv[4] = {nr.x, nr.y, nr.z, nr.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float sc = fmaf(-2.f, acc[g][4 * j + e], nv[e]);
          if (sc < best[g]) { best[g] = sc; bi[g] = c0 + 8 * j + 4 * half + e; }
        }
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ob = __shfl_xor(best[g], 32);
    const int oi = __shfl_xor(bi[g], 32);
    if (ob < best[g] || (ob == best[g] && oi < bi[g])) bi[g] = oi;
    const int i = tok0 + 32 * g + l32;
    if (half == 0 && i < N) {
      int32_t* dst = assign + (size_t)bh * N + i;
      if (i >= n) {
        *dst = -1;
        continue;
      }
      // rounds after the first count the tokens that moved
      if (changes && stop.it >= 1 && *dst != bi[g]) atomicAdd(&changes[(size_t)bh * stop.iters + stop.it], 1);
      *dst = bi[g];
    }
  }
}

// changes[bh][0] = n (no earlier round to compare with), the rest 0.
__global__ __launch_bounds__(256) void changes_init_kernel(int32_t* __restrict__ changes, size_t total, int iters,
                                                           int n) {
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (size_t)gridDim.x * 256)
    changes[u] = u % (size_t)iters == 0 ? n : 0;
}

// Per-chunk cluster histogram: cnt[bh][chunk][c].
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ assign, int N, int n,
                                                   int C, int32_t* __restrict__ cnt, Stop stop) {
  extern __shared__ int h[];
  const int bh = blockIdx.y, ch = blockIdx.x, nchunk = gridDim.x;
  if (stop(bh)) return;
  for (int c = threadIdx.x; c < C; c += 256) h[c] = 0;
  __syncthreads();
  const int i = ch * kChunk + threadIdx.x;
  if (i < n) atomicAdd(&h[assign[(size_t)bh * N + i]], 1);
  __syncthreads();
  int32_t* out = cnt + ((size_t)bh * nchunk + ch) * C;
  for (int c = threadIdx.x; c < C; c += 256) out[c] = h[c];
}

// Per head: running offsets over chunks for every cluster, cluster sizes and
// starts; off[bh][chunk][c] becomes the first output slot of chunk's members.
// Thread c walks cluster c's column in batches of 16 loads (so their
// latencies overlap); the starts are an exclusive scan of the sizes over the
// workgroup (integer sums: exact in any order).
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ off, int nchunk, int C,
                                                    int32_t* __restrict__ start,
                                                    int32_t* __restrict__ size, Stop stop) {
  constexpr int kB = 16;
  __shared__ int wsum[16];
  const int bh = blockIdx.x;
  if (stop(bh)) return;
  const int c = threadIdx.x, lane = c & 63, w = c >> 6;
  int32_t* o = off + (size_t)bh * nchunk * C;
  int run = 0;
  if (c < C)
    for (int ch0 = 0; ch0 < nchunk; ch0 += kB) {
      int t[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) t[j] = ch0 + j < nchunk ? o[(size_t)(ch0 + j) * C + c] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) run += t[j];
    }
  int incl = c < C ? run : 0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int st = incl - (c < C ? run : 0);
  for (int j = 0; j < w; ++j) st += wsum[j];
  if (c < C) {
    start[(size_t)bh * C + c] = st;
    size[(size_t)bh * C + c] = run;
    int acc = st;
    for (int ch0 = 0; ch0 < nchunk; ch0 += kB) {
      int t[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) t[j] = ch0 + j < nchunk ? o[(size_t)(ch0 + j) * C + c] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (ch0 + j < nchunk) {
          o[(size_t)(ch0 + j) * C + c] = acc;
          acc += t[j];
        }
    }
  }
}

// Stable scatter: token i goes to off[chunk][a_i] + (# earlier tokens of the
// chunk in the same cluster). Rows >= n map to themselves.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ assign, int N,
                                                      int n, int C,
                                                      const int32_t* __restrict__ off,
                                                      int32_t* __restrict__ order, Stop stop) {
  __shared__ int ids[kChunk];
  const int bh = blockIdx.y, ch = blockIdx.x, nchunk = gridDim.x;
  if (stop(bh)) return;
  const int i = ch * kChunk + threadIdx.x;
  ids[threadIdx.x] = i < n ? assign[(size_t)bh * N + i] : -1;
  __syncthreads();
  if (i < n) {
    const int a = ids[threadIdx.x];
    int rank = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) rank += ids[j] == a;
    order[(size_t)bh * N + off[((size_t)bh * nchunk + ch) * C + a] + rank] = i;
  }
  // padding rows (and the tail beyond the last chunk) map to themselves
  for (int t = n + ch * kChunk + threadIdx.x; t < N; t += kChunk * nchunk)
    order[(size_t)bh * N + t] = t;
}

// Cluster means: token p of a cluster (ascending token order) goes to group
// p % G; each group reads its tokens' rows in 16-byte pieces (D / 8 threads
// per row), and the groups are combined in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void mean_kernel(const uint16_t* __restrict__ x, int N, int C,
                                                   const int32_t* __restrict__ order,
                                                   const int32_t* __restrict__ start,
                                                   const int32_t* __restrict__ size,
                                                   float* __restrict__ cent, Stop stop) {
  constexpr int TPR = D / 8;     // threads per token row
  constexpr int G = 256 / TPR;   // token groups
  __shared__ float red[G][D];
  const int bh = blockIdx.y, c = blockIdx.x;
  if (stop(bh)) return;
  const int sz = size[(size_t)bh * C + c];
  if (sz == 0) return;   // empty cluster keeps its centroid
  const int st = start[(size_t)bh * C + c];
  const int pc = threadIdx.x % TPR, g = threadIdx.x / TPR;
  const int32_t* ord = order + (size_t)bh * N + st;
  const uint16_t* xh = x + (size_t)bh * N * D + 8 * pc;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(ws[e]);
      acc[2 * e + 1] += bf16_hi(ws[e]);
    }
  };
  int p = g;
  for (; p + 3 * G < sz; p += 4 * G) {
    const int i0 = ord[p], i1 = ord[p + G], i2 = ord[p + 2 * G], i3 = ord[p + 3 * G];
    const uint4 w0 = *reinterpret_cast<const uint4*>(xh + (size_t)i0 * D);
    const uint4 w1 = *reinterpret_cast<const uint4*>(xh + (size_t)i1 * D);
    const uint4 w2 = *reinterpret_cast<const uint4*>(xh + (size_t)i2 * D);
    const uint4 w3 = *reinterpret_cast<const uint4*>(xh + (size_t)i3 * D);
    add(w0); add(w1); add(w2); add(w3);
  }
  for (; p < sz; p += G) add(*reinterpret_cast<const uint4*>(xh + (size_t)ord[p] * D));
#pragma unroll
  for (int e = 0; e < 8; ++e) red[g][8 * pc + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int dd = threadIdx.x;
    float s = red[0][dd];
    for (int k = 1; k < G; ++k) s += red[k][dd];
    cent[((size_t)bh * C + c) * D + dd] = s / (float)sz;
  }
}

static KmWs carve(void* ws, int BH, int N, int C) {
  const int nchunk = (N + kChunk - 1) / kChunk;
  char* p = reinterpret_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += (bytes + 255) & ~(size_t)255;
    return r;
  };
  KmWs w;
  w.d2 = reinterpret_cast<float*>(take(sizeof(float) * 2 * (size_t)BH * N));
  w.part = reinterpret_cast<float*>(take(sizeof(float) * 2 * (size_t)BH * nchunk));
  w.off = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * nchunk * C));
  w.order = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * N));
  w.start = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * C));
  w.size = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * C));
  return w;
}

size_t kmeans_ws_bytes(int BH, int N, int C, int /*d*/) {
  const int nchunk = (N + kChunk - 1) / kChunk;
  auto r = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return r(sizeof(float) * 2 * (size_t)BH * N) + r(sizeof(float) * 2 * (size_t)BH * nchunk) +
         r(sizeof(int32_t) * (size_t)BH * nchunk * C) + r(sizeof(int32_t) * (size_t)BH * N) +
         2 * r(sizeof(int32_t) * (size_t)BH * C);
}

size_t cluster_order_ws_bytes(int BH, int N, int C) {
  const int nchunk = (N + kChunk - 1) / kChunk;
  return ((sizeof(int32_t) * (size_t)BH * nchunk * C) + 255) & ~(size_t)255;
}

static hipError_t sort_by_cluster(const int32_t* assign, int BH, int N, int n, int C, int32_t* off,
                                  int32_t* order, int32_t* start, int32_t* size, hipStream_t s,
                                  Stop stop = Stop{nullptr, 0, 0, 0}) {
  const int nchunk = (N + kChunk - 1) / kChunk;
  hist_kernel<<<dim3(nchunk, BH), 256, C * sizeof(int), s>>>(assign, N, n, C, off, stop);
  scan_kernel<<<BH, 1024, 0, s>>>(off, nchunk, C, start, size, stop);
  scatter_kernel<<<dim3(nchunk, BH), 256, 0, s>>>(assign, N, n, C, off, order, stop);
  return hipGetLastError();
}

// uni != null: k-means++ seeding into cent first (cold start); otherwise cent
// holds the initial centroids and changes ([BH][iters], iters >= 1) receives
// the per-round move counts (warm start with early exit).
template <int D>
static hipError_t kmeans_t(const uint16_t* x, int BH, int N, int n, int C, int iters,
                           const float* uni, float* cent, int32_t* assign, int32_t* sizes,
                           int32_t* changes, int tol, void* wsp, hipStream_t s) {
  KmWs ws = carve(wsp, BH, N, C);
  const int nchunk_n = (n + kChunk - 1) / kChunk;
  if (uni)
    for (int r = 0; r < C; ++r)
      kpp_round_kernel<D><<<dim3(nchunk_n, BH), 320, 0, s>>>(x, N, n, C, r, uni, cent, ws, BH);
  if (changes && iters > 0) {
    const size_t total = (size_t)BH * iters;
    changes_init_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(changes, total, iters, n);
  }
  const int nchunk = (N + kChunk - 1) / kChunk;
  for (int it = 0; it < iters; ++it) {
    const Stop stop{changes, it, iters, tol};
    assign_kernel<D><<<dim3(nchunk, BH), 256, 0, s>>>(x, N, n, C, cent, assign, stop, changes);
    hipError_t e = sort_by_cluster(assign, BH, N, n, C, ws.off, ws.order, ws.start, ws.size, s, stop);
    if (e != hipSuccess) return e;
    mean_kernel<D><<<dim3(C, BH), 256, 0, s>>>(x, N, C, ws.order, ws.start, ws.size, cent, stop);
  }
  if (iters == 0) {
    const Stop none{nullptr, 0, 0, 0};
    assign_kernel<D><<<dim3(nchunk, BH), 256, 0, s>>>(x, N, n, C, cent, assign, none, nullptr);
    hipError_t e = sort_by_cluster(assign, BH, N, n, C, ws.off, ws.order, ws.start, ws.size, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipMemcpyAsync(sizes, ws.size, sizeof(int32_t) * (size_t)BH * C,
                                hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_kmeans(const uint16_t* x, int BH, int N, int d, int n_valid, int C, int iters,
                         const float* uniforms, float* centroids, int32_t* assign,
                         int32_t* sizes, int32_t* changes, int tol, void* ws, hipStream_t s) {
  if (BH == 0) return hipSuccess;
  if (d == 128)
    return kmeans_t<128>(x, BH, N, n_valid, C, iters, uniforms, centroids, assign, sizes, changes, tol, ws, s);
  return kmeans_t<64>(x, BH, N, n_valid, C, iters, uniforms, centroids, assign, sizes, changes, tol, ws, s);
}

hipError_t launch_cluster_order(const int32_t* assign, int BH, int N, int n_valid, int C,
                                int32_t* perm, int32_t* start, int32_t* len, void* ws,
                                hipStream_t s) {
  if (BH == 0) return hipSuccess;
  return sort_by_cluster(assign, BH, N, n_valid, C, reinterpret_cast<int32_t*>(ws), perm, start,
                         len, s);
}

}  // namespace bsa

// Reduced attention + CDF selection of key blocks (NABLA summary, Metodologia
// section 2, "Attenzione Ridotta" and "CDF Thresholding"; section 3 for the
// window union; Sparse VideoGen2 summary, Metodologia B for the
// size-weighted centroid variant).
//
// One workgroup (4 waves) owns R consecutive rows of one head's reduced map.
//
// Phase 1 -- scores. s[r][J] = scale * qbar_r . kbar_J (+ log n_J) for all
// key blocks, on fp32 MFMA 16x16x4 (A = 16 pooled query rows, B = 16 pooled
// key rows, the 4-wide k slot of the MFMA split over the four 16-lane groups
// so each lane streams a contiguous quarter of the channel vector). The R x nkb
// fp32 score rows stay in LDS; the reduced map never touches HBM.
//
// Phase 2 -- selection, one wave per row (rows of up to 2048 key blocks are
// held in registers, longer rows are streamed from LDS). p_J = exp(s_J - max)
// in fp32.
// Masses are converted to 2^-31 fixed point (m_J = floor(p_J * 2^31)) so that
// every sum is exact and order-independent. The cut is found by an MSB-first
// radix select over the 43-bit key (bits(p_J) << 13 | (8191 - J)): keys order
// blocks lightest first with ties broken toward the higher index. Each 8-bit
// digit pass builds a 256-bin mass histogram of the keys still matching the
// prefix (LDS 64-bit integer atomics, order-independent), scans it and
// descends into the first bin where the cumulative mass reaches
// T = ceil(thr * Z). After 6 passes k* is the smallest key whose inclusive
// cumulative mass reaches T: exactly the blocks with key < k* are dropped.
// The kept ids are written in ascending order with wave ballots; the window
// test, if any, is OR'd in at that point.
#include "common.h"

#include <math.h>

namespace bsa {

namespace {
constexpr int kIdxBits = 13;          // supports nkb <= 8192
constexpr int kKeyBits = 30 + kIdxBits;
constexpr int kDigit = 8;
constexpr int kPasses = (kKeyBits + kDigit - 1) / kDigit;   // 6
constexpr int kBins = 1 << kDigit;
constexpr int kSelWaves = 4;          // waves per workgroup
constexpr float kMassScale = 0x1p31f; // block masses in 2^-31 fixed point
constexpr int kHist = 512;           // histogram words per wave
constexpr int kDigit0 = 192;          // first-digit value of p = 2^-31 (bits(p) >> 22)
}  // namespace

// Selection of one row with its elements held in registers (E per lane,
// element j = lane + 64 t): the same exact radix select as the LDS path
// below, but every pass streams registers instead of re-reading and
// re-converting the scores. Writes the kept ids in ascending order and
// returns their count (lane-uniform).
template <int E>
__device__ __forceinline__ int select_row_regs(const float* sr, int nkb, float thr, int row,
                                               const int32_t* ksz, const Window& win,
                                               unsigned long long* h, int32_t* out, int lane) {
  // per element: pb = bits of p (the key is pb << 13 | 8191 - j) and the
  // fixed-point mass mm = floor(p * 2^31)
  uint32_t pb[E], mm[E];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int j = lane + kWave * t;
    const float sj = j < nkb ? sr[j] : -INFINITY;
    pb[t] = __float_as_uint(sj);
    mx = fmaxf(mx, sj);
  }
  mx = wave_max(mx);
  unsigned long long z = 0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int j = lane + kWave * t;
    // exp(s - max) as exp2 on the hardware unit: relative error ~1e-6
    const float pj = j < nkb ? __builtin_amdgcn_exp2f((__uint_as_float(pb[t]) - mx) * 1.4426950408889634f) : 0.f;
    pb[t] = __float_as_uint(pj);
    mm[t] = (uint32_t)(pj * kMassScale);
    z += mm[t];
  }
  auto key_of = [&](int t) -> unsigned long long {
    return ((unsigned long long)pb[t] << kIdxBits) | (unsigned)((1 << kIdxBits) - 1 - (lane + kWave * t));
  };
  z = wave_sum_u64(z);
  const double tt = ceil((double)thr * (double)z);
  const unsigned long long tint = tt >= (double)z ? z : (unsigned long long)tt;

  unsigned long long prefix = 0, below = 0;
  bool done = false;
  unsigned long long kstar = 0;
  // a zero threshold keeps every block: k* = 0 without any pass
#pragma unroll 1
  for (int pass = 0; pass < kPasses && tint > 0; ++pass) {
    // digits from the top: 8 bits at 35, 27, 19, 11, 3, then bits 2..0
    const int width = pass < kPasses - 1 ? kDigit : kKeyBits - kDigit * (kPasses - 1);
    const int shift = pass < kPasses - 1 ? kKeyBits - kDigit * (pass + 1) : 0;
    // rebuild keys inside each pass instead of keeping 64-bit copies of all
    // of them alive across passes (register pressure)
#pragma unroll
    for (int t = 0; t < E; ++t) asm volatile("" : "+v"(pb[t]));
    if (pass == 2) {
      // The cut lies among the keys that share the 16-bit prefix (bits 42..27). When there
      // are at most 64 of them, finish exactly with one candidate per lane:
      // k* is the smallest candidate key whose inclusive cumulative mass
      // (below + candidates with keys <= it) reaches the threshold.
      int ncand = 0;
#pragma unroll
      for (int t = 0; t < E; ++t) ncand += __popcll(__ballot((key_of(t) >> (shift + width)) == prefix));
      if (ncand <= kWave) {
        unsigned long long* slot = h;          // 64 x (key, mass) = 1 KiB of this wave's histogram
        int at = 0;
#pragma unroll
        for (int t = 0; t < E; ++t) {
          const unsigned long long kt = key_of(t);
          const bool c = (kt >> (shift + width)) == prefix;
          const unsigned long long bal = __ballot(c);
          if (c) {
            const int r = at + __popcll(bal & ((1ull << lane) - 1ull));
            slot[2 * r] = kt;
            slot[2 * r + 1] = mm[t];
          }
          at += __popcll(bal);
        }
        wave_lds_sync();
        const unsigned long long ck = lane < ncand ? slot[2 * lane] : ~0ull;
        unsigned long long through = below;
#pragma unroll 8
        for (int i = 0; i < ncand; ++i) {
          const unsigned long long ki = slot[2 * i], mi = slot[2 * i + 1];   // same address in every lane
          through += ki <= ck ? mi : 0ull;
        }
        const bool ok = lane < ncand && through >= tint;
        // smallest qualifying key; some candidate always qualifies since
        // below + all candidate mass >= the threshold
        unsigned long long best = ok ? ck : ~0ull;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const unsigned long long other = __shfl_xor(best, o);
          best = other < best ? other : best;
        }
        kstar = best;
        done = true;
        wave_lds_sync();
        break;
      }
    }
    if (pass == 0) {
      // First digit (key bits 42..35 = bits 29..22 of p): a block with mass
      // has p >= 2^-31, so its digit is in [kDigit0, 255) -- 64 bins, one per
      // lane, accumulated in 8 private copies (lanes l, l+8, ... share one).
      unsigned long long* h0 = h;                  // [8][64]
#pragma unroll
      for (int q = 0; q < 8; ++q) h0[q * kWave + lane] = 0;
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < E; ++t)
        if (mm[t]) atomicAdd(&h0[(lane & 7) * kWave + ((pb[t] >> 22) - kDigit0)], (unsigned long long)mm[t]);
      wave_lds_sync();
      unsigned long long v = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) v += h0[q * kWave + lane];
      const unsigned long long through = wave_incl_scan_u64(v, lane);
      const int b0 = wave_min_i32(through >= tint ? lane : 1 << 30);
      below = __shfl(through - v, b0);
      prefix = (unsigned)(kDigit0 + b0);
      wave_lds_sync();
      continue;
    }
#pragma unroll
    for (int q = 0; q < kBins / kWave; ++q) h[lane * (kBins / kWave) + q] = 0;
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < E; ++t) {
      const unsigned long long kt = key_of(t);
      if ((kt >> (shift + width)) == prefix && mm[t])
        atomicAdd(&h[(kt >> shift) & ((1 << width) - 1)], (unsigned long long)mm[t]);
    }
    wave_lds_sync();
    // lane owns bins [4*lane, 4*lane+4)
    unsigned long long hv[kBins / kWave];
    unsigned long long loc = 0;
#pragma unroll
    for (int q = 0; q < kBins / kWave; ++q) {
      hv[q] = h[lane * (kBins / kWave) + q];
      loc += hv[q];
    }
    const unsigned long long incl = wave_incl_scan_u64(loc, lane);
    const unsigned long long run = incl - loc;
    const unsigned long long need = tint > below ? tint - below : 0ull;
    int cand = 1 << 30;
    unsigned long long before = 0;
#pragma unroll
    for (int q = kBins / kWave - 1; q >= 0; --q) {
      unsigned long long through = run;
#pragma unroll
      for (int f = 0; f <= q; ++f) through += hv[f];
      if (through >= need) {
        cand = lane * (kBins / kWave) + q;
        before = through - hv[q];
      }
    }
    int b = wave_min_i32(cand);
    if (b >= kBins) b = kBins - 1;   // unreachable for finite inputs
    before = __shfl(before, b / (kBins / kWave));
    below += before;
    prefix = (prefix << width) | (unsigned)b;
    wave_lds_sync();
  }
  if (!done) kstar = prefix;

  int base = 0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int j = lane + kWave * t;
    bool keep = j < nkb && key_of(t) >= kstar;
    if (keep && ksz && ksz[j] <= 0) keep = false;
    if (j < nkb && win.enabled && win.inside(row, j)) keep = true;
    const unsigned long long bal = __ballot(keep);
    if (keep) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
    base += __popcll(bal);
  }
  return base;
}

template <int D, int R, int E>
__global__ __launch_bounds__(64 * kSelWaves) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int nkb_pad,
    Sizes sz, float thr, float scale, Window win, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
    int kv_stride) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc = reinterpret_cast<float*>(smem);                                  // [R][nkb_pad]
  unsigned long long* hist =
      reinterpret_cast<unsigned long long*>(smem + (size_t)R * nkb_pad * sizeof(float));  // [4][kBins]

  constexpr int KQ = D / 4;
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, i16 = lane & 15;

  // ---------------- phase 1: score rows into LDS
  float a[KQ];
  {
    const int row = row0 + i16;
    const bool ok = i16 < R && row < nqb;
    const float4* src =
        reinterpret_cast<const float4*>(qbar + ((size_t)bh * nqb + (ok ? row : 0)) * D + g * KQ);
#pragma unroll
    for (int s = 0; s < KQ / 4; ++s) {
      const float4 v = ok ? src[s] : make_float4(0.f, 0.f, 0.f, 0.f);
      a[4 * s + 0] = v.x; a[4 * s + 1] = v.y; a[4 * s + 2] = v.z; a[4 * s + 3] = v.w;
    }
  }
  const float* kbh = kbar + (size_t)bh * nkb * D;
  const int ntiles = (nkb + 15) >> 4;
  // key rows of tile t for this lane (B operand), loaded one tile ahead
  auto load_b = [&](int t, float* b) {
    const int key = t * 16 + i16;
    const bool kok = key < nkb;
    const float4* src = reinterpret_cast<const float4*>(kbh + (size_t)(kok ? key : 0) * D + g * KQ);
#pragma unroll
    for (int s4 = 0; s4 < KQ / 4; ++s4) {
      const float4 v = kok ? src[s4] : make_float4(0.f, 0.f, 0.f, 0.f);
      b[4 * s4 + 0] = v.x; b[4 * s4 + 1] = v.y; b[4 * s4 + 2] = v.z; b[4 * s4 + 3] = v.w;
    }
  };
  float b[KQ], bn[KQ] = {};
  if (wave < ntiles) load_b(wave, b);
  for (int t = wave; t < ntiles; t += kSelWaves) {
    const int key = t * 16 + i16;
    const bool kok = key < nkb;
    if (t + kSelWaves < ntiles) load_b(t + kSelWaves, bn);
    // four independent accumulation chains, summed at the end
    f32x4 acc4[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) acc4[c4] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KQ; ++s) acc4[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc4[s & 3], 0, 0, 0);
    const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    if (kok) {
      float bias = 0.f;
      bool excluded = false;
      if (const int32_t* ks = sz.krow(bh, nkb)) {
        const int n = ks[key];
        excluded = n <= 0;
        bias = excluded || !sz.bias ? 0.f : logf((float)n);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 4 * g + v;   // MFMA output row held in register v
        if (rr < R) sc[rr * nkb_pad + key] = excluded ? -INFINITY : acc[v] * scale + bias;
      }
    }
#pragma unroll
    for (int s4 = 0; s4 < KQ; ++s4) b[s4] = bn[s4];
  }
  __syncthreads();

  // ---------------- phase 2: per-row CDF selection
  unsigned long long* h = hist + wave * kHist;
  for (int rr = wave; rr < R; rr += kSelWaves) {
    const int row = row0 + rr;
    if (row >= nqb) break;
    const size_t orow = (size_t)bh * nqb + row;
    int32_t* out = kv_index + orow * kv_stride;
    if (sz.q_empty(bh, nqb, row)) {
      if (lane == 0) kv_count[orow] = 0;
      continue;
    }
    float* sr = sc + rr * nkb_pad;
    if constexpr (E > 0) {
      const int n = select_row_regs<E>(sr, nkb, thr, row, sz.krow(bh, nkb),
                                       win, h, out, lane);
      if (lane == 0) kv_count[orow] = n;
      continue;
    }
    float mx = -INFINITY;
    for (int j = lane; j < nkb; j += kWave) mx = fmaxf(mx, sr[j]);
    mx = wave_max(mx);
    unsigned long long z = 0;
    for (int j = lane; j < nkb; j += kWave) {
      const float p = expf(sr[j] - mx);     // in [0, 1]; exp(-inf) = 0
      sr[j] = p;
      z += (unsigned long long)(p * kMassScale);
    }
    z = wave_sum_u64(z);
    const double tt = ceil((double)thr * (double)z);
    const unsigned long long tint = tt >= (double)z ? z : (unsigned long long)tt;
    wave_lds_sync();

    unsigned long long prefix = 0, below = 0;
#pragma unroll 1
    for (int pass = 0; pass < kPasses; ++pass) {
      const int shift = kDigit * (kPasses - 1 - pass);
#pragma unroll
      for (int e = 0; e < kBins / kWave; ++e) h[lane * (kBins / kWave) + e] = 0;
      wave_lds_sync();
      for (int j = lane; j < nkb; j += kWave) {
        const float p = sr[j];
        const unsigned long long key =
            ((unsigned long long)__float_as_uint(p) << kIdxBits) | (unsigned)((1 << kIdxBits) - 1 - j);
        if ((key >> (shift + kDigit)) == prefix) {
          const unsigned long long m = (unsigned long long)(p * kMassScale);
          if (m) atomicAdd(&h[(key >> shift) & (kBins - 1)], m);
        }
      }
      wave_lds_sync();
      // lane owns bins [4*lane, 4*lane+4)
      unsigned long long hv[kBins / kWave];
      unsigned long long loc = 0;
#pragma unroll
      for (int e = 0; e < kBins / kWave; ++e) {
        hv[e] = h[lane * (kBins / kWave) + e];
        loc += hv[e];
      }
      const unsigned long long incl = wave_incl_scan_u64(loc, lane);
      unsigned long long run = incl - loc;
      const unsigned long long need = tint > below ? tint - below : 0ull;
      int cand = 1 << 30;
      unsigned long long before = 0;
#pragma unroll
      for (int e = kBins / kWave - 1; e >= 0; --e) {
        // cumulative mass through bin (4*lane + e)
        unsigned long long through = run;
#pragma unroll
        for (int f = 0; f <= e; ++f) through += hv[f];
        if (through >= need) {
          cand = lane * (kBins / kWave) + e;
          before = through - hv[e];
        }
      }
      int b = wave_min_i32(cand);
      if (b >= kBins) b = kBins - 1;   // unreachable for finite inputs
      before = __shfl(before, b / (kBins / kWave));
      below += before;
      prefix = (prefix << kDigit) | (unsigned)b;
      wave_lds_sync();
    }
    const unsigned long long kstar = prefix;

    int base = 0;
    for (int j0 = 0; j0 < nkb; j0 += kWave) {
      const int j = j0 + lane;
      bool keep = false;
      if (j < nkb) {
        const unsigned long long key =
            ((unsigned long long)__float_as_uint(sr[j]) << kIdxBits) | (unsigned)((1 << kIdxBits) - 1 - j);
        keep = key >= kstar;
        if (const int32_t* ks = sz.krow(bh, nkb)) keep = keep && ks[j] > 0;
        if (win.enabled && win.inside(row, j)) keep = true;
      }
      const unsigned long long bal = __ballot(keep);
      if (keep) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
      base += __popcll(bal);
    }
    if (lane == 0) kv_count[orow] = base;
  }
}

template <int D, int R, int E>
static hipError_t launch_select_t(const float* qbar, const float* kbar, int BH, int nqb, int nkb,
                                  const Sizes& sz, float thr, float scale, const Window& win, int32_t* kv_count,
                                  int32_t* kv_index, int kv_stride, hipStream_t s) {
  const int nkb_pad = (nkb + 3) & ~3;
  const size_t lds = (size_t)R * nkb_pad * sizeof(float) + kSelWaves * kHist * sizeof(unsigned long long);
  auto kern = select_kernel<D, R, E>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((nqb + R - 1) / R, BH);
  kern<<<grid, 64 * kSelWaves, lds, s>>>(qbar, kbar, nqb, nkb, nkb_pad, sz, thr, scale, win,
                              kv_count, kv_index, kv_stride);
  return hipGetLastError();
}

hipError_t launch_select(const float* qbar, const float* kbar, int BH, int nqb, int nkb, int d,
                         const Sizes& sz, float thr, float scale,
                         const Window& win, int32_t* kv_count, int32_t* kv_index, int kv_stride,
                         hipStream_t s) {
  if (BH == 0 || nqb == 0) return hipSuccess;
#define BSA_SEL(DD, RR, EE) \
  launch_select_t<DD, RR, EE>(qbar, kbar, BH, nqb, nkb, sz, thr, scale, win, kv_count, kv_index, kv_stride, s)
  // rows of up to 2048 key blocks are selected from registers (E per lane)
  if (d == 128) {
    if (nkb <= 512) return BSA_SEL(128, 16, 8);
    if (nkb <= 1024) return BSA_SEL(128, 16, 16);
    if (nkb <= 2048) return BSA_SEL(128, 16, 32);
    if (nkb <= 4096) return BSA_SEL(128, 8, 0);
    return BSA_SEL(128, 4, 0);
  }
  if (nkb <= 512) return BSA_SEL(64, 16, 8);
  if (nkb <= 1024) return BSA_SEL(64, 16, 16);
  if (nkb <= 2048) return BSA_SEL(64, 16, 32);
  if (nkb <= 4096) return BSA_SEL(64, 8, 0);
  return BSA_SEL(64, 4, 0);
#undef BSA_SEL
}

}  // namespace bsa

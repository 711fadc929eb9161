// Reduced attention + CDF selection of key blocks (NABLA summary, Metodologia
// section 2, "Attenzione Ridotta" and "CDF Thresholding"; section 3 for the
// window union; Sparse VideoGen2 summary, Metodologia B for the
// size-weighted centroid variant).
//
// One workgroup of 4 waves owns R consecutive rows of one head's reduced map;
// rows of 1025..2048 key blocks at d = 128 go to a pipelined kernel in which
// some waves score the next 16 rows while the others select the previous 16.
//
// Phase 1 -- scores. s[r][J] = scale * qbar_r . kbar_J (+ log n_J) for all
// key blocks, on fp32 MFMA 16x16x4 (A = 16 pooled query rows, B = 16 pooled
// key rows, the 4-wide k slot of the MFMA split over the four 16-lane
// groups), or in the pipelined kernel on bf16 MFMA over exact three-way
// bf16 splits of both fp32 operands. Lane group g takes the 16-byte pieces
// 4s + g of a row, so one load instruction reads 64 contiguous bytes of each
// of its 16 rows rather than 16 bytes of 64 separate lines. The R x nkb fp32
// score rows stay in LDS; the reduced map never touches HBM.
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

#include <algorithm>
#include <atomic>

namespace bsa {

// Rows of 1025..2048 key blocks at d = 128 (the 118,800-token layer) take the
// pipelined kernel below: 4 scoring waves and 8 selecting waves per
// workgroup, each selecting wave holding two rows in registers (168 VGPRs at
// three waves per SIMD). Measured at 1857 key blocks, mask stage (pool +
// select) in the bench loop: 0.94 ms with one 8-wave workgroup per 16 rows
// (scoring, then selecting), 0.86 pipelined with fp32 MFMA scores (those
// hold the SIMD's VALU, so the two roles took turns), 0.73 with the scores
// on bf16 MFMA over exact three-way splits.
constexpr int kSelPW = 4, kSelSW = 8;

namespace {
constexpr int kIdxBits = 13;          // supports nkb <= 8192
constexpr int kKeyBits = 30 + kIdxBits;
constexpr int kDigit = 8;
constexpr int kPasses = (kKeyBits + kDigit - 1) / kDigit;   // 6
constexpr int kBins = 1 << kDigit;
constexpr float kMassScale = 0x1p31f; // block masses in 2^-31 fixed point
// histogram words per wave: 8 private copies of the first-digit histogram
// (64 bins), or 4 with 16 waves sharing the LDS; later passes use 256
template <int W>
constexpr int hist_words() { return W >= 16 ? 256 : 512; }
constexpr int kDigit0 = 192;          // first-digit value of p = 2^-31 (bits(p) >> 22)

// Wave-wide scans and reductions on DPP lane moves (GFX9 controls): four
// shifts inside each row of 16 lanes, then the row broadcasts of lanes 15
// and 31 into the following rows. A step costs a VALU move with no trip
// through the LDS crossbar, which is what the shuffles of a radix pass
// chain on. Source lanes outside a row, and rows the mask leaves out, read
// the identity `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t id, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long id, unsigned long long x) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)id, (uint32_t)x);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(id >> 32), (uint32_t)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ unsigned long long scan_u64(unsigned long long x) {
  x += dpp_u64<kRowShr1, 0xf>(0, x);
  x += dpp_u64<kRowShr2, 0xf>(0, x);
  x += dpp_u64<kRowShr4, 0xf>(0, x);
  x += dpp_u64<kRowShr8, 0xf>(0, x);
  x += dpp_u64<kRowBcast15, 0xa>(0, x);
  x += dpp_u64<kRowBcast31, 0xc>(0, x);
  return x;
}
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long x, int l) {   // l wave-uniform
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long sum_u64(unsigned long long x) { return lane_u64(scan_u64(x), 63); }
__device__ __forceinline__ float max_f32(float x) {
  const uint32_t id = __float_as_uint(-INFINITY);
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowShr1, 0xf>(id, __float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowShr2, 0xf>(id, __float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowShr4, 0xf>(id, __float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowShr8, 0xf>(id, __float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowBcast15, 0xa>(id, __float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_u32<kRowBcast31, 0xc>(id, __float_as_uint(x))));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), 63));
}
__device__ __forceinline__ unsigned long long min_u64(unsigned long long x) {
  const unsigned long long id = ~0ull;
  unsigned long long t;
  t = dpp_u64<kRowShr1, 0xf>(id, x); x = t < x ? t : x;
  t = dpp_u64<kRowShr2, 0xf>(id, x); x = t < x ? t : x;
  t = dpp_u64<kRowShr4, 0xf>(id, x); x = t < x ? t : x;
  t = dpp_u64<kRowShr8, 0xf>(id, x); x = t < x ? t : x;
  t = dpp_u64<kRowBcast15, 0xa>(id, x); x = t < x ? t : x;
  t = dpp_u64<kRowBcast31, 0xc>(id, x); x = t < x ? t : x;
  return lane_u64(x, 63);
}
// first lane whose predicate holds (64 when none)
__device__ __forceinline__ int first_lane(bool p) {
  const unsigned long long m = __ballot(p);
  return m ? __builtin_ctzll(m) : kWave;
}
}  // namespace

// Selection of one row with its elements held in registers (E per lane,
// element j = lane + 64 t): the same exact radix select as the LDS path
// below, but every pass streams registers instead of re-reading and
// re-converting the scores. On entry pb holds the bits of the row's scores
// (-inf past nkb); it is overwritten. Writes the kept ids in ascending order
// and returns their count (lane-uniform).
template <int E, int COPIES>
__device__ __forceinline__ int select_row_core(uint32_t (&pb)[E], int nkb, float thr, int row,
                                               const int32_t* ksz, const Window& win,
                                               unsigned long long* h, int32_t* out, int lane) {
  // per element: pb = bits of p (the key is pb << 13 | 8191 - j); its
  // fixed-point mass floor(p * 2^31) is recomputed where needed (mass_of)
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < E; ++t) mx = fmaxf(mx, __uint_as_float(pb[t]));
  mx = max_f32(mx);
  unsigned long long z = 0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int j = lane + kWave * t;
    // exp(s - max) as exp2 on the hardware unit: relative error ~1e-6
    const float pj = j < nkb ? __builtin_amdgcn_exp2f((__uint_as_float(pb[t]) - mx) * 1.4426950408889634f) : 0.f;
    pb[t] = __float_as_uint(pj);
    z += (uint32_t)(pj * kMassScale);
  }
  auto mass_of = [&](int t) -> uint32_t { return (uint32_t)(__uint_as_float(pb[t]) * kMassScale); };
  auto key_of = [&](int t) -> unsigned long long {
    return ((unsigned long long)pb[t] << kIdxBits) | (unsigned)((1 << kIdxBits) - 1 - (lane + kWave * t));
  };
  z = sum_u64(z);
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
    asm volatile("" : "+v"(lane));
    if (pass == 2) {
      // The cut lies among the keys that share the 16-bit prefix (bits 42..27). When there
      // are at most 64 of them, finish exactly with one candidate per lane:
      // k* is the smallest candidate key whose inclusive cumulative mass
      // (below + candidates with keys <= it) reaches the threshold.
      // (key >> 27 == pb >> 14: the prefix lies in the probability bits, so
      // the test is one 32-bit shift and compare per element)
      const uint32_t pfx = (uint32_t)prefix;
      int ncand = 0;
#pragma unroll
      for (int t = 0; t < E; ++t) ncand += __popcll(__ballot((pb[t] >> 14) == pfx));
      if (ncand <= kWave) {
        unsigned long long* slot = h;          // 64 x (key, mass) = 1 KiB of this wave's histogram
        int at = 0;
#pragma unroll
        for (int t = 0; t < E; ++t) {
          const bool c = (pb[t] >> 14) == pfx;
          const unsigned long long bal = __ballot(c);
          if (c) {
            const int r = at + __popcll(bal & ((1ull << lane) - 1ull));
            slot[2 * r] = key_of(t);
            slot[2 * r + 1] = mass_of(t);
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
        kstar = min_u64(ok ? ck : ~0ull);
        done = true;
        wave_lds_sync();
        break;
      }
    }
    if (pass == 0) {
      // First digit (key bits 42..35 = bits 29..22 of p): a block with mass
      // has p >= 2^-31, so its digit is in [kDigit0, 255) -- 64 bins, one per
      // lane, accumulated in COPIES private copies (lanes l, l+COPIES, ...
      // share one).
      unsigned long long* h0 = h;                  // [COPIES][64]
#pragma unroll
      for (int q = 0; q < COPIES; ++q) h0[q * kWave + lane] = 0;
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < E; ++t)
        if (const uint32_t mt = mass_of(t))
          atomicAdd(&h0[(lane & (COPIES - 1)) * kWave + ((pb[t] >> 22) - kDigit0)], (unsigned long long)mt);
      wave_lds_sync();
      unsigned long long v = 0;
#pragma unroll
      for (int q = 0; q < COPIES; ++q) v += h0[q * kWave + lane];
      // the cumulative mass grows with the lane: the first lane reaching the
      // threshold holds the digit
      const unsigned long long through = scan_u64(v);
      const int f0 = first_lane(through >= tint);
      const int b0 = f0 < kWave ? f0 : 1 << 30;   // none: unreachable for finite inputs
      below = lane_u64(through - v, f0 & (kWave - 1));
      prefix = (unsigned)(kDigit0 + b0);
      wave_lds_sync();
      continue;
    }
#pragma unroll
    for (int q = 0; q < kBins / kWave; ++q) h[lane * (kBins / kWave) + q] = 0;
    wave_lds_sync();
    if (shift >= kIdxBits) {
      // the digit and the prefix lie in the probability bits (passes 1, 2):
      // key >> n == pb >> (n - 13) for n >= 13, in 32-bit arithmetic
      const int ps = shift - kIdxBits;
      const uint32_t pfx = (uint32_t)prefix;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        const uint32_t mt = mass_of(t);
        if ((pb[t] >> (ps + width)) == pfx && mt)
          atomicAdd(&h[(pb[t] >> ps) & ((1 << width) - 1)], (unsigned long long)mt);
      }
    } else {
#pragma unroll
      for (int t = 0; t < E; ++t) {
        const unsigned long long kt = key_of(t);
        const uint32_t mt = mass_of(t);
        if ((kt >> (shift + width)) == prefix && mt)
          atomicAdd(&h[(kt >> shift) & ((1 << width) - 1)], (unsigned long long)mt);
      }
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
    const unsigned long long incl = scan_u64(loc);
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
    // the first lane whose bins reach the need holds the digit (the
    // cumulative mass grows with the lane); none: unreachable for finite
    // inputs, the last bin
    const int fl = first_lane(incl >= need) & (kWave - 1);
    int b = __builtin_amdgcn_readlane(cand, fl);
    if (b >= kBins) b = kBins - 1;
    before = lane_u64(before, fl);
    below += before;
    prefix = (prefix << width) | (unsigned)b;
    wave_lds_sync();
  }
  if (!done) kstar = prefix;

  int base = 0;
  asm volatile("" : "+v"(lane));
  // key >= k*  <=>  pb > k*_hi, or pb == k*_hi and 8191 - j >= k*_lo
  const uint32_t ks_hi = (uint32_t)(kstar >> kIdxBits), ks_lo = (uint32_t)(kstar & ((1u << kIdxBits) - 1));
  const bool none = (kstar >> kIdxBits) > 0xffffffffull;   // k* past every key: keep nothing by the CDF
#pragma unroll
  for (int t = 0; t < E; ++t) {
    // j through an empty asm: the window coordinates of the lane's E blocks
    // are the same for every row, and hoisted out of the row loop they
    // would hold 3 E registers (spilled)
    int j = lane + kWave * t;
    asm volatile("" : "+v"(j));
    const uint32_t lo = (uint32_t)((1 << kIdxBits) - 1 - j);
    bool keep = j < nkb && !none && (pb[t] > ks_hi || (pb[t] == ks_hi && lo >= ks_lo));
    if (keep && ksz && ksz[j] <= 0) keep = false;
    if (j < nkb && win.enabled && win.inside(row, j)) keep = true;
    const unsigned long long bal = __ballot(keep);
    if (keep) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
    base += __popcll(bal);
  }
  return base;
}

// The row's scores from LDS into registers, then the selection above.
template <int E, int COPIES>
__device__ __forceinline__ int select_row_regs(const float* sr, int nkb, float thr, int row,
                                               const int32_t* ksz, const Window& win,
                                               unsigned long long* h, int32_t* out, int lane) {
  uint32_t pb[E];
#pragma unroll
  for (int t = 0; t < E; ++t) {
    const int j = lane + kWave * t;
    pb[t] = __float_as_uint(j < nkb ? sr[j] : -INFINITY);
  }
  return select_row_core<E, COPIES>(pb, nkb, thr, row, ksz, win, h, out, lane);
}

// Exact three-way split of eight fp32 values into bf16 planes, x = x1 + x2 +
// x3: x1 keeps the top 8 significant bits of x (truncation), x2 the top 8 of
// the remainder, and the last remainder has at most 8 significant bits, so
// it is a bf16 exactly. Both subtractions are exact (same sign, same
// exponent). Element e of each plane is x[e].
__device__ __forceinline__ void split3_bf16(const float* x, bf16x8& p1, bf16x8& p2, bf16x8& p3) {
  uint32_t w1[4], w2[4], w3[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a0 = __float_as_uint(x[2 * i]), a1 = __float_as_uint(x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(a0 & 0xffff0000u);
    const float r1 = x[2 * i + 1] - __uint_as_float(a1 & 0xffff0000u);
    const uint32_t b0 = __float_as_uint(r0), b1 = __float_as_uint(r1);
    const float s0 = r0 - __uint_as_float(b0 & 0xffff0000u);
    const float s1 = r1 - __uint_as_float(b1 & 0xffff0000u);
    // high halves of two words -> one word (element 2i low, 2i+1 high)
    w1[i] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    w2[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
    w3[i] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
  }
  __builtin_memcpy(&p1, w1, 16);
  __builtin_memcpy(&p2, w2, 16);
  __builtin_memcpy(&p3, w3, 16);
}

// Phase 1: the scores of rows row0..row0+R-1 of head bh against every key
// block, into sc ([R][nkb_pad]), by NW waves of which this is number wv.
// Products on fp32 MFMA 16x16x4, or with SPLIT on bf16 MFMA 16x16x32 over
// the three-way splits of both operands: every cross product but x3 y3
// (below 2^-28 of |x||y|), each exact in fp32 and summed in fp32. A lane's
// 32 values of a row (the pieces 4s + g) form chunk c from a[8c..8c+7], on
// both sides, so the d order matches. The bf16 products run beside other
// waves' VALU work; the fp32 ones hold the SIMD's VALU while they run.
template <int D, int R, int NW, bool SPLIT = false>
__device__ __forceinline__ void score_rows(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                           int bh, int row0, int nqb, int nkb, int nkb_pad, const Sizes& sz,
                                           float scale, float* sc, int wv, int lane) {
  constexpr int KQ = D / 4;
  const int g = lane >> 4, i16 = lane & 15;
  float a[KQ];
  {
    const int row = row0 + i16;
    const bool ok = i16 < R && row < nqb;
    const float4* src = reinterpret_cast<const float4*>(qbar + ((size_t)bh * nqb + (ok ? row : 0)) * D);
#pragma unroll
    for (int s = 0; s < KQ / 4; ++s) {
      const float4 v = ok ? src[4 * s + g] : make_float4(0.f, 0.f, 0.f, 0.f);
      a[4 * s + 0] = v.x; a[4 * s + 1] = v.y; a[4 * s + 2] = v.z; a[4 * s + 3] = v.w;
    }
  }
  constexpr int NC = D / 32;
  bf16x8 qa[SPLIT ? 3 : 1][SPLIT ? NC : 1];
  if constexpr (SPLIT) {
#pragma unroll
    for (int c = 0; c < NC; ++c) split3_bf16(&a[8 * c], qa[0][c], qa[1][c], qa[2][c]);
  }
  const float* kbh = kbar + (size_t)bh * nkb * D;
  const int ntiles = (nkb + 15) >> 4;
  // key rows of tile t for this lane (B operand). Rows past nkb read the
  // last row (their scores are never stored), so every load is
  // unconditional and the compiler can count them.
  auto load_b = [&](int t, float* b) {
    const int key = min(t * 16 + i16, nkb - 1);
    const float4* src = reinterpret_cast<const float4*>(kbh + (size_t)key * D);
#pragma unroll
    for (int s4 = 0; s4 < KQ / 4; ++s4) {
      const float4 v = src[4 * s4 + g];
      b[4 * s4 + 0] = v.x; b[4 * s4 + 1] = v.y; b[4 * s4 + 2] = v.z; b[4 * s4 + 3] = v.w;
    }
  };
  auto score_tile = [&](int t, const float* b) {
    const int key = t * 16 + i16;
    // four independent accumulation chains, summed at the end
    f32x4 acc4[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) acc4[c4] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 kb[3];
        split3_bf16(&b[8 * c], kb[0], kb[1], kb[2]);
        // (q plane, k plane): every pair but (3, 3)
        constexpr int PQ[8] = {0, 0, 1, 0, 1, 2, 1, 2}, PK[8] = {0, 1, 0, 2, 1, 0, 2, 1};
#pragma unroll
        for (int p = 0; p < 8; ++p)
          acc4[p & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[PQ[p]][c], kb[PK[p]], acc4[p & 3], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KQ; ++s) acc4[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc4[s & 3], 0, 0, 0);
    }
    const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    if (key < nkb) {
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
  };
  // Two register buffers in turn: the loads of a wave's next tile are
  // issued before the MFMAs of the current one (the scheduling barrier
  // keeps them there), so they land while the products run.
  float b0[KQ], b1[KQ];
  if (wv < ntiles) load_b(wv, b0);
  for (int t = wv; t < ntiles; t += 2 * NW) {
    load_b(min(t + NW, ntiles - 1), b1);
    __builtin_amdgcn_sched_barrier(0);
    score_tile(t, b0);
    if (t + NW >= ntiles) break;
    load_b(min(t + 2 * NW, ntiles - 1), b0);
    __builtin_amdgcn_sched_barrier(0);
    score_tile(t + NW, b1);
  }
}

template <int D, int R, int E, int W>
__global__ __launch_bounds__(64 * W) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int nkb_pad,
    Sizes sz, float thr, float scale, Window win, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
    int kv_stride) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc = reinterpret_cast<float*>(smem);                                  // [R][nkb_pad]
  unsigned long long* hist =
      reinterpret_cast<unsigned long long*>(smem + (size_t)R * nkb_pad * sizeof(float));  // [W][kHist]

  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // ---------------- phase 1: score rows into LDS
  score_rows<D, R, W>(qbar, kbar, bh, row0, nqb, nkb, nkb_pad, sz, scale, sc, wave, lane);
  __syncthreads();

  // ---------------- phase 2: per-row CDF selection
  unsigned long long* h = hist + wave * hist_words<W>();
  for (int rr = wave; rr < R; rr += W) {
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
      const int n = select_row_regs<E, W >= 16 ? 4 : 8>(sr, nkb, thr, row, sz.krow(bh, nkb),
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

// Rows of 1025..2048 key blocks, pipelined over groups of 16 rows. Each
// workgroup takes a contiguous range of (head, 16-row group) pairs; PW
// scoring waves write the scores of group k into LDS while SW selecting
// waves select the rows of group k - 1, each holding 16 / SW rows in
// registers, so the fp32 MFMA and key-stream work of one group runs beside
// the VALU and LDS-atomic work of the previous one (with one group per
// workgroup the two phases take turns on the CU). Two workgroup barriers per
// group: after the first, the scores of group k are complete and the
// selecting waves copy their rows into registers; after the second the
// score rows are free for group k + 1. Both roles pass the same number of
// barriers. The ranges are laid out XCD by XCD (workgroup i runs on XCD
// i mod 8), so the groups running together on one XCD share a few heads'
// pooled keys in its L2.
template <int D, int E, int PW, int SW>
__global__ __launch_bounds__(64 * (PW + SW)) void select_pipe_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int nkb_pad, int BH,
    Sizes sz, float thr, float scale, Window win, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index,
    int kv_stride) {
  constexpr int R = 16, RPW = R / SW;
  static_assert(R % SW == 0 && RPW <= 4, "each selecting wave holds the same number of rows, at most 4");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc = reinterpret_cast<float*>(smem);                                  // [R][nkb_pad]
  unsigned long long* hist =
      reinterpret_cast<unsigned long long*>(smem + (size_t)R * nkb_pad * sizeof(float));  // [SW][512]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ngr = (nqb + R - 1) / R;
  const long long total = (long long)BH * ngr;
  const int nwg = gridDim.x, i = blockIdx.x;
  const int L = (nwg & 7) == 0 ? (i & 7) * (nwg >> 3) + (i >> 3) : i;
  const int g0 = (int)(L * total / nwg);
  const int ng = (int)((L + 1) * total / nwg) - g0;
  if (wave < PW) {
    for (int k = 0; k <= ng; ++k) {
      if (k < ng) {
        const int g = g0 + k;
        score_rows<D, R, PW, true>(qbar, kbar, g / ngr, (g % ngr) * R, nqb, nkb, nkb_pad, sz, scale, sc, wave, lane);
      }
      __syncthreads();
      __syncthreads();
    }
  } else {
    const int sw = wave - PW;
    unsigned long long* h = hist + sw * 512;
    uint32_t rows[RPW][E];
    // One call site per held row (constant indices keep the rows in
    // registers). The lane index passes through an empty asm at each call so
    // that the per-lane values derived from it (element ids, bounds masks,
    // addresses) are formed where they are used, not hoisted out of the
    // group loop, where they would not fit beside the held rows.
    auto select_one = [&](uint32_t (&pb)[E], int bh, int row) __attribute__((always_inline)) {
      if (row >= nqb) return;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const size_t orow = (size_t)bh * nqb + row;
      int n = 0;
      if (!sz.q_empty(bh, nqb, row))
        n = select_row_core<E, 8>(pb, nkb, thr, row, sz.krow(bh, nkb), win, h, kv_index + orow * kv_stride, ln);
      if (ln == 0) kv_count[orow] = n;
    };
    for (int k = 0; k <= ng; ++k) {
      if (k > 0) {
        const int g = g0 + k - 1, bh = g / ngr, row0 = (g % ngr) * R + sw;
        select_one(rows[0], bh, row0);
        if constexpr (RPW > 1) select_one(rows[1], bh, row0 + SW);
        if constexpr (RPW > 2) select_one(rows[2], bh, row0 + 2 * SW);
        if constexpr (RPW > 3) select_one(rows[3], bh, row0 + 3 * SW);
      }
      __syncthreads();
      if (k < ng) {
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
          const float* sr = sc + (sw + SW * q) * nkb_pad;
#pragma unroll
          for (int t = 0; t < E; ++t) {
            const int j = lane + kWave * t;
            rows[q][t] = __float_as_uint(j < nkb ? sr[j] : -INFINITY);
          }
        }
      }
      __syncthreads();
    }
  }
}

template <int D, int R, int E, int W = 4>
static hipError_t launch_select_t(const float* qbar, const float* kbar, int BH, int nqb, int nkb,
                                  const Sizes& sz, float thr, float scale, const Window& win, int32_t* kv_count,
                                  int32_t* kv_index, int kv_stride, hipStream_t s) {
  const int nkb_pad = (nkb + 3) & ~3;
  const size_t lds = (size_t)R * nkb_pad * sizeof(float) + W * hist_words<W>() * sizeof(unsigned long long);
  auto kern = select_kernel<D, R, E, W>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((nqb + R - 1) / R, BH);
  kern<<<grid, 64 * W, lds, s>>>(qbar, kbar, nqb, nkb, nkb_pad, sz, thr, scale, win,
                              kv_count, kv_index, kv_stride);
  return hipGetLastError();
}

// CU count of the current device, cached per device.
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int E, int PW, int SW>
static hipError_t launch_select_pipe(const float* qbar, const float* kbar, int BH, int nqb, int nkb,
                                     const Sizes& sz, float thr, float scale, const Window& win,
                                     int32_t* kv_count, int32_t* kv_index, int kv_stride, hipStream_t s) {
  const int nkb_pad = (nkb + 3) & ~3;
  const size_t lds = (size_t)16 * nkb_pad * sizeof(float) + (size_t)SW * 512 * sizeof(unsigned long long);
  auto kern = select_pipe_kernel<D, E, PW, SW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // the score rows take most of the LDS: one workgroup per CU, each over a
  // range of whole groups
  const long long groups = (long long)BH * ((nqb + 15) / 16);
  const int nwg = (int)std::min<long long>(groups, device_cus());
  kern<<<nwg, 64 * (PW + SW), lds, s>>>(qbar, kbar, nqb, nkb, nkb_pad, BH, sz, thr, scale, win,
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
    // E = 30 registers per row up to 1920 key blocks: no spills at the
    // 168-register bound of three waves per SIMD
    if (nkb <= 1920)
      return launch_select_pipe<128, 30, kSelPW, kSelSW>(qbar, kbar, BH, nqb, nkb, sz, thr, scale, win,
                                                         kv_count, kv_index, kv_stride, s);
    if (nkb <= 2048)
      return launch_select_pipe<128, 32, kSelPW, kSelSW>(qbar, kbar, BH, nqb, nkb, sz, thr, scale, win,
                                                         kv_count, kv_index, kv_stride, s);
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

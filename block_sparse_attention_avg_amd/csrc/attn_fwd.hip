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
// Data movement: K and V chunks go HBM -> LDS with direct-to-LDS loads (no
// staging registers), row-major, each row's 16-byte pieces XOR-swizzled so
// that both the K operand reads and the transposed V reads below are free of
// bank conflicts. The pipeline is split by phase: the next chunk's K is in
// flight while this chunk's softmax and PV run, the next V while the next S
// runs. Waits are explicit vmcnt counts; barriers carry no memory fence (a
// fence would drain every in-flight load).
//
// Math per wave and chunk:
//   S^T = K Q^T        bf16 MFMA 32x32x16; Q^T stays in registers as the B
//                      operand for the whole tile, so each lane ends up with
//                      32 key scores of ONE query: max/sum are lane-local plus
//                      one permlane32 swap with the lane holding the other 32.
//   online softmax     fp32, log2 domain (scale*log2e folded into one FMA),
//                      O rescaled only when some row max moved.
//   O^T += V^T P^T     bf16 MFMA 32x32x16; P^T is the S^T accumulator
//                      rounded to bf16 in registers (hardware convert), and
//                      V^T comes straight from the row-major V tile through the
//                      LDS transpose read (ds_read_b64_tr_b16), addressed so
//                      its key order matches the accumulator layout of S^T.
// O is divided by the row sum once at the end, staged through LDS and
// written as bf16 rows.
#include "attn.h"

#include <math.h>

namespace bsa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
// Read-only for the whole kernel: uniform loads through it become scalar loads.
typedef __attribute__((address_space(4))) const int32_t cint;

// Swizzle of the 16-byte piece index inside a K/V tile row.
template <int D>
__device__ __forceinline__ int swz(int r) {
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

// Workgroup barrier for the LDS pipeline: this wave's LDS accesses complete
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

// max over lanes l and l^32 (the two wave halves hold the same query)
__device__ __forceinline__ float halves_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

}  // namespace

// One query tile. K and V tiles are separate LDS arrays so the compiler can
// tell the two direct-to-LDS load streams apart; all waits on those loads are
// explicit vmcnt counts.
//
// Software pipeline (iteration c, every wave):
//   prep:      mask and row max of S(c); rare rescale of O;
//   region A:  S(c+1) = K(c+1) Q^T on MFMA, interleaved instruction by
//              instruction with exp2 / row sum / bf16 pack of S(c) on the
//              VALU (independent work, so the two pipes overlap in one wave);
//   region B:  O^T += V(c)^T P(c)^T on MFMA.
// Loads: K(c+2) is issued once every wave has finished region A, V(c+1) once
// every wave has finished region B. Each iteration issues exactly one K and
// one V tile load (after the last chunk they re-load rows of a chunk that
// exists into the free buffer, and the extra S is discarded), so the number
// of loads in flight is the same on every path. The loop body is unrolled
// twice so S(c) and S(c+1) swap registers instead of being copied.
//
// Loads go through buffer descriptors that end at the chunk's last row:
// rows past it (a partial last block, gathered rows past the chunk) read as
// zeros, so no clamping is needed and padding never reaches P V.
// Key blocks: KMODE 0 = uniform 64-token blocks, 1 = descriptor blocks of at
// most 64 tokens (each one chunk, loaded like a uniform block from its own
// start), 2 = descriptor blocks of any length (keys gathered row by row into
// 64-key chunks).
template <int D, int KMODE>
__device__ __forceinline__ void attn_tile(const AttnArgs& a, int bh, int I, int qs, int ql,
                                          lds_u8* Kp, lds_u8* Vp, int* tok, int* chunk_rows) {
  constexpr int ROWB = D * 2;                  // bytes per K/V row
  constexpr int TILE = 64 * ROWB;              // bytes per K or V tile
  constexpr int NI = TILE / 1024 / 2;          // direct-to-LDS loads per wave per tile
  constexpr int RPI = 1024 / ROWB;             // rows per load instruction
  constexpr int PPR = ROWB / 16;               // 16-byte pieces per row
  constexpr float TAU = 8.f;                   // rescale O only when a row max grows by > 2^TAU
  constexpr uint32_t OOB = 0xFFFFFFF0u;        // lane offset past every descriptor: loads zeros
  constexpr bool KVAR = KMODE == 2;            // gathered keys
  // A chunk's length doubles as "the chunk exists" (> 0). A kept short block
  // with no tokens is still a chunk: its length is coded as kEmpty (no rows
  // loaded, every key masked).
  constexpr int kEmpty = 1 << 16;
  auto rows_of = [](int kl) { return KMODE == 1 ? kl & (kEmpty - 1) : kl; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const size_t head_off = (size_t)bh * a.N * D;
  const uint16_t* qh = a.q + head_off;
  const unsigned char* kh = reinterpret_cast<const unsigned char*>(a.k + head_off);
  const unsigned char* vh = reinterpret_cast<const unsigned char*>(a.v + head_off);

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
  // reference row max in log2 units; short blocks start from a finite floor
  // so that a first chunk with every key masked (an empty block) gives
  // exp2(-inf) = 0 rather than exp2(-inf + inf)
  float m_run = KMODE == 1 ? -1e30f : -INFINITY, l_run = 0.f;

  const size_t qrow = (size_t)bh * a.nqb + I;
  const int cnt = ((const cint*)a.kv_count)[qrow];
  const int32_t* list = a.kv_index + qrow * a.kv_stride;
  const cint* slist = (const cint*)list;

  // ---- per-lane LDS offsets (loop invariant)
  // K operand of S^T: row 32kb + l32, piece 2c + half.
  const int fk = swz<D>(l32 & 15);
  // V^T operand via the transpose read: lane (16-lane group g, slot 4j+q)
  // addresses key row 32kb + 16hh + 8t + 4*half + j, channels
  // 32dg + 16(g&1) + 4q .. +3, so the lane receives channel 32dg + l32 of
  // keys 32kb + 16hh + 8t + 4*half + 0..3 -- the P^T slot order.
  const int g16 = (lane >> 4) & 1, sj = (lane & 15) >> 2, sq = lane & 3;
  int voff[D / 32][2];
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 8 * t + 4 * half + sj;               // + 32kb + 16hh (multiple of 16)
      const int piece = 4 * dg + 2 * g16 + (sq >> 1);
      voff[dg][t] = row * ROWB + ((piece ^ swz<D>(row & 15)) << 4) + ((sq & 1) << 3);
    }

  // Lane byte offsets of the loads of a full chunk of 64 consecutive rows.
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wave * NI + i) * RPI + lane / PPR;
    loff[i] = r * ROWB + (((lane % PPR) ^ swz<D>(r & 15)) << 4);
  }
  // Buffer descriptor over `rows` rows starting at row `ks` of a head.
  auto desc = [&](const unsigned char* base, int ks, int rows) -> __amdgpu_buffer_rsrc_t {
    return make_rsrc(base + (size_t)ks * ROWB, (uint32_t)rows * (uint32_t)ROWB);
  };
  // Direct-to-LDS issue of one K or V tile. Row r comes from token ks + r
  // (uniform blocks) or tk[r] (gathered); rows >= kl load zeros.
  auto issue_tile = [&](bool isv, int ks, int kl, const int* tk) {
    uint32_t off[NI];
    const __amdgpu_buffer_rsrc_t rs = KVAR ? desc(isv ? vh : kh, 0, a.N) : desc(isv ? vh : kh, ks, rows_of(kl));
    if constexpr (KVAR) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = (wave * NI + i) * RPI + lane / PPR;
        const int t = tk[r < kl ? r : 0];
        off[i] = (r < kl && (unsigned)t < (unsigned)a.N)
                     ? (uint32_t)t * ROWB + (((lane % PPR) ^ swz<D>(r & 15)) << 4)
                     : OOB;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) off[i] = loff[i];
    }
    // separate call sites: each load names its own destination tile
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ins = wave * NI + i;
      if (isv)
        dma16(rs, Vp + ins * 1024, off[i]);
      else
        dma16(rs, Kp + ins * 1024, off[i]);
    }
  };

  // ---- chunk descriptors
  // Uniform blocks: chunk c is key block list[c] (scalar loads).
  auto chunk_uniform = [&](int c, int& ks, int& kl) {
    if (c >= cnt) { ks = 0; kl = 0; return; }
    int J = slist[c];
    J = (unsigned)J < (unsigned)a.nkb ? J : a.nkb - 1;   // invalid ids stay in bounds
    if constexpr (KMODE == 1) {
      a.kb.get(bh, J, ks, kl);         // a short block is one chunk
      kl = kl > 0 ? min(kl, 64) : kEmpty;
    } else {
      ks = J * 64;                     // uniform 64-token key blocks
      kl = min(64, a.n_valid - ks);
    }
  };
  // Gathered blocks: wave 0 writes the token indices of chunk c to the ring
  // slot tok[c & 3] with a cursor (list entry e_cur, offset off_cur).
  int e_cur = 0, off_cur = 0;
  auto next_chunk = [&](int slot) {   // wave 0 only
    int rows = 0;
    while (rows == 0 && e_cur < cnt) {
      const int ent = e_cur + lane;
      int ks = 0, n = 0;
      if (ent < cnt) {
        const int J = list[ent];
        if ((unsigned)J < (unsigned)a.nkb) a.kb.get(bh, J, ks, n);   // invalid ids: empty
        n = max(n, 0);
      }
      int incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int total = __shfl(incl, 63);
      rows = max(0, min(64, total - off_cur));
      const int pos = off_cur + lane;
      int lo = 0, hi = 64;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (__shfl(incl, mid & 63) > pos) hi = mid; else lo = mid + 1;
      }
      const int src = lo & 63;
      const int excl_src = __shfl(incl, src) - __shfl(n, src);
      const int ks_src = __shfl(ks, src);
      if (lane < rows) tok[slot * 64 + lane] = ks_src + (pos - excl_src);
      const int pend = off_cur + rows;
      int lo2 = 0, hi2 = 64;
      while (lo2 < hi2) {
        const int mid = (lo2 + hi2) >> 1;
        if (__shfl(incl, mid & 63) > pend) hi2 = mid; else lo2 = mid + 1;
      }
      if (lo2 >= 64) {
        e_cur += 64;
        off_cur = pend - total;
      } else {
        off_cur = pend - (__shfl(incl, lo2) - __shfl(n, lo2));
        e_cur += lo2;
      }
    }
    if (lane == 0) chunk_rows[slot] = rows;
  };
  auto chunk_info = [&](int c, int& ks, int& kl) {
    if constexpr (KVAR) {
      ks = 0;
      kl = __builtin_amdgcn_readfirstlane(chunk_rows[c & 3]);
    } else {
      chunk_uniform(c, ks, kl);
    }
  };

  // ---- LDS operand reads
  // K operand of S^T step j (k-step cc = j / 2, key half kb = j % 2)
  auto k_read = [&](int j) -> bf16x8 {
    const int cc = j >> 1, kb = j & 1;
    const int off = (32 * kb + l32) * ROWB + (((2 * cc + half) ^ fk) << 4);
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(Kp + off);
  };
  // V^T operand of PV step j (key half kb, 16-key group hh, channel group dg)
  auto v_read = [&](int j) -> bf16x8 {
    const int kb = j / (2 * (D / 32)), hh = (j / (D / 32)) & 1, dg = j % (D / 32);
    const int base = (32 * kb + 16 * hh) * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vp + base + voff[dg][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vp + base + voff[dg][1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int NS = D / 8;            // MFMA steps of S^T (and of PV)
  constexpr int EPS = 32 / NS;         // softmax elements per step

  // S^T = K Q^T from the K tile into s (prologue only)
  auto compute_s = [&](f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) s[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_read(j), qf[j >> 1], s[j & 1], 0, 0, 0);
  };
  // keys >= kl of a chunk get -inf
  auto mask_tail = [&](f32x16* s, int kl_s) {
    kl_s = rows_of(kl_s);
    if (kl_s < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kl_s) s[kb][r] = -INFINITY;
        }
    }
  };
  // row max in log2 units -> move the reference max when it grew by > TAU
  auto settle_max = [&](float mx) {
    const float mloc = halves_max(mx) * a.sl2;
    const bool grow = mloc > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow)) {   // rare: rescale O and l
      const float m_new = grow ? mloc : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dg][r] *= alpha;
      m_run = m_new;
    }
  };

  // ---- prologue: descriptors of chunks 0 and 1, load K0, S(0), loads K1 V0
  if constexpr (KVAR) {
    if (wave == 0) {
      next_chunk(0);
      next_chunk(1);
    }
    wait_lgkm0();
    wg_barrier();
  }
  int ks0, kl0, ks1, kl1;
  chunk_info(0, ks0, kl0);
  if (kl0 == 0) {                      // nothing kept: zero rows
    ks1 = ks0; kl1 = kl0;
  } else {
    chunk_info(1, ks1, kl1);
  }
  f32x16 sA[2], sB[2];
  int c = 0;
  int kl = kl0, ks_c = ks0;            // chunk c
  int ks_n = ks1, kl_n = kl1;          // chunk c+1

  // One pipeline iteration; sc holds S(c) (masked, reference max settled),
  // sn receives S(c+1).
  auto iter = [&](f32x16* sc, f32x16* sn) -> bool {
    int ks_2 = 0, kl_2 = 0;
    if constexpr (KVAR) {
      if (wave == 0) next_chunk((c + 2) & 3);   // ring slot of chunk c+2
    } else {
      chunk_uniform(c + 2, ks_2, kl_2);         // scalar load, lands by the barrier
    }
    // outstanding loads, oldest first: [K(c+1)] [V(c)]
    wait_vm<NI>();                     // K(c+1) landed
    wait_lgkm0();
    wg_barrier();
    if constexpr (KVAR) chunk_info(c + 2, ks_2, kl_2);

    // Region A runs at raised wave priority: when the two waves of a SIMD are
    // in different regions, the one interleaving S MFMAs with the softmax
    // issues first, keeping the MFMA pipe fed while the other's PV waits
    // (measured +4 % over equal priority; raising region B too loses it).
    __builtin_amdgcn_s_setprio(1);
    // ---- region A: S(c+1) on MFMA || P(c) = exp2(S(c) - m) on VALU.
    // Step j: K read for step j+3, MFMA j, softmax elements of step j.
    uint32_t pw[2][2][4];
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[kb][r] = 0.f;
      bf16x8 kr[4];
      kr[0] = k_read(0);
      kr[1] = k_read(1);
      kr[2] = k_read(2);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j + 3 < NS) kr[(j + 3) & 3] = k_read(j + 3);
        sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[j & 3], qf[j >> 1], sn[j & 1], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPS; e += 2) {
          const int el = j * EPS + e;            // element 0..31 of this lane
          const int kb = el >> 4, r = el & 15;
          const float x0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], a.sl2, -m_run));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r + 1], a.sl2, -m_run));
          rsum[el & 3] += x0;
          rsum[(el + 1) & 3] += x1;
          pw[kb][r >> 3][(r & 7) >> 1] = pack2(x0, x1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // keep the softmax in region A: without a use here the compiler sinks it
    // past the barriers to its consumer, region B
    asm volatile("" ::"v"(pw[0][0][0]), "v"(pw[0][0][1]), "v"(pw[0][0][2]), "v"(pw[0][0][3]),
                 "v"(pw[0][1][0]), "v"(pw[0][1][1]), "v"(pw[0][1][2]), "v"(pw[0][1][3]),
                 "v"(pw[1][0][0]), "v"(pw[1][0][1]), "v"(pw[1][0][2]), "v"(pw[1][0][3]),
                 "v"(pw[1][1][0]), "v"(pw[1][1][1]), "v"(pw[1][1][2]), "v"(pw[1][1][3]),
                 "v"(rsum[0]), "v"(rsum[1]), "v"(rsum[2]), "v"(rsum[3]));
    l_run += (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        pf[kb][hh] = __builtin_bit_cast(bf16x8, (u32x4){pw[kb][hh][0], pw[kb][hh][1], pw[kb][hh][2], pw[kb][hh][3]});

    __builtin_amdgcn_s_setprio(0);
    wg_barrier();                      // every wave is done reading K(c+1)
    {
      // K(c+2); without a chunk c+2 a re-load of a chunk that has rows
      // (c+1 if it exists, else c itself) into the free buffer
      const int kc = kl_2 > 0 ? c + 2 : (kl_n > 0 ? c + 1 : c);
      const int ks_k = kl_2 > 0 ? ks_2 : (kl_n > 0 ? ks_n : ks_c);
      const int kl_k = kl_2 > 0 ? kl_2 : (kl_n > 0 ? kl_n : kl);
      issue_tile(false, ks_k, kl_k, tok + (kc & 3) * 64);
    }

    // ---- region B: O^T += V(c)^T P(c)^T on MFMA || row max of S(c+1)
    // outstanding loads, oldest first: [V(c)] [K(c+2)]
    wait_vm<NI>();                     // V(c) landed
    wg_barrier();
    mask_tail(sn, kl_n);
    float mx = -INFINITY;
    {
      bf16x8 vr[4];
      vr[0] = v_read(0);
      vr[1] = v_read(1);
      vr[2] = v_read(2);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j + 3 < NS) vr[(j + 3) & 3] = v_read(j + 3);
        const int kb = j / (2 * (D / 32)), hh = (j / (D / 32)) & 1, dg = j % (D / 32);
        oacc[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[j & 3], pf[kb][hh], oacc[dg], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPS; e += 2) {
          const int el = j * EPS + e;
          mx = fmaxf(mx, fmaxf(sn[el >> 4][el & 15], sn[el >> 4][(el & 15) + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wg_barrier();                      // every wave is done reading V(c)
    {
      // V(c+1), or a re-load of chunk c's rows when there is no chunk c+1
      const bool more = kl_n > 0;
      const int vc = more ? c + 1 : c;
      issue_tile(true, more ? ks_n : ks_c, more ? kl_n : kl, tok + (vc & 3) * 64);
    }
    settle_max(mx);                    // reference max for S(c+1)
    // advance: chunk c+1 becomes current
    ks_c = ks_n; kl = kl_n;
    ks_n = ks_2; kl_n = kl_2;
    ++c;
    return kl > 0;
  };

  if (kl0 > 0) {
    issue_tile(false, ks0, kl0, tok);
    wait_vm<0>();                      // K0 landed
    wg_barrier();
    compute_s(sA);
    wg_barrier();
    {
      const bool more = kl1 > 0;
      issue_tile(false, more ? ks1 : ks0, more ? kl1 : kl0, tok + (more ? 1 : 0) * 64);
    }
    // V0 after K1: an iteration starts with loads outstanding in the order
    // [K(c+1)] [V(c)]
    issue_tile(true, ks0, kl0, tok);
    mask_tail(sA, kl0);
    {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sA[kb][r]);
      settle_max(mx);
    }
    for (;;) {
      if (!iter(sA, sB)) break;
      if (!iter(sB, sA)) break;
    }
  }
  wait_vm<0>();                        // no load may still target LDS

  // ---- epilogue: O = O^T / l, staged through the K tile (swizzled rows),
  // stored as bf16 rows.
  const float lt = halves_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int orow = 32 * wave + l32;
  const int fo = swz<D>(orow & 15);
  // log sum_j exp(scale s_ij) = ln 2 * (m + log2 l), m the reference max in
  // log2 units; rows with no kept key get -inf
  if (a.lse && half == 0 && orow < ql)
    a.lse[(size_t)bh * a.N + qs + orow] = lt > 0.f ? (m_run + log2f(lt)) * 0.69314718055994531f : -INFINITY;
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      // channels 32dg + 8*j4 + 4*half .. +3 = piece 4dg + j4, byte 8*half
      const u32x2 w = {pack2(oacc[dg][4 * j4 + 0] * inv, oacc[dg][4 * j4 + 1] * inv),
                       pack2(oacc[dg][4 * j4 + 2] * inv, oacc[dg][4 * j4 + 3] * inv)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          Kp + orow * ROWB + (((4 * dg + j4) ^ fo) << 4) + 8 * half) = w;
    }
  wait_lgkm0();
  wg_barrier();
  uint16_t* oh = a.o + head_off;
#pragma unroll
  for (int r = 0; r < TILE / 16 / 128; ++r) {
    const int u = tid + 128 * r;            // 16-byte piece of the 64 x D tile
    const int row = u / PPR, p = u % PPR;
    if (row < ql)
      *reinterpret_cast<u32x4*>(oh + (size_t)(qs + row) * D + p * 8) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              Kp + row * ROWB + ((p ^ swz<D>(row & 15)) << 4));
  }
}

template <int D, bool QVAR, int KMODE>
__global__ __launch_bounds__(128, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int TILE = 64 * D * 2;
  __shared__ __align__(16) unsigned char Ks[TILE];
  __shared__ __align__(16) unsigned char Vs[TILE];
  __shared__ int tok[4 * 64];
  __shared__ int chunk_rows[4];

  // Flat id -> (head, tile). Consecutive workgroups are dealt round-robin to
  // the 8 XCDs, so workgroup 8i + x is the i-th one XCD x runs; XCD x takes a
  // contiguous range of the flattened (head, tile) order. A head's tiles then
  // share one XCD's L2 (the same K/V block is not fetched into all eight L2s)
  // and the tiles running together on an XCD come from one or two heads.
  int L = blockIdx.x;
  {
    const int total = a.bh * a.tiles, per = total >> 3, rem = total & 7;
    const int x = L & 7, i = L >> 3;
    if (i >= per + (x < rem ? 1 : 0)) return;
    L = x * per + min(x, rem) + i;
  }
  const int bh = L / a.tiles;
  const int tile = L - bh * a.tiles;

  int I, qs, ql;
  if (!QVAR) {
    if (tile >= a.nqb) return;
    I = a.order ? ((const cint*)a.order)[(size_t)bh * a.nqb + tile] : tile;
    a.qb.get(bh, I, qs, ql);          // uniform, or a short block: one tile
    ql = min(ql, 64);
  } else {
    const cint* tb = (const cint*)a.tile_base + (size_t)bh * (a.nqb + 1);
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
  attn_tile<D, KMODE>(a, bh, I, qs, ql, (lds_u8*)Ks, (lds_u8*)Vs, tok, chunk_rows);
}

// Processing order of uniform query blocks: longest first. The query blocks
// of one head are sorted (counting sort) by descending number of kept key
// blocks, so the long tiles start early and do not finish last; together with
// the contiguous per-XCD ranges this keeps the XCDs busy until the end.
// Affects scheduling only: every tile computes the same bits in any order.
// With `o` given, the workgroup of head bh also zeroes that head's padding
// rows [n_valid, N) of O (cpr 16-byte pieces per row) and sets their lse to
// -inf, which spares the attention call a launch.
__global__ __launch_bounds__(256) void qorder_kernel(const int32_t* __restrict__ kv_count, int nqb, int nkb,
                                                     int32_t* __restrict__ order, uint4* __restrict__ o,
                                                     float* __restrict__ lse, int N, int n_valid, int cpr) {
  extern __shared__ int sm[];
  int* cnt = sm;              // [nkb + 1] bucket counts, then cursors
  int* key = sm + nkb + 1;    // [nqb]
  __shared__ int part[257];
  const int bh = blockIdx.x;
  if (o) {
    const size_t base = ((size_t)bh * N + n_valid) * cpr;
    for (int u = threadIdx.x; u < (N - n_valid) * cpr; u += 256) o[base + u] = make_uint4(0, 0, 0, 0);
    if (lse)
      for (int r = n_valid + threadIdx.x; r < N; r += 256) lse[(size_t)bh * N + r] = -INFINITY;
  }
  for (int b = threadIdx.x; b <= nkb; b += 256) cnt[b] = 0;
  __syncthreads();
  for (int I = threadIdx.x; I < nqb; I += 256) {
    const int c = kv_count[(size_t)bh * nqb + I];
    const int k = nkb - (c < 0 ? 0 : (c > nkb ? nkb : c));   // descending count
    key[I] = k;
    atomicAdd(&cnt[k], 1);
  }
  __syncthreads();
  // exclusive scan of the bucket counts
  const int per = (nkb + 1 + 255) / 256;
  const int b0 = threadIdx.x * per, b1 = min(nkb + 1, b0 + per);
  int loc = 0;
  for (int b = b0; b < b1; ++b) loc += cnt[b];
  part[threadIdx.x] = loc;
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
  for (int b = b0; b < b1; ++b) {
    const int v = cnt[b];
    cnt[b] = run;
    run += v;
  }
  __syncthreads();
  for (int I = threadIdx.x; I < nqb; I += 256) order[(size_t)bh * nqb + atomicAdd(&cnt[key[I]], 1)] = I;
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

__global__ __launch_bounds__(256) void zero_rows_kernel(uint4* __restrict__ o, float* __restrict__ lse, int N,
                                                        int n_valid, int cpr, size_t total) {
  const size_t per_head = (size_t)(N - n_valid) * cpr;
  for (size_t u = blockIdx.x * (size_t)256 + threadIdx.x; u < total; u += (size_t)gridDim.x * 256) {
    const size_t bh = u / per_head, rem = u % per_head;
    o[(bh * N + n_valid) * cpr + rem] = make_uint4(0, 0, 0, 0);
    if (lse && rem % cpr == 0) lse[bh * N + n_valid + rem / cpr] = -INFINITY;
  }
}

// Longest-first order of n rows per head by count (counts clamped to [0, cap]);
// false when the counting sort does not fit in LDS.
bool launch_qorder(const int32_t* counts, int BH, int n, int cap, int32_t* order, hipStream_t s) {
  const size_t lds = sizeof(int) * ((size_t)cap + 1 + n);
  if (lds > 64 * 1024) return false;
  qorder_kernel<<<BH, 256, lds, s>>>(counts, n, cap, order, nullptr, nullptr, 0, 0, 0);
  return true;
}

// Key-block count from which uniform d = 128 attention runs one wave per tile.
constexpr int kOneWaveKeyBlocks = 1024;

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int BH, int N, int d, int n_valid, const Blocks& qb, const Blocks& kb,
                           const int32_t* kv_count, const int32_t* kv_index, int kv_stride,
                           float scale, int32_t* tile_ws, float* lse, hipStream_t s) {
  if (BH == 0) return hipSuccess;
  // padding rows of O are zero (and their lse -inf): folded into the ordering
  // launch when there is one, else a launch of their own
  bool pad_done = n_valid >= N;
  auto zero_pad = [&]() {
    const int cpr = d / 8;
    const size_t total = (size_t)BH * (N - n_valid) * cpr;
    const size_t want = (total + 255) / 256;
    const int grid = (int)(want < 4096 ? want : 4096);
    zero_rows_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<uint4*>(o), lse, N, n_valid, cpr, total);
    pad_done = true;
  };
  if (qb.nblocks == 0) {
    if (!pad_done) zero_pad();
    return hipGetLastError();
  }
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.N = N; a.n_valid = n_valid; a.nqb = qb.nblocks; a.nkb = kb.nblocks;
  a.qb = qb; a.kb = kb;
  a.kv_count = kv_count; a.kv_index = kv_index; a.kv_stride = kv_stride;
  a.sl2 = scale * 1.4426950408889634f;
  a.lse = lse;
  // Uniform 64-token query blocks, and descriptor blocks the caller bounds to
  // 64 tokens, are one tile each (longest first); longer query blocks are cut
  // into 64-row tiles through a tiling table. Key blocks bounded to 64 tokens
  // are one chunk each; others are gathered row by row.
  const bool qvar = qb.start != nullptr && !(qb.max_len >= 1 && qb.max_len <= 64);
  const bool kshort = kb.start != nullptr && kb.max_len >= 1 && kb.max_len <= 64;
  const bool kvar = kb.start != nullptr && !kshort;
  const int kmode = kvar ? 2 : kshort ? 1 : 0;
  a.tile_base = tile_ws;
  a.order = nullptr;
  if (qvar) {
    tile_base_kernel<<<BH, 256, 0, s>>>(qb, tile_ws);
    a.tiles = (N + 63) / 64 + qb.nblocks;
  } else {
    a.tiles = qb.nblocks;
    const size_t lds = sizeof(int) * ((size_t)kb.nblocks + 1 + qb.nblocks);
    if (lds <= 64 * 1024) {
      int32_t* order = tile_ws;
      qorder_kernel<<<BH, 256, lds, s>>>(kv_count, qb.nblocks, kb.nblocks, order,
                                         pad_done ? nullptr : reinterpret_cast<uint4*>(o), lse, N, n_valid,
                                         d / 8);
      a.order = order;
      pad_done = true;
    }
  }
  if (!pad_done) zero_pad();
  a.bh = BH;
  const long long grid = 8LL * (((long long)BH * a.tiles + 7) / 8);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // Rows over many key blocks (large heads) leave the kernel bound by K/V
  // traffic that mostly misses L2; there one wave per 64-row tile, which
  // shares each K/V operand read between both query halves, does better
  // (measured at 1857 key blocks: +8..11 %; at 512: -12 %).
  if (d == 128 && !qvar && qb.start == nullptr && kmode == 0 && a.order && kb.nblocks >= kOneWaveKeyBlocks)
    return launch_attn_fwd_1w(a, (int)grid, s);
#define BSA_ATTN(DD, QV, KM) attn_fwd_kernel<DD, QV, KM><<<(int)grid, 128, 0, s>>>(a)
#define BSA_ATTN_K(DD, QV)               \
  do {                                   \
    if (kmode == 2) BSA_ATTN(DD, QV, 2); \
    else if (kmode == 1) BSA_ATTN(DD, QV, 1); \
    else BSA_ATTN(DD, QV, 0);            \
  } while (0)
  if (d == 128) {
    if (qvar) BSA_ATTN_K(128, true);
    else BSA_ATTN_K(128, false);
  } else {
    if (qvar) BSA_ATTN_K(64, true);
    else BSA_ATTN_K(64, false);
  }
#undef BSA_ATTN_K
#undef BSA_ATTN
  return hipGetLastError();
}

}  // namespace bsa

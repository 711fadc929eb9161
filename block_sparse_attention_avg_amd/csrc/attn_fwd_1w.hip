// Block-sparse flash-attention forward, one-wave variant for uniform 64-token
// blocks at d = 128 (NABLA summary, Metodologia section 2, "Espansione": only
// the kept N x N tiles are computed). The launcher in attn_fwd.hip picks it
// for rows over many key blocks (the 118k-token layer), where K/V traffic
// mostly misses L2: one wave per 64-row query tile shares every K and V
// operand read between two 32-row query halves, so a CU keeps the same
// number of tiles in flight with half the LDS reads per MFMA.
//
// Work item: one 64-row query tile of one head on one wave (a one-wave
// workgroup). The kept key blocks of the tile's query block are walked in
// ascending order, one 64-key chunk per block.
//
// Data movement: K and V chunks go HBM -> LDS with direct-to-LDS buffer loads
// (no staging registers), row-major, each row's 16-byte pieces XOR-swizzled so
// that both the K operand reads and the transposed V reads below are free of
// bank conflicts. The next chunk's K is in flight while this chunk's softmax
// and PV run, the next V while the next S runs. Waits are explicit vmcnt
// counts; a single wave needs no barrier.
//
// Math per chunk (two 32-row query halves qh share each operand read):
//   S^T = K Q^T        bf16 MFMA 32x32x16; Q^T stays in registers as the B
//                      operand for the whole tile, so each lane ends up with
//                      32 key scores of one query per half: max/sum are
//                      lane-local plus one permlane32 swap with the lane
//                      holding the other 32.
//   online softmax     fp32, log2 domain (scale*log2e folded into one FMA),
//                      O rescaled only when some row max grew by > 2^64.
//   O^T += V^T P^T     bf16 MFMA 32x32x16; P^T is the S^T accumulator
//                      rounded to bf16 in registers (hardware convert), and
//                      V^T comes straight from the row-major V tile through the
//                      LDS transpose read (ds_read_b64_tr_b16), addressed so
//                      its key order matches the accumulator layout of S^T.
// O is divided by the row sum once at the end, staged through LDS and
// written as bf16 rows.
#include "lds_tile.h"

#include <math.h>

namespace bsa {

// One query tile of 64 rows on ONE wave. The two 32-row halves qh = 0, 1 of
// the MFMA output share every K and V operand read from LDS (half the LDS
// traffic per FLOP of two 32-row waves), and a one-wave workgroup needs no
// barrier: LDS reads and refills are ordered by the wave's own waits. K and V
// tiles are separate LDS arrays so the compiler can tell the two
// direct-to-LDS load streams apart; all waits on those loads are explicit
// vmcnt counts.
//
// Software pipeline (iteration c):
//   region A:  S(c+1) = K(c+1) Q^T on MFMA, interleaved instruction by
//              instruction with exp2 / row sum / bf16 pack of S(c) on the
//              VALU (independent work, so the two pipes overlap);
//   region B:  O^T += V(c)^T P(c)^T on MFMA, interleaved with the row max of
//              S(c+1); then the rare rescale of O for S(c+1)'s max.
// K(c+2) is issued when region A has read K(c+1), V(c+1) when region B has
// read V(c). Each iteration issues exactly one K and one V tile load (after
// the last chunk they re-load rows of a chunk that exists into the free
// buffer, and the extra S is discarded), so the number of loads in flight is
// the same on every path. The loop body is unrolled twice so S(c) and S(c+1)
// swap registers instead of being copied.
//
// Loads go through buffer descriptors that end at the chunk's last row: rows
// past it (a partial last block, gathered rows past the chunk) read as zeros,
// so no clamping is needed and padding never reaches P V.
template <int D>
__device__ __forceinline__ void attn_tile_1w(const AttnArgs& a, int bh, int I, int qs, int ql,
                                             lds_u8* Kp, lds_u8* Vp) {
  constexpr int ROWB = D * 2;                  // bytes per K/V row
  constexpr int TILE = 64 * ROWB;              // bytes per K or V tile
  constexpr int NI = TILE / 1024;              // direct-to-LDS loads per tile
  constexpr int RPI = 1024 / ROWB;             // rows per load instruction
  constexpr int PPR = ROWB / 16;               // 16-byte pieces per row
  // rescale O only when a row max grows by > 2^TAU: until then P <= 2^TAU,
  // and O, l stay far inside fp32 / bf16 range (their ratio is unaffected);
  // a small TAU would rescale on most chunks, since any of the 64 rows can
  // trigger it
  constexpr float TAU = 64.f;
  constexpr uint32_t OOB = 0xFFFFFFF0u;        // lane offset past every descriptor: loads zeros
  constexpr int NS = D / 8;                    // K (and V) operand reads per chunk
  constexpr int EPS = 64 / NS;                 // softmax elements per lane per read

  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const size_t head_off = (size_t)bh * a.N * D;
  const uint16_t* qh_ = a.q + head_off;
  const unsigned char* kh = reinterpret_cast<const unsigned char*>(a.k + head_off);
  const unsigned char* vh = reinterpret_cast<const unsigned char*>(a.v + head_off);

  // Q^T as MFMA B operand: lane supplies Q[32qh + l32][16c + 8*half .. +7].
  bf16x8 qf[2][D / 16];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int qr = 32 * q2 + l32;
    const bool ok = qr < ql;
    const uint16_t* src = qh_ + (size_t)(qs + (ok ? qr : 0)) * D + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(src + 16 * c) : make_uint4(0, 0, 0, 0);
      qf[q2][c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 oacc[D / 32][2];
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dg][q2][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const size_t qrow = (size_t)bh * a.nqb + I;
  // counts outside [0, kv_stride] (a caller's contract) stay inside the row
  const int cnt = min(max(((const cint*)a.kv_count)[qrow], 0), a.kv_stride);
  const int32_t* list = a.kv_index + qrow * a.kv_stride;
  const cint* slist = (const cint*)list;

  // ---- per-lane LDS offsets (loop invariant)
  const KvOperands<D> kvo(lane);
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = i * RPI + lane / PPR;
    loff[i] = r * ROWB + (((lane % PPR) ^ swz<D>(r & 15)) << 4);
  }
  auto desc = [&](const unsigned char* base, int ks, int rows) -> __amdgpu_buffer_rsrc_t {
    return make_rsrc(base + (size_t)ks * ROWB, (uint32_t)rows * (uint32_t)ROWB);
  };
  // rows >= kl of the chunk read as zeros: the descriptor ends at row kl
  auto issue_tile = [&](bool isv, int ks, int kl) {
    const __amdgpu_buffer_rsrc_t rs = desc(isv ? vh : kh, ks, kl);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (isv)
        dma16(rs, Vp + i * 1024, loff[i]);
      else
        dma16(rs, Kp + i * 1024, loff[i]);
    }
  };

  // ---- chunk descriptors: chunk c is key block list[c] (scalar loads)
  auto chunk_info = [&](int c, int& ks, int& kl) {
    if (c >= cnt) { ks = 0; kl = 0; return; }
    int J = slist[c];
    J = (unsigned)J < (unsigned)a.nkb ? J : a.nkb - 1;   // invalid ids stay in bounds
    ks = J * 64;
    kl = min(64, a.n_valid - ks);
  };

  // ---- LDS operand reads
  auto k_read = [&](int j) -> bf16x8 { return kvo.k(Kp, j); };
  auto v_read = [&](int j) -> bf16x8 { return kvo.v(Vp, j); };
  // S[kb][qh] (s has 4 accumulators, index 2*kb + qh)
  auto compute_s = [&](f32x16* s) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[x][r] = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bf16x8 ka = k_read(j);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
        s[2 * (j & 1) + q2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[q2][j >> 1], s[2 * (j & 1) + q2], 0, 0, 0);
    }
  };
  auto mask_tail = [&](f32x16* s, int kl_s) {
    if (kl_s < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= kl_s) s[2 * kb + q2][r] = -INFINITY;
          }
    }
  };
  auto settle_max = [&](const float* mx) {
    float mloc[2];
    bool grow[2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      mloc[q2] = halves_max(mx[q2]) * a.sl2;
      grow[q2] = mloc[q2] > m_run[q2] + TAU;
    }
    if (__builtin_amdgcn_ballot_w64(grow[0] || grow[1])) {   // rare: rescale O and l
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const float m_new = grow[q2] ? mloc[q2] : m_run[q2];
        const float alpha = __builtin_amdgcn_exp2f(m_run[q2] - m_new);
        l_run[q2] *= alpha;
#pragma unroll
        for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dg][q2][r] *= alpha;
        m_run[q2] = m_new;
      }
    }
  };

  // ---- prologue
  int ks0, kl0, ks1, kl1;
  chunk_info(0, ks0, kl0);
  if (kl0 == 0) {
    ks1 = ks0; kl1 = kl0;
  } else {
    chunk_info(1, ks1, kl1);
  }
  f32x16 sA[4], sB[4];
  int c = 0;
  int kl = kl0, ks_c = ks0;
  int ks_n = ks1, kl_n = kl1;

  auto iter = [&](f32x16* sc, f32x16* sn) -> bool {
    int ks_2 = 0, kl_2 = 0;
    chunk_info(c + 2, ks_2, kl_2);
    // outstanding loads, oldest first: [K(c+1)] [V(c)]
    wait_vm<NI>();                     // K(c+1) landed
    wait_lgkm0();
    asm volatile("" ::: "memory");

    // ---- region A: S(c+1) on MFMA || P(c) on VALU
    uint32_t pw[2][2][2][4];           // [kb][hh][qh][word]
    {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[x][r] = 0.f;
      bf16x8 kr[4];
      kr[0] = k_read(0);
      kr[1] = k_read(1);
      kr[2] = k_read(2);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j + 3 < NS) kr[(j + 3) & 3] = k_read(j + 3);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
          sn[2 * (j & 1) + q2] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[j & 3], qf[q2][j >> 1], sn[2 * (j & 1) + q2], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPS; e += 2) {
          const int el = j * EPS + e;            // element 0..63: qh, kb, r
          const int q2 = el >> 5, kb = (el >> 4) & 1, r = el & 15;
          const float x0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * kb + q2][r], a.sl2, -m_run[q2]));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * kb + q2][r + 1], a.sl2, -m_run[q2]));
          pw[kb][r >> 3][q2][(r & 7) >> 1] = pack2(x0, x1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // keep the softmax in region A: without a use here the compiler sinks it
    // past the refill of the K tile to its consumer, region B
    asm volatile("" ::"v"(pw[0][0][0][0]), "v"(pw[0][0][0][1]), "v"(pw[0][0][0][2]), "v"(pw[0][0][0][3]),
                 "v"(pw[0][0][1][0]), "v"(pw[0][0][1][1]), "v"(pw[0][0][1][2]), "v"(pw[0][0][1][3]),
                 "v"(pw[0][1][0][0]), "v"(pw[0][1][0][1]), "v"(pw[0][1][0][2]), "v"(pw[0][1][0][3]),
                 "v"(pw[0][1][1][0]), "v"(pw[0][1][1][1]), "v"(pw[0][1][1][2]), "v"(pw[0][1][1][3]));
    asm volatile("" ::"v"(pw[1][0][0][0]), "v"(pw[1][0][0][1]), "v"(pw[1][0][0][2]), "v"(pw[1][0][0][3]),
                 "v"(pw[1][0][1][0]), "v"(pw[1][0][1][1]), "v"(pw[1][0][1][2]), "v"(pw[1][0][1][3]),
                 "v"(pw[1][1][0][0]), "v"(pw[1][1][0][1]), "v"(pw[1][1][0][2]), "v"(pw[1][1][0][3]),
                 "v"(pw[1][1][1][0]), "v"(pw[1][1][1][1]), "v"(pw[1][1][1][2]), "v"(pw[1][1][1][3]));
    bf16x8 pf[2][2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
          pf[kb][hh][q2] = __builtin_bit_cast(
              bf16x8, (u32x4){pw[kb][hh][q2][0], pw[kb][hh][q2][1], pw[kb][hh][q2][2], pw[kb][hh][q2][3]});

    wait_lgkm0();                      // K(c+1) reads done before the buffer is refilled
    asm volatile("" ::: "memory");
    {
      // K(c+2); without a chunk c+2 a re-load of c+1 (or c) into the free
      // buffer keeps every iteration's loads in step
      const int ks_k = kl_2 > 0 ? ks_2 : (kl_n > 0 ? ks_n : ks_c);
      const int kl_k = kl_2 > 0 ? kl_2 : (kl_n > 0 ? kl_n : kl);
      issue_tile(false, ks_k, kl_k);
    }

    // ---- region B: O^T += V(c)^T P(c)^T || row max of S(c+1)
    // outstanding loads, oldest first: [V(c)] [K(c+2)]
    wait_vm<NI>();                     // V(c) landed
    asm volatile("" ::: "memory");
    mask_tail(sn, kl_n);
    float mx[2] = {-INFINITY, -INFINITY};
    // row sums of the bf16-rounded P that PV multiplies (so the output is a
    // convex combination with exactly the weights used), one bf16 dot
    // product with (1, 1) per packed pair, in the VALU slack of region B
    float rsum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    {
      bf16x8 vr[4];
      vr[0] = v_read(0);
      vr[1] = v_read(1);
      vr[2] = v_read(2);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j + 3 < NS) vr[(j + 3) & 3] = v_read(j + 3);
        const int kb = j / (2 * (D / 32)), hh = (j / (D / 32)) & 1, dg = j % (D / 32);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
          oacc[dg][q2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[j & 3], pf[kb][hh][q2], oacc[dg][q2], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPS; e += 2) {
          const int el = j * EPS + e;
          const int q2 = el >> 5, kb2 = (el >> 4) & 1, r = el & 15;
          mx[q2] = fmaxf(mx[q2], fmaxf(sn[2 * kb2 + q2][r], sn[2 * kb2 + q2][r + 1]));
        }
        // the 8 words of pf[kb][hh][*] are summed over the D/32 steps that use them
#pragma unroll
        for (int u = 0; u < 8 / (D / 32); ++u) {
          const int wi = dg * (8 / (D / 32)) + u;          // word 0..7 of this (kb, hh)
          const int q2 = wi >> 2;
          rsum[q2][u & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[kb][hh][q2][wi & 3]),
                                                            __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                                            rsum[q2][u & 1], false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) l_run[q2] += rsum[q2][0] + rsum[q2][1];
    wait_lgkm0();                      // V(c) reads done before the buffer is refilled
    asm volatile("" ::: "memory");
    {
      const bool more = kl_n > 0;
      issue_tile(true, more ? ks_n : ks_c, more ? kl_n : kl);
    }
    settle_max(mx);
    ks_c = ks_n; kl = kl_n;
    ks_n = ks_2; kl_n = kl_2;
    ++c;
    return kl > 0;
  };

  if (kl0 > 0) {
    issue_tile(false, ks0, kl0);
    wait_vm<0>();
    asm volatile("" ::: "memory");
    compute_s(sA);
    wait_lgkm0();
    asm volatile("" ::: "memory");
    {
      const bool more = kl1 > 0;
      issue_tile(false, more ? ks1 : ks0, more ? kl1 : kl0);
    }
    issue_tile(true, ks0, kl0);
    mask_tail(sA, kl0);
    {
      float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx[q2] = fmaxf(mx[q2], sA[2 * kb + q2][r]);
      settle_max(mx);
    }
    for (;;) {
      if (!iter(sA, sB)) break;
      if (!iter(sB, sA)) break;
    }
  }
  wait_vm<0>();                        // no load may still target LDS
  asm volatile("" ::: "memory");

  // ---- epilogue: O = O^T / l, staged through the K tile, stored as bf16 rows
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const float lt = halves_sum(l_run[q2]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int orow = 32 * q2 + l32;
    const int fo = swz<D>(orow & 15);
    if (a.lse && half == 0 && orow < ql)
      a.lse[(size_t)bh * a.N + qs + orow] =
          lt > 0.f ? (m_run[q2] + log2f(lt)) * 0.69314718055994531f : -INFINITY;
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const u32x2 w = {pack2(oacc[dg][q2][4 * j4 + 0] * inv, oacc[dg][q2][4 * j4 + 1] * inv),
                         pack2(oacc[dg][q2][4 * j4 + 2] * inv, oacc[dg][q2][4 * j4 + 3] * inv)};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
            Kp + orow * ROWB + (((4 * dg + j4) ^ fo) << 4) + 8 * half) = w;
      }
  }
  wait_lgkm0();
  asm volatile("" ::: "memory");
  uint16_t* oh = a.o + head_off;
#pragma unroll
  for (int r = 0; r < TILE / 16 / 64; ++r) {
    const int u = lane + 64 * r;            // 16-byte piece of the 64 x D tile
    const int row = u / PPR, p = u % PPR;
    if (row < ql)
      *reinterpret_cast<u32x4*>(oh + (size_t)(qs + row) * D + p * 8) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              Kp + row * ROWB + ((p ^ swz<D>(row & 15)) << 4));
  }
}

// Uniform 64-token query blocks only (a.order set); one wave per workgroup.
__global__ __launch_bounds__(64) void attn_fwd_1w_kernel(AttnArgs a) {
  constexpr int D = 128;
  constexpr int TILE = 64 * D * 2;
  __shared__ __align__(16) unsigned char Ks[TILE];
  __shared__ __align__(16) unsigned char Vs[TILE];

  // Flat id -> (head, tile), as in the two-wave kernel: workgroup 8i + x is
  // the i-th one XCD x runs, and XCD x takes a contiguous range of the
  // flattened (head, tile) order, so a head's K/V stays in one XCD's L2.
  int L = blockIdx.x;
  {
    const int total = a.bh * a.tiles, per = total >> 3, rem = total & 7;
    const int x = L & 7, i = L >> 3;
    if (i >= per + (x < rem ? 1 : 0)) return;
    L = x * per + min(x, rem) + i;
  }
  const int bh = L / a.tiles;
  const int tile = L - bh * a.tiles;
  if (tile >= a.nqb) return;
  const int I = ((const cint*)a.order)[(size_t)bh * a.nqb + tile];
  int qs, ql;
  a.qb.get(bh, I, qs, ql);
  if (ql <= 0) return;
  attn_tile_1w<D>(a, bh, I, qs, ql, (lds_u8*)Ks, (lds_u8*)Vs);
}

hipError_t launch_attn_fwd_1w(const AttnArgs& a, int grid, hipStream_t s) {
  attn_fwd_1w_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bsa

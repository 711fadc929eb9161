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
#include "lds_tile.h"

#include <math.h>

namespace bsa {

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
// Loads and barriers, two per iteration: at the top every wave waits for its
// share of K(c+1), and the barrier then also tells that every wave is done
// with region B of c-1, so V(c) goes out into the free V buffer (it lands
// during region A). After region A every wave waits for its share of V(c);
// the second barrier also tells that K(c+1) has been read, so K(c+2) goes
// out (it lands during region B). One tile is in flight at each wait. After
// the last chunk no K is loaded and the extra S (from the stale buffer) is
// discarded. The loop body is unrolled twice so S(c) and S(c+1) swap
// registers instead of being copied.
//
// Loads go through buffer descriptors that end at the chunk's last row:
// rows past it (a partial last block, gathered rows past the chunk) read as
// zeros, so no clamping is needed and padding never reaches P V.
// Key blocks: KMODE 0 = uniform 64-token blocks, 1 = descriptor blocks of at
// most 64 tokens (each one chunk, loaded like a uniform block from its own
// start), 2 = descriptor blocks of any length (keys gathered row by row into
// 64-key chunks), 3 = descriptor blocks of any length as contiguous runs
// (each kept block cut into 64-key chunks from its own start, the last one
// partial: no gathering, at the price of the partial chunks).
template <int D>
__device__ __forceinline__ void store_rows(const AttnArgs& a, int bh, int qs, int ql, const f32x16* oacc,
                                           float m_run, float l_run, lds_u8* Kp);

// The tile walks the `cnt` list entries from `list` (a query block's whole
// kept list, or one key segment of it). With `part` set it ends by storing
// its unnormalised partial result there instead of output rows; with
// `mslots` set (the slots of its query block's segments, its own being
// `s_own`) it combines the other segments' partial results with its own
// before writing the rows.
template <int D, int KMODE>
__device__ __forceinline__ void attn_tile(const AttnArgs& a, int bh, int I, int qs, int ql,
                                          const int32_t* list, int cnt, float* part, const cint* mslots,
                                          int s_own, lds_u8* Kp, lds_u8* Vp, int* tok, int* chunk_rows) {
  constexpr int ROWB = D * 2;                  // bytes per K/V row
  constexpr int TILE = 64 * ROWB;              // bytes per K or V tile
  constexpr int NI = TILE / 1024 / 2;          // direct-to-LDS loads per wave per tile
  constexpr int RPI = 1024 / ROWB;             // rows per load instruction
  constexpr int PPR = ROWB / 16;               // 16-byte pieces per row
  constexpr float TAU = 8.f;                   // rescale O only when a row max grows by > 2^TAU
  constexpr uint32_t OOB = 0xFFFFFFF0u;        // lane offset past every descriptor: loads zeros
  constexpr bool KVAR = KMODE == 2;            // gathered keys
  constexpr bool KRUN = KMODE == 3;            // runs
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

  const cint* slist = (const cint*)list;

  // ---- per-lane LDS offsets (loop invariant)
  const KvOperands<D> kvo(lane);

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
  // Runs: a cursor (entry, piece) over the kept blocks, advanced once per
  // chunk in chunk order (scalar loads; blocks without tokens and invalid
  // ids give no chunk).
  int r_e = 0, r_p = 0;
  auto next_run = [&](int& ks, int& kl) {
    ks = 0;
    kl = 0;
    while (r_e < cnt) {
      const int J = slist[r_e];
      int st = 0, n = 0;
      if ((unsigned)J < (unsigned)a.nkb) a.kb.get(bh, J, st, n);
      if (64 * r_p < n) {
        ks = st + 64 * r_p;
        kl = min(64, n - 64 * r_p);
        ++r_p;
        return;
      }
      ++r_e;
      r_p = 0;
    }
  };
  // Uniform blocks: chunk c is key block list[c] (scalar loads).
  auto chunk_uniform = [&](int c, int& ks, int& kl) {
    if constexpr (KRUN) {
      next_run(ks, kl);                // chunks are asked for in order
      return;
    }
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
  auto k_read = [&](int j) -> bf16x8 { return kvo.k(Kp, j); };
  // V^T operand of PV step j (key half kb, 16-key group hh, channel group dg)
  auto v_read = [&](int j) -> bf16x8 { return kvo.v(Vp, j); };
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
    // outstanding: K(c+1) only
    wait_vm<0>();                      // this wave's share of K(c+1) landed
    wait_lgkm0();
    wg_barrier();                      // every share landed; every wave is done with V(c-1)
    if constexpr (KVAR) chunk_info(c + 2, ks_2, kl_2);
    issue_tile(true, ks_c, kl, tok + (c & 3) * 64);   // V(c), lands during region A

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
    wait_vm<0>();                      // this wave's share of V(c) landed
    wg_barrier();                      // every share landed; every wave is done reading K(c+1)
    if (kl_2 > 0) issue_tile(false, ks_2, kl_2, tok + ((c + 2) & 3) * 64);   // K(c+2), lands during region B

    // ---- region B: O^T += V(c)^T P(c)^T on MFMA || row max of S(c+1)
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
    if (kl1 > 0) issue_tile(false, ks1, kl1, tok + 64);   // K1; V0 goes out in the first iteration
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

  if (part) {
    // partial result of one key segment: the registers as they are (rows of
    // both waves, [wave][dg][r/4][lane][4]), then the reference max and row
    // sum of each lane; combined by the query block's last item
    if constexpr (D == 128) {
      const int w64 = wave * 64 + lane;
#pragma unroll
      for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(part + (((wave * (D / 32) + dg) * 4 + r4) * 64 + lane) * 4) =
              (f32x4){oacc[dg][4 * r4], oacc[dg][4 * r4 + 1], oacc[dg][4 * r4 + 2], oacc[dg][4 * r4 + 3]};
      part[2 * (D / 32) * 16 * 64 + w64] = m_run;
      part[2 * (D / 32) * 16 * 64 + 128 + w64] = l_run;
    }
    return;
  }
  if (mslots) {
    // the query block's last item: every segment's partial (its own from
    // the registers) rescaled to the largest reference max and summed in
    // segment order, so the rows do not depend on which item ran last
    if constexpr (D == 128) {
      constexpr int MOFF = 2 * (D / 32) * 16 * 64;
      const float* base = a.part + (size_t)bh * a.max_items * kSplitSlotFloats;
      const int w64 = wave * 64 + lane;
      float m = -1e30f;
      for (int s = 0; s < a.nsegs; ++s) {
        const int k = mslots[s];
        if (s == s_own)
          m = fmaxf(m, m_run);
        else if (k >= 0)
          m = fmaxf(m, base[(size_t)k * kSplitSlotFloats + MOFF + w64]);
      }
      // the own segment is the block's highest: its term starts the sum
      const float w0 = __builtin_amdgcn_exp2f(m_run - m);
      float l = l_run * w0;
#pragma unroll
      for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dg][r] *= w0;
      for (int s = 0; s < s_own; ++s) {
        const int k = mslots[s];
        if (k < 0) continue;
        const float* p = base + (size_t)k * kSplitSlotFloats;
        const float w = __builtin_amdgcn_exp2f(p[MOFF + w64] - m);
        l += p[MOFF + 128 + w64] * w;
#pragma unroll
        for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 x =
                *reinterpret_cast<const f32x4*>(p + (((wave * (D / 32) + dg) * 4 + r4) * 64 + lane) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[dg][4 * r4 + j] += x[j] * w;
          }
      }
      store_rows<D>(a, bh, qs, ql, oacc, m, l, Kp);
    }
    return;
  }
  store_rows<D>(a, bh, qs, ql, oacc, m_run, l_run, Kp);
}

// Epilogue of a 64-row tile (two waves, wave w owning rows 32w..32w+31):
// O = O^T / l, staged through LDS (swizzled rows) and stored as bf16 rows,
// plus the row log-normaliser when asked for. l_run is each lane's partial
// row sum (the two wave halves hold the two halves of a row's keys).
template <int D>
__device__ __forceinline__ void store_rows(const AttnArgs& a, int bh, int qs, int ql, const f32x16* oacc,
                                           float m_run, float l_run, lds_u8* Kp) {
  constexpr int ROWB = D * 2;
  constexpr int TILE = 64 * ROWB;
  constexpr int PPR = ROWB / 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const size_t head_off = (size_t)bh * a.N * D;
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

// Blocks of any length: runs when cutting each kept block into its own
// 64-key chunks costs at most twice the chunks of packing the keys densely
// (then no token lists are built per chunk); else gathering. A gathered
// chunk costs more than 1.5 run chunks (one wave builds its token list
// while the others wait), so runs win up to about twice the chunks. Every
// wave computes the same answer.
__device__ __forceinline__ bool runs_pay(const AttnArgs& a, int bh, const int32_t* list, int cnt) {
  const int lane = threadIdx.x & 63;
  int padded = 0, keys = 0;
  for (int e0 = 0; e0 < cnt; e0 += 64) {
    const int e = e0 + lane;
    int n = 0;
    if (e < cnt) {
      const int J = list[e];
      int st = 0;
      if ((unsigned)J < (unsigned)a.nkb) a.kb.get(bh, J, st, n);
      n = max(n, 0);
    }
    padded += (n + 63) >> 6;
    keys += n;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    padded += __shfl_xor(padded, o);
    keys += __shfl_xor(keys, o);
  }
  return padded <= 2 * ((keys + 63) >> 6);
}

template <int D, bool QVAR, int KMODE, bool SPLIT>
__global__ __launch_bounds__(128, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int TILE = 64 * D * 2;
  __shared__ __align__(16) unsigned char Ks[TILE];
  __shared__ __align__(16) unsigned char Vs[TILE];
  __shared__ int tok[4 * 64];
  __shared__ int chunk_rows[4];

  if constexpr (SPLIT) {
    // One item (query block, key segment) per workgroup. The grid is an upper
    // bound; the launch's items of all heads are dealt to the XCDs as
    // contiguous ranges of their order (head, then segment, then longest
    // first), so the tiles running together on an XCD read the same key
    // segment of a head.
    const int total = ((const cint*)a.item_base)[a.bh];
    const int L = blockIdx.x, x = L & 7, i = L >> 3;
    const int per = total >> 3, rem = total & 7;
    if (i >= per + (x < rem ? 1 : 0)) return;
    const int flat = x * per + min(x, rem) + i;
    int lo = 0, hi = a.bh - 1;                  // position: last p with item_base[p] <= flat
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (((const cint*)a.item_base)[mid] <= flat) lo = mid; else hi = mid - 1;
    }
    const int bh = ((const cint*)a.head_order)[lo];
    const int k = flat - ((const cint*)a.item_base)[lo] + (a.item_first ? ((const cint*)a.item_first)[bh] : 0);
    const cint* it = (const cint*)a.items + ((size_t)bh * a.max_items + k) * 4;
    const int I = it[0], off = it[1], cnt = it[2], s_own = it[3];
    int qs, ql;
    a.qb.get(bh, I, qs, ql);
    ql = min(ql, 64);
    if (ql <= 0) return;
    const size_t qrow = (size_t)bh * a.nqb + I;
    // first items store their partial result; a last item merges when its
    // query block has more than one, else writes its rows
    const bool many = ((const cint*)a.nseg)[qrow] > 1;
    float* part = !a.item_first && many ? a.part + ((size_t)bh * a.max_items + k) * kSplitSlotFloats : nullptr;
    const cint* mslots = a.item_first && many ? (const cint*)a.slot_of + qrow * a.nsegs : nullptr;
    attn_tile<D, KMODE>(a, bh, I, qs, ql, a.kv_index + qrow * a.kv_stride + off, cnt, part, mslots, s_own,
                        (lds_u8*)Ks, (lds_u8*)Vs, tok, chunk_rows);
    return;
  }

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
  const size_t qrow = (size_t)bh * a.nqb + I;
  // counts outside [0, kv_stride] (a caller's contract) stay inside the row
  const int cnt = min(max(((const cint*)a.kv_count)[qrow], 0), a.kv_stride);
  const int32_t* list = a.kv_index + qrow * a.kv_stride;
  if constexpr (KMODE == 2) {
    if (runs_pay(a, bh, list, cnt)) {
      attn_tile<D, 3>(a, bh, I, qs, ql, list, cnt, nullptr, nullptr, 0, (lds_u8*)Ks, (lds_u8*)Vs, tok, chunk_rows);
      return;
    }
  }
  attn_tile<D, KMODE>(a, bh, I, qs, ql, list, cnt, nullptr, nullptr, 0, (lds_u8*)Ks, (lds_u8*)Vs, tok, chunk_rows);
}

// ---- split over key segments (uniform blocks, long rows)
//
// Per head, the kept list of every query block is cut where the key block id
// crosses a multiple of `sg` into at most `nsegs` segments; every non-empty
// (query block, segment) pair is an item, computed by one workgroup of the
// forward above. Two launches: the first runs every item but the last
// (highest segment) of each query block and stores their partial results;
// the second runs the last items, which combine the block's partials with
// their own and write its rows. The items of a launch are ordered
// segment-major (longest first inside a segment): tiles that run together
// on an XCD then read the K/V blocks of one key segment, which its L2 holds
// while they are reused. Scheduling only: every partial is the exact online
// softmax of its segment's keys, merged in segment order.
// Where each key segment starts in every query block's (ascending) list, one
// wave per query block: segoff[row][s] = number of entries below s * sg;
// nseg[row] = number of non-empty segments; slot_of[row][*] = -1. A query
// block with no kept key block (no item) gets its zero rows and lse -inf
// here.
__global__ __launch_bounds__(1024) void split_rows_kernel(const int32_t* __restrict__ kv_count,
                                                          const int32_t* __restrict__ kv_index, int kv_stride,
                                                          int nqb, int nsegs, int sg, int32_t* __restrict__ segoff,
                                                          int32_t* __restrict__ slot_of,
                                                          int32_t* __restrict__ nseg, uint4* __restrict__ o,
                                                          float* __restrict__ lse, int N, int n_valid) {
  const int lane = threadIdx.x & 63;
  const int I = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (I >= nqb) return;
  const size_t row = (size_t)blockIdx.y * nqb + I;
  const int cnt = min(max(kv_count[row], 0), kv_stride);
  const int32_t* lst = kv_index + row * kv_stride;
  int below = 0;                        // lane s: entries below s * sg
  for (int c0 = 0; c0 < cnt; c0 += 64) {
    const int J = c0 + lane < cnt ? lst[c0 + lane] : 0x7fffffff;
    for (int s = 1; s < nsegs; ++s) {
      const unsigned long long b = __ballot(J < s * sg);
      if (lane == s) below += __popcll(b);
    }
  }
  if (lane >= nsegs) below = cnt;      // lane nsegs: end of the list
  const int nxt = __shfl_down(below, 1);
  const int c_s = lane < nsegs ? nxt - below : 0;
  if (lane < nsegs) {
    segoff[row * nsegs + lane] = below;
    slot_of[row * nsegs + lane] = -1;
  }
  const int ns = __popcll(__ballot(c_s > 0));
  if (lane == 0) nseg[row] = ns;
  if (ns == 0) {                        // uniform 64-token query blocks, d = 128: 16 pieces per row
    const int qs = 64 * I, ql = min(64, n_valid - qs);
    const size_t r0 = (size_t)blockIdx.y * N + qs;
    for (int u = lane; u < 16 * ql; u += 64) o[r0 * 16 + u] = make_uint4(0, 0, 0, 0);
    if (lse && lane < ql) lse[r0 + lane] = -INFINITY;
  }
}

// Item order of one head (one workgroup): a counting sort of the non-empty
// (query block, segment) pairs by last-of-their-block (the other items
// first), then by segment, then by descending count. n_first[bh] = number of
// items that are not the last of their query block.
__global__ __launch_bounds__(1024) void split_plan_kernel(const int32_t* __restrict__ kv_count, int kv_stride,
                                                          int nqb, int nsegs, int sg, int max_items,
                                                          const int32_t* __restrict__ segoff,
                                                          int32_t* __restrict__ items, int32_t* __restrict__ slot_of,
                                                          int32_t* __restrict__ n_items, int32_t* __restrict__ n_first,
                                                          int32_t* __restrict__ head_work) {
  extern __shared__ int hist[];          // [2 * nsegs * (sg + 1)] bucket counts, then cursors
  __shared__ int part[1025];
  __shared__ int work;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int half = nsegs * (sg + 1);     // buckets of the first items; the last items' follow
  const int nbk = 2 * half;
  const int npairs = nqb * nsegs;
  for (int b = tid; b < nbk; b += 1024) hist[b] = 0;
  if (tid == 0) work = 0;
  __syncthreads();
  {
    // kept tiles of the head: the XCD balance of the item order
    int w = 0;
    for (int I = tid; I < nqb; I += 1024) w += min(max(kv_count[(size_t)bh * nqb + I], 0), kv_stride);
    for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o);
    if ((tid & 63) == 0) atomicAdd(&work, w);
  }
  // count of pair p = (I, s): the next segment's start (or the list end)
  // minus its own; its bucket in the counting sort (a pair is its block's
  // last item when nothing of the list lies past its segment)
  auto pair = [&](int p, int& I, int& s, int& off, int& bucket) -> int {
    I = p / nsegs;
    s = p - I * nsegs;
    const size_t row = (size_t)bh * nqb + I;
    off = segoff[row * nsegs + s];
    const int total = min(max(kv_count[row], 0), kv_stride);
    const int end = s + 1 < nsegs ? segoff[row * nsegs + s + 1] : total;
    const int c = end - off;
    bucket = (end == total ? half : 0) + s * (sg + 1) + (sg - min(c, sg));
    return c;
  };
  for (int p = tid; p < npairs; p += 1024) {
    int I, s, off, b;
    const int c = pair(p, I, s, off, b);
    if (c > 0) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  // exclusive scan of the buckets
  const int per = (nbk + 1023) / 1024;
  const int b0 = tid * per, b1 = min(nbk, b0 + per);
  int loc = 0;
  for (int b = b0; b < b1; ++b) loc += hist[b];
  part[tid] = loc;
  __syncthreads();
  if (tid < 64) {                       // scan of the 1024 partial sums by one wave
    int v[16], run = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[j] = part[tid * 16 + j];
      run += v[j];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (tid >= o) incl += t;
    }
    int ex = incl - run;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      part[tid * 16 + j] = ex;
      ex += v[j];
    }
    if (tid == 63) part[1024] = incl;
  }
  __syncthreads();
  int run = part[tid];
  for (int b = b0; b < b1; ++b) {
    const int v = hist[b];
    hist[b] = run;
    run += v;
  }
  __syncthreads();
  if (tid == 0) {
    n_items[bh] = part[1024];
    n_first[bh] = hist[half];
    head_work[bh] = work;
  }
  __syncthreads();
  // scatter the items
  for (int p = tid; p < npairs; p += 1024) {
    int I, s, off, b;
    const int c = pair(p, I, s, off, b);
    if (c > 0) {
      const int k = atomicAdd(&hist[b], 1);
      int32_t* it = items + ((size_t)bh * max_items + k) * 4;
      it[0] = I;
      it[1] = off;
      it[2] = c;
      it[3] = s;
      slot_of[((size_t)bh * nqb + I) * nsegs + s] = k;
    }
  }
}

// Order of the heads in the item sequences, and their prefixes: a launch's
// sequence is dealt to the 8 XCDs as contiguous ranges of equal item counts,
// so each XCD runs about BH / 8 consecutive heads. Heads differ in kept tiles
// (up to 2.3x at the 720p layer), so the heads are first grouped by XCD
// greedily -- heaviest first, each to the least-loaded XCD that has fewer
// than ceil(BH / 8) -- and the groups laid out one after the other.
// head_order[p] = head at position p (identity for BH > kBalanceHeads);
// base_first[p] / base_last[p] = first / last items of the heads at
// positions before p; [BH] = totals.
constexpr int kBalanceHeads = 2048;
__global__ __launch_bounds__(256) void split_prefix_kernel(const int32_t* __restrict__ n_items,
                                                           const int32_t* __restrict__ n_first,
                                                           const int32_t* __restrict__ head_work, int BH,
                                                           int32_t* __restrict__ head_order,
                                                           int32_t* __restrict__ base_first,
                                                           int32_t* __restrict__ base_last) {
  __shared__ int part[257];
  __shared__ int sorted[kBalanceHeads];
  __shared__ int order[kBalanceHeads];
  const int tid = threadIdx.x;
  if (BH <= kBalanceHeads) {
    for (int h = tid; h < BH; h += 256) {            // rank by work, descending (ties: lower head)
      const int wh = head_work[h];
      int r = 0;
      for (int j = 0; j < BH; ++j) {
        const int wj = head_work[j];
        r += (wj > wh || (wj == wh && j < h)) ? 1 : 0;
      }
      sorted[r] = h;
    }
    __syncthreads();
    if (tid == 0) {
      const int cap = (BH + 7) / 8;
      long long load[8];
      int cnt[8];
      for (int x = 0; x < 8; ++x) { load[x] = 0; cnt[x] = 0; }
      for (int r = 0; r < BH; ++r) {                 // order[] doubles as the per-XCD slots
        const int h = sorted[r];
        int best = -1;
        for (int x = 0; x < 8; ++x)
          if (cnt[x] < cap && (best < 0 || load[x] < load[best])) best = x;
        order[best * cap + cnt[best]] = h;
        ++cnt[best];
        load[best] += head_work[h];
      }
      int p = 0;                                     // compact the groups in XCD order
      for (int x = 0; x < 8; ++x)
        for (int i = 0; i < cnt[x]; ++i) sorted[p++] = order[x * cap + i];
    }
    __syncthreads();
    for (int p = tid; p < BH; p += 256) head_order[p] = sorted[p];
  } else {
    for (int p = tid; p < BH; p += 256) head_order[p] = p;
  }
  __syncthreads();
  const int per = (BH + 255) / 256;
  const int b0 = tid * per, b1 = min(BH, b0 + per);
  auto head_at = [&](int p) { return BH <= kBalanceHeads ? sorted[p] : p; };
  auto prefix = [&](bool last, int32_t* base) {
    auto items_at = [&](int p) {
      const int h = head_at(p);
      return last ? n_items[h] - n_first[h] : n_first[h];
    };
    int loc = 0;
    for (int p = b0; p < b1; ++p) loc += items_at(p);
    part[tid] = loc;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int t = 0; t < 256; ++t) {
        const int v = part[t];
        part[t] = run;
        run += v;
      }
      part[256] = run;
    }
    __syncthreads();
    int run = part[tid];
    for (int p = b0; p < b1; ++p) {
      base[p] = run;
      run += items_at(p);
    }
    if (tid == 0) base[BH] = part[256];
    __syncthreads();
  };
  prefix(false, base_first);
  prefix(true, base_last);
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

// Key-block count from which uniform d = 128 attention runs one wave per tile
// (when the workspace is too small for the split path).
constexpr int kOneWaveKeyBlocks = 1024;

// Split over key segments: rows over at least kSplitMinKeyBlocks uniform key
// blocks at d = 128 are cut into S = ceil(nkb / kSplitSegBlocks) equal key
// segments (at the 720p layer 4 segments of 465 blocks, 14.5 MiB of K and V
// each: the tiles running together on an XCD read one segment, and ~2/3 of
// their requests hit its L2). Fewer, longer segments lose L2 hits; more,
// shorter ones add items and partial results.
constexpr int kSplitMinKeyBlocks = 1024;
constexpr int kSplitSegBlocks = 512;

namespace {
struct SplitLayout {
  int nsegs = 0, sg = 0, max_items = 0;
  size_t segoff = 0, slot_of = 0, nseg = 0, n_items = 0, n_first = 0, head_work = 0, head_order = 0,
         base_first = 0, base_last = 0, items = 0, part = 0, end = 0;
};
size_t r256(size_t b) { return (b + 255) & ~(size_t)255; }
// Workspace layout of the split path after the order table; nsegs = 0 when
// the path does not apply.
SplitLayout split_layout(int BH, int nqb, int nkb, int d) {
  SplitLayout L;
  L.end = r256(sizeof(int32_t) * (size_t)BH * (nqb + 1));
  if (d != 128 || nkb < kSplitMinKeyBlocks || nqb <= 0) return L;
  const int S = (nkb + kSplitSegBlocks - 1) / kSplitSegBlocks;
  const int sg = (nkb + S - 1) / S;
  if (S < 2 || S > 63 || 2 * sizeof(int) * (size_t)S * (sg + 1) > 64 * 1024) return L;
  const size_t pairs = (size_t)BH * nqb * S;
  if ((size_t)nqb * S > 0x7fffffff / 8) return L;
  L.nsegs = S;
  L.sg = sg;
  L.max_items = nqb * S;
  size_t o = L.end;
  L.segoff = o; o += r256(4 * pairs);
  L.slot_of = o; o += r256(4 * pairs);
  L.nseg = o; o += r256(4 * (size_t)BH * nqb);
  L.n_items = o; o += r256(4 * (size_t)BH);
  L.n_first = o; o += r256(4 * (size_t)BH);
  L.head_work = o; o += r256(4 * (size_t)BH);
  L.head_order = o; o += r256(4 * (size_t)BH);
  L.base_first = o; o += r256(4 * ((size_t)BH + 1));
  L.base_last = o; o += r256(4 * ((size_t)BH + 1));
  L.items = o; o += r256(16 * pairs);
  L.part = o; o += r256(sizeof(float) * (size_t)kSplitSlotFloats * pairs);
  L.end = o;
  return L;
}
}  // namespace

size_t attn_fwd_ws_bytes(int BH, int nqb, int nkb, int d) { return split_layout(BH, nqb, nkb, d).end; }

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int BH, int N, int d, int n_valid, const Blocks& qb, const Blocks& kb,
                           const int32_t* kv_count, const int32_t* kv_index, int kv_stride,
                           float scale, int32_t* tile_ws, size_t ws_bytes, float* lse, hipStream_t s) {
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
  a.items = nullptr; a.item_base = nullptr; a.item_first = nullptr; a.head_order = nullptr; a.nseg = nullptr;
  a.slot_of = nullptr;
  a.part = nullptr;
  a.max_items = 0; a.nsegs = 0;
  // Long uniform rows with a workspace of the full size: split over key
  // segments (plan, items, merge).
  if (!qvar && kmode == 0 && qb.start == nullptr && kb.start == nullptr && d == 128) {
    const SplitLayout L = split_layout(BH, qb.nblocks, kb.nblocks, d);
    if (L.nsegs >= 2 && ws_bytes >= L.end) {
      char* w = reinterpret_cast<char*>(tile_ws);
      int32_t* segoff = reinterpret_cast<int32_t*>(w + L.segoff);
      a.slot_of = reinterpret_cast<int32_t*>(w + L.slot_of);
      a.nseg = reinterpret_cast<int32_t*>(w + L.nseg);
      int32_t* n_items = reinterpret_cast<int32_t*>(w + L.n_items);
      int32_t* n_first = reinterpret_cast<int32_t*>(w + L.n_first);
      int32_t* head_work = reinterpret_cast<int32_t*>(w + L.head_work);
      int32_t* base_first = reinterpret_cast<int32_t*>(w + L.base_first);
      int32_t* base_last = reinterpret_cast<int32_t*>(w + L.base_last);
      a.head_order = reinterpret_cast<int32_t*>(w + L.head_order);
      a.items = reinterpret_cast<int32_t*>(w + L.items);
      a.part = reinterpret_cast<float*>(w + L.part);
      a.max_items = L.max_items;
      a.nsegs = L.nsegs;
      a.tiles = 0;
      a.bh = BH;
      if (!pad_done) zero_pad();
      const size_t lds = 2 * sizeof(int) * (size_t)L.nsegs * (L.sg + 1);
      split_rows_kernel<<<dim3((qb.nblocks + 15) / 16, BH), 1024, 0, s>>>(
          kv_count, kv_index, kv_stride, qb.nblocks, L.nsegs, L.sg, segoff, const_cast<int32_t*>(a.slot_of),
          const_cast<int32_t*>(a.nseg), reinterpret_cast<uint4*>(o), lse, N, n_valid);
      split_plan_kernel<<<BH, 1024, lds, s>>>(kv_count, kv_stride, qb.nblocks, L.nsegs, L.sg, L.max_items, segoff,
                                              const_cast<int32_t*>(a.items), const_cast<int32_t*>(a.slot_of),
                                              n_items, n_first, head_work);
      split_prefix_kernel<<<1, 256, 0, s>>>(n_items, n_first, head_work, BH, const_cast<int32_t*>(a.head_order),
                                            base_first, base_last);
      // every item but the last of its query block (at most all pairs but
      // one per block), then the last items (at most one per block)
      const long long grid1 = 8LL * (((long long)BH * (L.max_items - qb.nblocks) + 7) / 8);
      const long long grid2 = 8LL * (((long long)BH * qb.nblocks + 7) / 8);
      if (grid1 > 0x7fffffffLL || grid2 > 0x7fffffffLL) return hipErrorInvalidValue;
      a.item_base = base_first;
      a.item_first = nullptr;
      attn_fwd_kernel<128, false, 0, true><<<(int)grid1, 128, 0, s>>>(a);
      a.item_base = base_last;
      a.item_first = n_first;
      attn_fwd_kernel<128, false, 0, true><<<(int)grid2, 128, 0, s>>>(a);
      return hipGetLastError();
    }
  }
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
#define BSA_ATTN(DD, QV, KM) attn_fwd_kernel<DD, QV, KM, false><<<(int)grid, 128, 0, s>>>(a)
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

// Block-sparse attention backward: dQ, dK, dV of the forward in attn_fwd.hip
// over the same kept-block lists (NABLA summary, Contributi Chiave,
// "Accelerazione a Due Fasi", and Risultati Sperimentali 2: the sparse
// attention is used in pre-training and fine-tuning too, so its gradient runs
// over the same tiles). Uniform 64-token blocks, d in {64, 128}.
//
// Per query block I and kept key block J (S, P, dP, dS are 64 x 64 tiles):
//   S  = scale Q_I K_J^T,   P = exp(S - lse_I)     (lse from the forward)
//   dP = dO_I V_J^T,        dS = P * (dP - Dr_I)   (Dr_i = dO_i . O_i)
//   dQ_I += scale dS K_J,   dK_J += scale dS^T Q_I,   dV_J += P^T dO_I
// Every kernel is deterministic (no atomics on the gradients):
//   bwd_dot_kernel   Dr = rowsum(dO * O), fp32, stored beside lse * log2e;
//   csc_*_kernel     the lists transposed (key block -> query blocks that
//                    kept it): a bit matrix, then ascending lists;
//   bwd_grad_kernel  one launch with two roles, 4 waves per workgroup:
//                    key tiles (dK, dV) walk the query blocks that kept them,
//                    query tiles (dQ) walk their kept key blocks (the
//                    forward's lists). Each wave computes S and dP of a
//                    32 x 32 quarter of every 64 x 64 chunk. In a query tile
//                    the two key halves' partial dQ meet in LDS at the end;
//                    in a key tile the two waves of a key half trade P and dS
//                    through LDS every chunk, so one accumulates dV and the
//                    other dK over all 64 query rows.
// The MFMA layouts are those of the forward: a 32 x 32 accumulator whose
// lane holds one column (query, resp. key) and 16 rows; the second product of
// each pair takes its bf16 B operand straight from that accumulator, and the
// A operand through the LDS transpose read whose row order matches it.
#include "mfma_tile.h"

#include <math.h>

namespace bsa {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;           // [BH][N] natural-log row normaliser from the forward
  float* lsd;                 // [BH][N][2] (lse * log2e, rowsum(dO * O)), written by bwd_dot_kernel
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int N, n_valid, nqb, nkb;
  Blocks qb, kb;              // query / key blocks: uniform 64-token, or descriptors of at most 64 tokens
  const int32_t* kv_count;    // [BH][nqb] kept key blocks per query block
  const int32_t* kv_index;    // [BH][nqb][kv_stride]
  int kv_stride;
  int32_t* q_count;           // [BH][nkb] query blocks that kept each key block
  int32_t* q_index;           // [BH][nkb][nqb], ascending
  uint32_t* bits;             // [BH][nkb][W] bit matrix key block x query block
  int W;                      // 32-bit words per bit-matrix row
  const int32_t* order_q;     // null, or [BH][nqb] longest-first order of the query tiles
  const int32_t* order_k;     // null, or [BH][nkb] longest-first order of the key tiles
  float scale;
};

// Workgroup -> (head, tile): workgroups are dealt round-robin to the 8 XCDs,
// and XCD x takes a contiguous range of the flattened (head, position) order,
// so a head's operands stay in one XCD's L2; within a head, longest first.
__device__ __forceinline__ void tile_of(int L, int n, int BH, const int32_t* order, int& bh, int& t) {
  const int total = BH * n, per = total >> 3, rem = total & 7;
  const int x = L & 7, i = L >> 3;
  const int p = x * per + min(x, rem) + i;
  bh = p / n;
  const int pos = p - bh * n;
  t = order ? ((const __attribute__((address_space(4))) int32_t*)order)[(size_t)bh * n + pos] : pos;
}

// Block i of head bh: uniform 64-token blocks (geometry known at compile
// time) or a descriptor bounded to 64 tokens.
template <bool DESC>
__device__ __forceinline__ void block_at(const Blocks& b, int bh, int i, int n_valid, int& s, int& n) {
  if constexpr (DESC) {
    b.get(bh, i, s, n);
    n = min(max(n, 0), 64);
  } else {
    s = 64 * i;
    n = min(64, n_valid - s);
  }
}

// Per row: (lse * log2e, Dr = sum_c dO[row, c] O[row, c]) in fp32, one
// 8-byte pair, so that a chunk's pairs are one contiguous run; (+inf, 0) on
// pad rows.
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdArgs a, size_t rows) {
  constexpr int LPR = D / 8;                       // lanes per row, 8 channels each
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows && (int)(row % a.N) < a.n_valid) {
    const uint4 x = *reinterpret_cast<const uint4*>(a.o + row * D + part * 8);
    const uint4 y = *reinterpret_cast<const uint4*>(a.dout + row * D + part * 8);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(xs[i]) * bf16_lo(ys[i]) + bf16_hi(xs[i]) * bf16_hi(ys[i]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    const bool valid = (int)(row % a.N) < a.n_valid;
    *reinterpret_cast<f32x2*>(a.lsd + 2 * row) = (f32x2){valid ? a.lse[row] * kLog2e : INFINITY, acc};
  }
}

// Transposed lists, step 1: clear the bit matrix.
__global__ __launch_bounds__(256) void csc_clear_kernel(uint32_t* bits, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) bits[i] = 0u;
}
// Step 2: bit I of row (bh, J) for every kept pair (I, J); one wave per query
// block row. Invalid key ids are skipped.
__global__ __launch_bounds__(256) void csc_set_kernel(BwdArgs a, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const size_t bh = row / a.nqb;
  const int I = (int)(row % a.nqb);
  const int c = min(max(a.kv_count[row], 0), a.kv_stride);
  for (int e = lane; e < c; e += 64) {
    const int J = a.kv_index[row * a.kv_stride + e];
    if ((unsigned)J < (unsigned)a.nkb) atomicOr(&a.bits[(bh * a.nkb + J) * a.W + (I >> 5)], 1u << (I & 31));
  }
}
// Step 3: one wave per key-block row turns its bits into an ascending list.
__global__ __launch_bounds__(256) void csc_list_kernel(BwdArgs a, size_t cols) {
  const size_t col = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (col >= cols) return;
  const uint32_t* b = a.bits + col * a.W;
  int32_t* out = a.q_index + col * a.nqb;
  int base = 0;
  for (int w0 = 0; w0 < a.W; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = w < a.W ? b[w] : 0u;
    const int n = __popc(word);
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int pos = base + incl - n;
    while (word) {
      out[pos++] = 32 * w + (__ffs(word) - 1);
      word &= word - 1u;
    }
    base += __shfl(incl, 63);
  }
  if (lane == 0) a.q_count[col] = base;
}

// dQ of one 64-row query tile. Four waves: wave w owns query rows
// 32 (w & 1) .. +31 and key rows 32 (w >> 1) .. +31 of every chunk, so each
// wave holds half the per-chunk state and two waves share a SIMD.
// Per kept key block, on double-buffered K / V tiles:
//   S^T = K Q^T, dP^T = V dO^T      (32 keys x 32 queries; Q^T, dO^T in registers)
//   P = exp2(S * scale * log2e - lse * log2e), dS = P (dP - Dr)   (lane-local)
//   dQ^T += K^T dS^T                (K^T through the transpose read)
// The two key halves' partial dQ^T meet in LDS at the end (fixed order).
template <int D, bool DESC>
__device__ __forceinline__ void bwd_dq_tile(const BwdArgs& a, int L, int BH, unsigned char* K0, unsigned char* V0,
                                            unsigned char* K1, unsigned char* V1) {
  using T = Tile<D, 4>;
  constexpr int NC = D / 16;                       // MFMA k-steps over the channels

  int bh, I;
  tile_of(L, a.nqb, BH, a.order_q, bh, I);
  int qs, ql;
  block_at<DESC>(a.qb, bh, I, a.n_valid, qs, ql);
  if (ql <= 0) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wave & 1, kw = wave >> 1;
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * a.N;
  const uint16_t* kh = a.k + head * D;
  const uint16_t* vh = a.v + head * D;
  const float sl2 = a.scale * kLog2e;

  // Q^T and dO^T as MFMA B operands: lane supplies row 32qw + l32,
  // channels 16 c + 8 half .. +7
  const int qr = 32 * qw + l32;
  const bool qok = qr < ql;
  bf16x8 qf[NC], gf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const size_t off = (head + qs + (qok ? qr : 0)) * D + 16 * c + 8 * half;
    qf[c] = qok ? *reinterpret_cast<const bf16x8*>(a.q + off) : bf16x8{};
    gf[c] = qok ? *reinterpret_cast<const bf16x8*>(a.dout + off) : bf16x8{};
  }
  const float lse2 = qok ? a.lsd[2 * (head + qs + qr)] : INFINITY;   // pad rows: P = 0
  const float drow = qok ? a.lsd[2 * (head + qs + qr) + 1] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dg][r] = 0.f;

  const size_t lrow = (size_t)bh * a.nqb + I;
  const int cnt = min(max(((const cint*)a.kv_count)[lrow], 0), a.kv_stride);
  const cint* list = (const cint*)(a.kv_index + lrow * a.kv_stride);
  uint32_t off[T::NI];
  tile_offsets<D, 4>(wave, lane, off);
  const TrOffsets<D> tro(lane);
  auto block_of = [&](int c, int& ks, int& kl) {   // chunk c of the list (clamped into range)
    int J = list[c < cnt ? c : cnt - 1];
    J = (unsigned)J < (unsigned)a.nkb ? J : a.nkb - 1;
    block_at<DESC>(a.kb, bh, J, a.n_valid, ks, kl);
  };

  // one chunk: loads of chunk c+1 (or a reload of c) into (Kn, Vn) go out
  // first; chunk c must have landed in (Kc, Vc)
  auto step = [&](int c, const lds_u8* Kc, const lds_u8* Vc, lds_u8* Kn, lds_u8* Vn) {
    int ks, kl, ks1, kl1;
    block_of(c, ks, kl);
    block_of(c + 1, ks1, kl1);
    tile_load<D, 4>(kh, ks1, kl1, Kn, wave, off);
    tile_load<D, 4>(vh, ks1, kl1, Vn, wave, off);
    wait_vm<2 * T::NI>();                          // this wave's share of chunk c landed
    wg_barrier();                                  // and the other waves'
    // the score products and the exp/pack that follow go first among the
    // waves sharing this SIMD; the other workgroup's loads fill the gaps
    __builtin_amdgcn_s_setprio(1);
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(Kc, kw, cc, l32, half), qf[cc], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(Vc, kw, cc, l32, half), gf[cc], dp, 0, 0, 0);
    }
    uint32_t pw[2][4];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float d2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = 32 * kw + acc_row(r + u, half);
        const float p = key < kl ? __builtin_amdgcn_exp2f(fmaf(s[r + u], sl2, -lse2)) : 0.f;
        d2[u] = p * (dp[r + u] - drow);
      }
      pw[r >> 3][(r & 7) >> 1] = pack2(d2[0], d2[1]);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 ds = __builtin_bit_cast(bf16x8, (u32x4){pw[hh][0], pw[hh][1], pw[hh][2], pw[hh][3]});
#pragma unroll
      for (int dg = 0; dg < D / 32; ++dg)
        dq[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(Kc, tro, kw, hh, dg), ds, dq[dg], 0, 0, 0);
    }
    wg_barrier();                                  // (Kc, Vc) free for chunk c+2
  };

  if (cnt > 0) {
    int ks0, kl0;
    block_of(0, ks0, kl0);
    tile_load<D, 4>(kh, ks0, kl0, (lds_u8*)K0, wave, off);
    tile_load<D, 4>(vh, ks0, kl0, (lds_u8*)V0, wave, off);
    for (int c = 0;;) {
      step(c, (const lds_u8*)K0, (const lds_u8*)V0, (lds_u8*)K1, (lds_u8*)V1);
      if (++c >= cnt) break;
      step(c, (const lds_u8*)K1, (const lds_u8*)V1, (lds_u8*)K0, (lds_u8*)V0);
      if (++c >= cnt) break;
    }
  }
  wait_vm<0>();                                    // no load of this wave targets LDS
  wg_barrier();                                    // nor one of the other waves
  // the second key half's partial dQ^T joins the first's: 16 KiB per wave
  lds_f32* park = (lds_f32*)(qw ? V0 : K0);
  if (kw == 1) {
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int r = 0; r < 16; ++r) park[(dg * 16 + r) * 64 + lane] = dq[dg][r];
  }
  wg_barrier();
  if (kw == 0) {
#pragma unroll
    for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[dg][r] += park[(dg * 16 + r) * 64 + lane];
  }
  store_rows<D, 256>(dq, a.scale, (lds_u8*)K1, a.dq + head * D, qs, ql, qw, lane, kw == 0);
}

// dK, dV of one 64-key tile. Four waves: wave w takes keys 32 (w & 1) .. +31
// and query rows 32 (w >> 1) .. +31 of every chunk. Per query block that kept
// the tile, on double-buffered Q / dO tiles:
//   S = Q K^T, dP = dO V^T          (32 queries x 32 keys; K^T, V^T in registers)
//   P = exp2(S * scale * log2e - lse * log2e), dS = P (dP - Dr)
// The two waves of a key half then trade their quarter of P or dS through
// LDS (2 KiB each, lane-aligned: lane = key), and over the chunk's 64 query
// rows the first accumulates dV^T += dO^T P, the second dK^T += Q^T dS (dO^T,
// Q^T through the transpose read). One 32-key x D accumulator per wave, in
// place of a partial dK^T and dV^T each, keeps a wave within the 256
// registers of two waves per SIMD.
template <int D, bool DESC>
__device__ __forceinline__ void bwd_dkdv_tile(const BwdArgs& a, int L, int BH, unsigned char* Q0, unsigned char* G0,
                                              unsigned char* Q1, unsigned char* G1, unsigned char* X) {
  using T = Tile<D, 4>;
  constexpr int NC = D / 16;                       // MFMA k-steps over the channels

  int bh, J;
  tile_of(L, a.nkb, BH, a.order_k, bh, J);
  int ks, kl;
  block_at<DESC>(a.kb, bh, J, a.n_valid, ks, kl);
  if (kl <= 0) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 1, g = wave >> 1;          // g = 0: dV, g = 1: dK
  const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t head = (size_t)bh * a.N;
  const uint16_t* qh = a.q + head * D;
  const uint16_t* gh = a.dout + head * D;
  const float sl2 = a.scale * kLog2e;

  // K^T and V^T as MFMA B operands: lane supplies key 32kw + l32, channels
  // 16 c + 8 half .. +7
  const int kr = 32 * kw + l32;
  const bool kok = kr < kl;
  bf16x8 kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const size_t o = (head + ks + (kok ? kr : 0)) * D + 16 * c + 8 * half;
    kf[c] = kok ? *reinterpret_cast<const bf16x8*>(a.k + o) : bf16x8{};
    vf[c] = kok ? *reinterpret_cast<const bf16x8*>(a.v + o) : bf16x8{};
  }
  f32x16 acc[D / 32];                              // dV^T (g = 0) or dK^T (g = 1) of keys 32kw ..
#pragma unroll
  for (int dg = 0; dg < D / 32; ++dg)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dg][r] = 0.f;

  const size_t lcol = (size_t)bh * a.nkb + J;
  const int cnt = ((const cint*)a.q_count)[lcol];
  const cint* list = (const cint*)(a.q_index + lcol * a.nqb);
  uint32_t off[T::NI];
  tile_offsets<D, 4>(wave, lane, off);
  const TrOffsets<D> tro(lane);
  // hand-over slots, [key half][writer's g][hh][lane][4 words]: this wave
  // writes its own, reads the other wave's of its key half
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u32x4* mine = (lds_u32x4*)((lds_u8*)X + (2 * kw + g) * 2048);
  const lds_u32x4* theirs = (const lds_u32x4*)((lds_u8*)X + (2 * kw + (g ^ 1)) * 2048);

  // chunk c (clamped into range): its Q and dO rows, and its rows'
  // (lse log2e, Dr) pairs straight into LDS after the Q tile (Qn + BYTES).
  // Every wave loads all 64 pairs (lanes 0..31, 16 bytes each; lanes 32..63
  // read past the descriptor and write zeros to the next 512 bytes): the
  // waves write the same bytes, every wave issues the same loads, and no
  // load sits under a branch (the compiler would then wait for it before
  // any LDS read). Rows past the block read as zeros: their Q and dO rows
  // are zero too, so they add nothing to dK or dV.
  auto issue = [&](int c, lds_u8* Qn, lds_u8* Gn) {
    const int I = list[c < cnt ? c : cnt - 1];
    int qs, ql;
    block_at<DESC>(a.qb, bh, I, a.n_valid, qs, ql);
    const int q0 = __builtin_amdgcn_readfirstlane(qs), n0 = __builtin_amdgcn_readfirstlane(max(ql, 0));
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lsd + 2 * (head + q0), (uint32_t)n0 * 8);
    dma16(rl, Qn + T::BYTES, lane < 32 ? 16 * lane : 0xFFFFFFF0u);
    tile_load<D, 4>(qh, qs, ql, Qn, wave, off);
    tile_load<D, 4>(gh, qs, ql, Gn, wave, off);
  };
  // one chunk: chunk c+1 (or a reload of c) goes out first; chunk c must
  // have landed in (Qc, Gc)
  auto step = [&](int c, const lds_u8* Qc, const lds_u8* Gc, lds_u8* Qn, lds_u8* Gn) {
    const lds_u8* LRc = Qc + T::BYTES;
    issue(c + 1, Qn, Gn);
    wait_vm<2 * T::NI + 1>();                      // this wave's share of chunk c landed
    wg_barrier();                                  // and the other waves'
    __builtin_amdgcn_s_setprio(1);                 // as in the query-tile step
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(Qc, g, cc, l32, half), kf[cc], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read<D>(Gc, g, cc, l32, half), vf[cc], dp, 0, 0, 0);
    }
    uint32_t pp[2][4], pd[2][4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      // rows 32g + 8 r4 + 4 half + 0..3 of the chunk
      const int row0 = 32 * g + 8 * r4 + 4 * half;
      typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;
      const f32x4 a01 = *reinterpret_cast<lds_f32x4*>(LRc + 8 * row0);        // rows row0, row0 + 1
      const f32x4 a23 = *reinterpret_cast<lds_f32x4*>(LRc + 8 * row0 + 16);   // rows row0 + 2, row0 + 3
      const f32x4 l4 = {a01[0], a01[2], a23[0], a23[2]};
      const f32x4 d4 = {a01[1], a01[3], a23[1], a23[3]};
      float p[4], d[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * r4 + u;
        p[u] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -l4[u]));
        d[u] = p[u] * (dp[r] - d4[u]);
      }
      pp[r4 >> 1][2 * (r4 & 1) + 0] = pack2(p[0], p[1]);
      pp[r4 >> 1][2 * (r4 & 1) + 1] = pack2(p[2], p[3]);
      pd[r4 >> 1][2 * (r4 & 1) + 0] = pack2(d[0], d[1]);
      pd[r4 >> 1][2 * (r4 & 1) + 1] = pack2(d[2], d[3]);
    }
    __builtin_amdgcn_s_setprio(0);
    // the dV wave keeps its P and hands over its dS, the dK wave the reverse
    u32x4 own[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const u32x4 P4 = {pp[hh][0], pp[hh][1], pp[hh][2], pp[hh][3]};
      const u32x4 D4 = {pd[hh][0], pd[hh][1], pd[hh][2], pd[hh][3]};
      own[hh] = g ? D4 : P4;
      mine[hh * 64 + lane] = g ? P4 : D4;
    }
    wg_barrier();
    // over the chunk's 64 query rows (half gq, 16-row group hh):
    //   g = 0: dV^T += dO^T P,  g = 1: dK^T += Q^T dS
    // (a branch per role rather than a selected pointer: the compiler then
    // knows which tile each LDS read touches and does not wait for the loads
    // in flight into the other buffers)
    auto accumulate = [&](const lds_u8* src) {
#pragma unroll
      for (int gq = 0; gq < 2; ++gq)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, gq == g ? own[hh] : theirs[hh * 64 + lane]);
#pragma unroll
          for (int dg = 0; dg < D / 32; ++dg)
            acc[dg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(src, tro, gq, hh, dg), b, acc[dg], 0, 0, 0);
        }
    };
    if (g)
      accumulate(Qc);
    else
      accumulate(Gc);
    wg_barrier();                                  // chunk c's buffers and the slots free again
  };

  if (cnt > 0) {
    issue(0, (lds_u8*)Q0, (lds_u8*)G0);
    for (int c = 0;;) {
      step(c, (const lds_u8*)Q0, (const lds_u8*)G0, (lds_u8*)Q1, (lds_u8*)G1);
      if (++c >= cnt) break;
      step(c, (const lds_u8*)Q1, (const lds_u8*)G1, (lds_u8*)Q0, (lds_u8*)G0);
      if (++c >= cnt) break;
    }
  }
  wait_vm<0>();
  wg_barrier();
  store_rows<D, 256>(acc, a.scale, (lds_u8*)Q0, a.dk + head * D, ks, kl, kw, lane, g == 1);
  wg_barrier();
  store_rows<D, 256>(acc, 1.f, (lds_u8*)G0, a.dv + head * D, ks, kl, kw, lane, g == 0);
}

// One launch for both gradients: workgroups [0, nkv) take key tiles (dK, dV;
// the longer work, dispatched first), the rest query tiles (dQ), which fill
// in as the key tiles drain. nkv is the key-tile count rounded up to a
// multiple of 8, so each part keeps its own per-XCD ranges; the LDS buffers
// are shared by the two roles.
template <int D, bool DESC>
__global__ __launch_bounds__(256, 2) void bwd_grad_kernel(BwdArgs a, int BH, int nkv) {
  // B0 and B2 hold a key tile's Q tiles, each followed by the chunk rows'
  // (lse log2e, Dr) pairs (512 bytes, then the 512 zero bytes of the load's
  // upper lanes)
  __shared__ __align__(16) unsigned char B0[Tile<D>::BYTES + 1024];
  __shared__ __align__(16) unsigned char B1[Tile<D>::BYTES];
  __shared__ __align__(16) unsigned char B2[Tile<D>::BYTES + 1024];
  __shared__ __align__(16) unsigned char B3[Tile<D>::BYTES];
  __shared__ __align__(16) unsigned char X[8192];  // P / dS hand-over of the key tiles
  const int G = blockIdx.x;
  if (G < nkv) {
    if (G >= BH * a.nkb) return;                  // padding of the key-tile range
    bwd_dkdv_tile<D, DESC>(a, G, BH, B0, B1, B2, B3, X);
  } else {
    bwd_dq_tile<D, DESC>(a, G - nkv, BH, B0, B1, B2, B3);
  }
}

// Pad rows n_valid .. N-1 of dq, dk, dv are zero.
__global__ __launch_bounds__(256) void bwd_zero_pad_kernel(uint4* dq, uint4* dk, uint4* dv, int N, int n_valid,
                                                           int cpr, size_t total) {
  const size_t per_head = (size_t)(N - n_valid) * cpr;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (size_t)gridDim.x * 256) {
    const size_t bh = u / per_head, rem = u % per_head;
    const size_t i = (bh * N + n_valid) * cpr + rem;
    dq[i] = dk[i] = dv[i] = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const uint16_t* dout, const float* lse, int BH, int N, int d, int n_valid,
                           const Blocks& qb, const Blocks& kb, const int32_t* kv_count, const int32_t* kv_index,
                           int kv_stride, float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws,
                           hipStream_t s) {
  if (BH == 0) return hipSuccess;
  const int nqb = qb.nblocks, nkb = kb.nblocks;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.N = N; a.n_valid = n_valid; a.nqb = nqb; a.nkb = nkb;
  a.qb = qb; a.kb = kb;
  a.kv_count = kv_count; a.kv_index = kv_index; a.kv_stride = kv_stride;
  a.W = (nqb + 31) / 32;
  a.scale = scale;
  // workspace: (lse log2e, Dr) [BH][N][2] fp32 | q_count [BH][nkb] | q_index [BH][nkb][nqb] | bits [BH][nkb][W]
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += (bytes + 255) & ~(size_t)255;
    return r;
  };
  a.lsd = reinterpret_cast<float*>(take(2 * sizeof(float) * (size_t)BH * N));
  a.q_count = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * nkb));
  a.q_index = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * nkb * nqb));
  a.bits = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)BH * nkb * a.W));
  int32_t* oq = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * nqb));
  int32_t* ok = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)BH * nkb));

  if (n_valid < N) {
    const int cpr = d / 8;
    const size_t total = (size_t)BH * (N - n_valid) * cpr;
    const size_t want = (total + 255) / 256;
    bwd_zero_pad_kernel<<<(int)(want < 4096 ? want : 4096), 256, 0, s>>>(
        reinterpret_cast<uint4*>(dq), reinterpret_cast<uint4*>(dk), reinterpret_cast<uint4*>(dv), N, n_valid, cpr,
        total);
  }
  if (nqb == 0 || nkb == 0) return hipGetLastError();
  const size_t rows = (size_t)BH * N;
  const size_t lanes = rows * (d / 8);
  if (d == 128)
    bwd_dot_kernel<128><<<(int)((lanes + 255) / 256), 256, 0, s>>>(a, rows);
  else
    bwd_dot_kernel<64><<<(int)((lanes + 255) / 256), 256, 0, s>>>(a, rows);
  const size_t nbits = (size_t)BH * nkb * a.W;
  csc_clear_kernel<<<(int)((nbits + 255) / 256 < 4096 ? (nbits + 255) / 256 : 4096), 256, 0, s>>>(a.bits, nbits);
  const size_t qrows = (size_t)BH * nqb, kcols = (size_t)BH * nkb;
  csc_set_kernel<<<(int)((qrows + 3) / 4), 256, 0, s>>>(a, qrows);
  csc_list_kernel<<<(int)((kcols + 3) / 4), 256, 0, s>>>(a, kcols);
  a.order_q = launch_qorder(kv_count, BH, nqb, nkb, oq, s) ? oq : nullptr;
  a.order_k = launch_qorder(a.q_count, BH, nkb, nqb, ok, s) ? ok : nullptr;
  const int nkv = ((int)kcols + 7) & ~7;
  const int grid = nkv + (int)qrows;
  const bool desc = qb.start != nullptr || kb.start != nullptr;
  if (d == 128) {
    if (desc) bwd_grad_kernel<128, true><<<grid, 256, 0, s>>>(a, BH, nkv);
    else bwd_grad_kernel<128, false><<<grid, 256, 0, s>>>(a, BH, nkv);
  } else {
    if (desc) bwd_grad_kernel<64, true><<<grid, 256, 0, s>>>(a, BH, nkv);
    else bwd_grad_kernel<64, false><<<grid, 256, 0, s>>>(a, BH, nkv);
  }
  return hipGetLastError();
}

size_t attn_bwd_workspace(int BH, int N, int nqb, int nkb) {
  auto r = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t W = ((size_t)nqb + 31) / 32;
  return r(2 * sizeof(float) * (size_t)BH * N) + r(sizeof(int32_t) * (size_t)BH * nkb) +
         r(sizeof(int32_t) * (size_t)BH * nkb * nqb) + r(sizeof(uint32_t) * (size_t)BH * nkb * W) +
         r(sizeof(int32_t) * (size_t)BH * nqb) + r(sizeof(int32_t) * (size_t)BH * nkb);
}

}  // namespace bsa

// C ABI of libbsa: argument validation, workspace carving and kernel launch
// (declarations and the contract of every entry point are in include/bsa.h).
#include <algorithm>
#include <mutex>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "lds_tile.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Validates a descriptor and converts it for the kernels.
int make_blocks(const bsa_blocks* in, int block, int n_valid, const char* what, bsa::Blocks& out) {
  out.block = block;
  out.n_valid = n_valid;
  if (in == nullptr) {
    if (block != 64) return fail(BSA_EUNSUPPORTED, "%s: uniform blocks must have 64 tokens (got %d)", what, block);
    out.start = nullptr;
    out.len = nullptr;
    out.nblocks = (n_valid + block - 1) / block;
    out.per_head = 0;
    out.max_len = 0;
    return BSA_OK;
  }
  if (in->nblocks < 0) return fail(BSA_EINVAL, "%s: nblocks < 0", what);
  if (in->nblocks > 0 && (in->start == nullptr || in->len == nullptr))
    return fail(BSA_EINVAL, "%s: null start/len array", what);
  out.start = in->start;
  out.len = in->len;
  out.nblocks = in->nblocks;
  out.per_head = in->per_head ? 1 : 0;
  out.max_len = in->max_len >= 1 && in->max_len <= 64 ? in->max_len : 0;
  // A non-null descriptor with no blocks is valid (nothing to do).
  if (out.start == nullptr) {
    // keep the device view distinguishable from uniform blocks
    static const int32_t dummy = 0;
    out.start = &dummy;
    out.len = &dummy;
  }
  return BSA_OK;
}

int check_shape(int B, int H, int N, int d, int n_valid) {
  if (B <= 0 || H <= 0 || N <= 0) return fail(BSA_EINVAL, "B, H and N must be positive (B=%d H=%d N=%d)", B, H, N);
  if ((long long)B * H > 65535) return fail(BSA_EUNSUPPORTED, "B*H must be <= 65535");
  if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
  if (n_valid <= 0 || n_valid > N) return fail(BSA_EINVAL, "n_valid must be in [1, N] (got %d, N=%d)", n_valid, N);
  return BSA_OK;
}

int make_window(const bsa_window* w, int nqb, int nkb, bsa::Window& out) {
  memset(&out, 0, sizeof out);
  if (w == nullptr) return BSA_OK;
  if (w->nt <= 0 || w->ny <= 0 || w->nx <= 0) return fail(BSA_EINVAL, "window grid must be positive");
  if (w->rt < 0 || w->ry < 0 || w->rx < 0) return fail(BSA_EINVAL, "window radii must be >= 0");
  const long long cells = (long long)w->nt * w->ny * w->nx;
  if (cells != nqb || cells != nkb)
    return fail(BSA_EINVAL, "window grid %dx%dx%d does not match %d query / %d key blocks", w->nt, w->ny, w->nx, nqb, nkb);
  out.nt = w->nt; out.ny = w->ny; out.nx = w->nx;
  out.rt = w->rt; out.ry = w->ry; out.rx = w->rx;
  out.enabled = 1;
  return BSA_OK;
}

}  // namespace

extern "C" {

int bsa_abi_version(void) { return BSA_ABI_VERSION; }

int bsa_lds_swizzle(int d, int row) {
  if (d != 64 && d != 128) return -1;
  return d == 128 ? bsa::swz<128>(row & 15) : bsa::swz<64>(row & 15);
}

const char* bsa_strerror(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_EINVAL: return "invalid argument";
    case BSA_EUNSUPPORTED: return "unsupported argument";
    case BSA_ENOSPC: return "workspace or capacity too small";
    case BSA_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bsa_last_error_message(void) { return g_msg; }

int bsa_pool_blocks(const void* x, int B, int H, int N, int d, int n_valid, int block,
                    const bsa_blocks* blocks, float* out, hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (!x || !out) return fail(BSA_EINVAL, "pool: null pointer");
  if (!aligned16(x)) return fail(BSA_EINVAL, "pool: x must be 16-byte aligned");
  bsa::Blocks b;
  if (int e = make_blocks(blocks, block, n_valid, "pool", b)) return e;
  return hip_status(bsa::launch_pool(static_cast<const uint16_t*>(x), B * H, N, d, b, out, stream), "pool");
}

int bsa_select_blocks(const float* qbar, const float* kbar, int B, int H, int nqb, int nkb, int d,
                      const int32_t* q_sizes, const int32_t* k_sizes, float thr, float scale,
                      const bsa_window* win, int32_t* kv_count, int32_t* kv_index, int kv_stride,
                      hipStream_t stream) {
  g_msg[0] = 0;
  if (B <= 0 || H <= 0) return fail(BSA_EINVAL, "select: B and H must be positive");
  if ((long long)B * H > 65535) return fail(BSA_EUNSUPPORTED, "B*H must be <= 65535");
  if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "select: d must be 64 or 128");
  if (nqb < 0 || nkb <= 0) return fail(BSA_EINVAL, "select: need nqb >= 0 and nkb >= 1");
  if (nkb > 8192) return fail(BSA_EUNSUPPORTED, "select: at most 8192 key blocks (got %d)", nkb);
  if (!qbar || !kbar || !kv_count || !kv_index) return fail(BSA_EINVAL, "select: null pointer");
  if (!aligned16(qbar) || !aligned16(kbar)) return fail(BSA_EINVAL, "select: pooled inputs must be 16-byte aligned");
  if (!(thr >= 0.f && thr <= 1.f)) return fail(BSA_EINVAL, "select: thr must be in [0, 1]");
  if (kv_stride < nkb) return fail(BSA_ENOSPC, "select: kv_stride %d < nkb %d", kv_stride, nkb);
  bsa::Window w;
  if (int e = make_window(win, nqb, nkb, w)) return e;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  const bsa::Sizes sz{q_sizes, k_sizes, 1, 1, 1};
  return hip_status(bsa::launch_select(qbar, kbar, B * H, nqb, nkb, d, sz, thr, sc, w,
                                       kv_count, kv_index, kv_stride, stream),
                    "select");
}

size_t bsa_build_block_mask_workspace(int B, int H, int nqb, int nkb, int d) {
  if (B <= 0 || H <= 0 || nqb < 0 || nkb < 0 || d <= 0) return 0;
  return round256(sizeof(float) * (size_t)B * H * nqb * d) + round256(sizeof(float) * (size_t)B * H * nkb * d);
}

int bsa_build_block_mask(const void* q, const void* k, int B, int H, int N, int d, int n_valid, int block,
                         const bsa_blocks* qb, const bsa_blocks* kb, float thr, const bsa_window* win,
                         int32_t* kv_count, int32_t* kv_index, int kv_stride, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (!q || !k || !kv_count || !kv_index) return fail(BSA_EINVAL, "build_block_mask: null pointer");
  if (!aligned16(q) || !aligned16(k)) return fail(BSA_EINVAL, "build_block_mask: q, k must be 16-byte aligned");
  bsa::Blocks bq, bk;
  if (int e = make_blocks(qb, block, n_valid, "query blocks", bq)) return e;
  if (int e = make_blocks(kb, block, n_valid, "key blocks", bk)) return e;
  if (bk.nblocks <= 0) return fail(BSA_EINVAL, "build_block_mask: no key blocks");
  if (bk.nblocks > 8192) return fail(BSA_EUNSUPPORTED, "build_block_mask: at most 8192 key blocks");
  if (!(thr >= 0.f && thr <= 1.f)) return fail(BSA_EINVAL, "build_block_mask: thr must be in [0, 1]");
  if (kv_stride < bk.nblocks) return fail(BSA_ENOSPC, "build_block_mask: kv_stride %d < nkb %d", kv_stride, bk.nblocks);
  bsa::Window w;
  if (int e = make_window(win, bq.nblocks, bk.nblocks, w)) return e;
  const size_t need = bsa_build_block_mask_workspace(B, H, bq.nblocks, bk.nblocks, d);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(BSA_ENOSPC, "build_block_mask: workspace %zu bytes < %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(BSA_EINVAL, "build_block_mask: workspace must be 16-byte aligned");
  float* qbar = static_cast<float*>(ws);
  float* kbar = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         round256(sizeof(float) * (size_t)B * H * bq.nblocks * d));
  const int BH = B * H;
  if (int e = hip_status(bsa::launch_pool2(static_cast<const uint16_t*>(q), bq, qbar, static_cast<const uint16_t*>(k),
                                           bk, kbar, BH, N, d, stream),
                         "pool q, k"))
    return e;
  const float sc = 1.f / sqrtf((float)d);
  // descriptor blocks: a block with no tokens takes no part (lengths, no bias)
  const bsa::Sizes sz{bq.start ? bq.len : nullptr, bk.start ? bk.len : nullptr, bq.per_head, bk.per_head, 0};
  return hip_status(bsa::launch_select(qbar, kbar, BH, bq.nblocks, bk.nblocks, d, sz, thr, sc, w,
                                       kv_count, kv_index, kv_stride, stream),
                    "select");
}

int bsa_build_centroid_mask(const float* cq, const int32_t* q_sizes, const float* ck, const int32_t* k_sizes,
                            int B, int H, int Cq, int Ck, int d, float top_p, float scale, int32_t* kv_count,
                            int32_t* kv_index, int kv_stride, hipStream_t stream) {
  g_msg[0] = 0;
  if (!q_sizes || !k_sizes) return fail(BSA_EINVAL, "centroid mask: cluster sizes are required");
  if (!(top_p >= 0.f && top_p <= 1.f)) return fail(BSA_EINVAL, "centroid mask: top_p must be in [0, 1]");
  return bsa_select_blocks(cq, ck, B, H, Cq, Ck, d, q_sizes, k_sizes, 1.f - top_p, scale, nullptr, kv_count,
                           kv_index, kv_stride, stream);
}

// The order table alone (B*H*(nqb+1) int32): the least workspace the forward runs with.
static size_t attn_fwd_min_ws(int B, int H, int nqb) { return round256(sizeof(int32_t) * (size_t)B * H * (nqb + 1)); }

size_t bsa_block_sparse_attn_fwd_workspace(int B, int H, int nqb, const bsa_blocks* qb) {
  if (B <= 0 || H <= 0 || nqb < 0) return 0;
  // uniform blocks (self-attention: as many key as query blocks) over long
  // rows also get room for the split over key segments (sized for d = 128)
  if (qb == nullptr) return bsa::attn_fwd_ws_bytes(B * H, nqb, nqb, 128);
  return attn_fwd_min_ws(B, H, nqb);
}

static int attn_fwd_impl(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                         int n_valid, int block, const bsa_blocks* qb, const bsa_blocks* kb,
                         const int32_t* kv_count, const int32_t* kv_index, int kv_stride, float scale,
                         float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (!q || !k || !v || !o || !kv_count || !kv_index) return fail(BSA_EINVAL, "attn_fwd: null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_EINVAL, "attn_fwd: q, k, v, o must be 16-byte aligned");
  if ((long long)N * d * 2 > 0xFFFFFFFFLL)
    return fail(BSA_EUNSUPPORTED, "attn_fwd: one head (N*d*2 bytes) must be below 4 GiB");
  bsa::Blocks bq, bk;
  if (int e = make_blocks(qb, block, n_valid, "query blocks", bq)) return e;
  if (int e = make_blocks(kb, block, n_valid, "key blocks", bk)) return e;
  if (kv_stride < 0 || (bk.nblocks > 0 && kv_stride < 1)) return fail(BSA_EINVAL, "attn_fwd: bad kv_stride");
  const size_t need = attn_fwd_min_ws(B, H, bq.nblocks);
  if (ws == nullptr || ws_bytes < need)
    return fail(BSA_ENOSPC, "attn_fwd: workspace %zu bytes < %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(BSA_EINVAL, "attn_fwd: workspace must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return hip_status(bsa::launch_attn_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), B * H, N, d,
                                         n_valid, bq, bk, kv_count, kv_index, kv_stride, sc,
                                         static_cast<int32_t*>(ws), ws_bytes, lse, stream),
                    "attn_fwd");
}

int bsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                              int n_valid, int block, const bsa_blocks* qb, const bsa_blocks* kb,
                              const int32_t* kv_count, const int32_t* kv_index, int kv_stride, float scale,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  return attn_fwd_impl(q, k, v, o, B, H, N, d, n_valid, block, qb, kb, kv_count, kv_index, kv_stride, scale,
                       nullptr, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- allocation-free forward
// The int32 table the forward needs (processing order of the query blocks,
// or the tile table of variable blocks) lives in this file-scope device
// array instead of a caller workspace. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): its
// device address, one per GPU, comes from hipGetSymbolAddress and is kept
// per device.
namespace {
constexpr size_t kScratchInts = (size_t)1 << 18;   // 1 MiB: B*H*(nqb+1) <= 262144
static __device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(int32_t** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "attn_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(BSA_EUNSUPPORTED, "attn_fwd_noalloc: device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
      return hip_status(e, "attn_fwd_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return fail(BSA_EHIP, "attn_fwd_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<int32_t*>(g_scratch_ptr[dev]);
  return BSA_OK;
}
}  // namespace

extern "C" {

size_t bsa_block_sparse_attn_fwd_noalloc_capacity(void) { return sizeof(int32_t) * kScratchInts; }

int bsa_block_sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                                      int d, int n_valid, int block, const bsa_blocks* qb, const bsa_blocks* kb,
                                      const int32_t* kv_count, const int32_t* kv_index, int kv_stride, float scale,
                                      hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  bsa::Blocks bq;
  if (int e = make_blocks(qb, block, n_valid, "query blocks", bq)) return e;
  const size_t need = attn_fwd_min_ws(B, H, bq.nblocks);
  if (need > sizeof(int32_t) * kScratchInts)
    return fail(BSA_ENOSPC,
                "attn_fwd_noalloc: B*H*(nqb+1) = %zu int32 entries exceed the fixed scratch of %zu; "
                "use bsa_block_sparse_attn_fwd with a workspace",
                (size_t)B * H * ((size_t)bq.nblocks + 1), kScratchInts);
  if (!q || !k || !v || !o || !kv_count || !kv_index) return fail(BSA_EINVAL, "attn_fwd_noalloc: null pointer");
  int32_t* ws = nullptr;
  if (int e = scratch_address(&ws)) return e;
  return attn_fwd_impl(q, k, v, o, B, H, N, d, n_valid, block, qb, kb, kv_count, kv_index, kv_stride, scale,
                       nullptr, ws, sizeof(int32_t) * kScratchInts, stream);
}

int bsa_block_sparse_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                  int N, int d, int n_valid, int block, const bsa_blocks* qb,
                                  const bsa_blocks* kb, const int32_t* kv_count, const int32_t* kv_index,
                                  int kv_stride, float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (!lse) return fail(BSA_EINVAL, "attn_fwd_lse: null lse");
  if (!aligned16(lse)) return fail(BSA_EINVAL, "attn_fwd_lse: lse must be 16-byte aligned");
  return attn_fwd_impl(q, k, v, o, B, H, N, d, n_valid, block, qb, kb, kv_count, kv_index, kv_stride, scale, lse,
                       ws, ws_bytes, stream);
}

size_t bsa_block_sparse_attn_bwd_workspace(int B, int H, int N, const bsa_blocks* qb, const bsa_blocks* kb) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  const int nqb = qb ? qb->nblocks : (N + 63) / 64, nkb = kb ? kb->nblocks : (N + 63) / 64;
  if (nqb < 0 || nkb < 0) return 0;
  return bsa::attn_bwd_workspace(B * H, N, nqb, nkb);
}

int bsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, int B, int H, int N, int d, int n_valid, int block,
                              const bsa_blocks* qb, const bsa_blocks* kb, const int32_t* kv_count,
                              const int32_t* kv_index, int kv_stride, float scale, void* dq, void* dk, void* dv,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (!q || !k || !v || !o || !dout || !lse || !kv_count || !kv_index || !dq || !dk || !dv)
    return fail(BSA_EINVAL, "attn_bwd: null pointer");
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(BSA_EINVAL, "attn_bwd: tensors must be 16-byte aligned");
  if ((long long)N * d * 2 > 0xFFFFFFFFLL)
    return fail(BSA_EUNSUPPORTED, "attn_bwd: one head (N*d*2 bytes) must be below 4 GiB");
  bsa::Blocks bq, bk;
  if (int e = make_blocks(qb, block, n_valid, "attn_bwd query blocks", bq)) return e;
  if (int e = make_blocks(kb, block, n_valid, "attn_bwd key blocks", bk)) return e;
  if ((qb && bq.max_len == 0) || (kb && bk.max_len == 0))
    return fail(BSA_EUNSUPPORTED, "attn_bwd: block descriptors need a length bound max_len in 1..64");
  if (kv_stride < 0 || (bk.nblocks > 0 && kv_stride < 1)) return fail(BSA_EINVAL, "attn_bwd: bad kv_stride");
  const size_t need = bsa::attn_bwd_workspace(B * H, N, bq.nblocks, bk.nblocks);
  if (ws == nullptr || ws_bytes < need)
    return fail(BSA_ENOSPC, "attn_bwd: workspace %zu bytes < %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(BSA_EINVAL, "attn_bwd: workspace must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return hip_status(bsa::launch_attn_bwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
                                         static_cast<const uint16_t*>(dout), lse, B * H, N, d, n_valid, bq, bk,
                                         kv_count, kv_index, kv_stride, sc, static_cast<uint16_t*>(dq),
                                         static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), ws, stream),
                    "attn_bwd");
}

static int permute_common(const void* x, void* y, const int32_t* perm, int B, int H, int N, int d,
                          int per_head, bool inverse, hipStream_t stream) {
  g_msg[0] = 0;
  if (B <= 0 || H <= 0 || N <= 0) return fail(BSA_EINVAL, "permute: B, H, N must be positive");
  if ((long long)B * H > 65535) return fail(BSA_EUNSUPPORTED, "B*H must be <= 65535");
  if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "permute: d must be 64 or 128");
  if (!x || !y || !perm) return fail(BSA_EINVAL, "permute: null pointer");
  if (x == y) return fail(BSA_EINVAL, "permute: x and y must not overlap");
  if (!aligned16(x) || !aligned16(y)) return fail(BSA_EINVAL, "permute: x, y must be 16-byte aligned");
  return hip_status(bsa::launch_permute(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), perm, B * H, N,
                                        d, per_head, inverse, stream),
                    "permute");
}

int bsa_permute_tokens(const void* x, void* y, const int32_t* perm, int B, int H, int N, int d, int perm_per_head,
                       hipStream_t stream) {
  return permute_common(x, y, perm, B, H, N, d, perm_per_head, false, stream);
}

int bsa_unpermute_tokens(const void* x, void* y, const int32_t* perm, int B, int H, int N, int d, int perm_per_head,
                         hipStream_t stream) {
  return permute_common(x, y, perm, B, H, N, d, perm_per_head, true, stream);
}

int bsa_tile_order(int T, int Hl, int Wl, int pt, int ph, int pw, int N, int32_t* perm, int32_t* blk_start,
                   int32_t* blk_len, int32_t* blk_coords, int max_blocks, int* nblocks) {
  g_msg[0] = 0;
  if (T <= 0 || Hl <= 0 || Wl <= 0) return fail(BSA_EINVAL, "tile_order: latent sizes must be positive");
  if (pt <= 0 || ph <= 0 || pw <= 0) return fail(BSA_EINVAL, "tile_order: box sizes must be positive");
  const long long n = (long long)T * Hl * Wl;
  if (n > 0x7fffffffLL || N < n) return fail(BSA_EINVAL, "tile_order: N must be >= T*Hl*Wl");
  if (!perm || !blk_start || !blk_len || !nblocks) return fail(BSA_EINVAL, "tile_order: null pointer");
  const int nbt = (T + pt - 1) / pt, nby = (Hl + ph - 1) / ph, nbx = (Wl + pw - 1) / pw;
  const long long nb = (long long)nbt * nby * nbx;
  *nblocks = (int)nb;
  if (nb > max_blocks) return fail(BSA_ENOSPC, "tile_order: %lld blocks > max_blocks %d", nb, max_blocks);
  // walk the boxes in grid order and each box in raster order
  int pos = 0, b = 0;
  for (int bt = 0; bt < nbt; ++bt)
    for (int by = 0; by < nby; ++by)
      for (int bx = 0; bx < nbx; ++bx) {
        blk_start[b] = pos;
        const int t1 = std::min(T, bt * pt + pt), y1 = std::min(Hl, by * ph + ph), x1 = std::min(Wl, bx * pw + pw);
        for (int t = bt * pt; t < t1; ++t)
          for (int y = by * ph; y < y1; ++y)
            for (int x = bx * pw; x < x1; ++x) perm[pos++] = (t * Hl + y) * Wl + x;
        blk_len[b] = pos - blk_start[b];
        if (blk_coords) {
          blk_coords[3 * b + 0] = bt;
          blk_coords[3 * b + 1] = by;
          blk_coords[3 * b + 2] = bx;
        }
        ++b;
      }
  for (int i = (int)n; i < N; ++i) perm[i] = i;
  return BSA_OK;
}

int bsa_fractal_order(int T, int Hl, int Wl, int P, int N, int32_t* perm, int32_t* blk_start, int32_t* blk_len,
                      int32_t* blk_coords, int max_blocks, int* nblocks) {
  // P x P patches of one frame: boxes of 1 x P x P
  if (P <= 0) {
    g_msg[0] = 0;
    return fail(BSA_EINVAL, "fractal_order: sizes must be positive");
  }
  return bsa_tile_order(T, Hl, Wl, 1, P, P, N, perm, blk_start, blk_len, blk_coords, max_blocks, nblocks);
}

int bsa_attention_tile_stats(const void* q, const void* k, const float* lse, int B, int H, int N, int d,
                             int n_valid, float scale, float* tile_max, float* tile_sum, float* tile_min,
                             hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (d != 64 && d != 128) return fail(BSA_EUNSUPPORTED, "tile_stats: d must be 64 or 128");
  if (!q || !k || !lse || !tile_max || !tile_sum || !tile_min) return fail(BSA_EINVAL, "tile_stats: null pointer");
  if (!aligned16(q) || !aligned16(k)) return fail(BSA_EINVAL, "tile_stats: q, k must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)d);
  return hip_status(bsa::launch_tile_stats(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), lse,
                                           B * H, N, d, n_valid, sc, tile_max, tile_sum, tile_min, stream),
                    "tile_stats");
}

int bsa_mask_recall(const float* tile_max, const float* tile_sum, const int32_t* kv_count, const int32_t* kv_index,
                    int kv_stride, int B, int H, int nqb, int nkb, float* oracle_recall, float* mass_recall,
                    hipStream_t stream) {
  g_msg[0] = 0;
  if (B <= 0 || H <= 0 || nqb < 0 || nkb <= 0) return fail(BSA_EINVAL, "mask_recall: bad sizes");
  if (nkb > 8192) return fail(BSA_EUNSUPPORTED, "mask_recall: at most 8192 key blocks (got %d)", nkb);
  if (kv_stride < 1) return fail(BSA_EINVAL, "mask_recall: kv_stride must be >= 1");
  if (!tile_max || !tile_sum || !kv_count || !kv_index || !oracle_recall || !mass_recall)
    return fail(BSA_EINVAL, "mask_recall: null pointer");
  return hip_status(bsa::launch_mask_recall(tile_max, tile_sum, kv_count, kv_index, kv_stride,
                                            (size_t)B * H * nqb, nkb, oracle_recall, mass_recall, stream),
                    "mask_recall");
}

int bsa_check_mask(const int32_t* kv_count, const int32_t* kv_index, int B, int H, int nqb, int nkb, int kv_stride,
                   int32_t* bad, hipStream_t stream) {
  g_msg[0] = 0;
  if (B <= 0 || H <= 0 || nqb < 0 || nkb <= 0) return fail(BSA_EINVAL, "check_mask: bad sizes");
  if (kv_stride < 1) return fail(BSA_EINVAL, "check_mask: kv_stride must be >= 1");
  if (!kv_count || !kv_index || !bad) return fail(BSA_EINVAL, "check_mask: null pointer");
  return hip_status(bsa::launch_check_mask(kv_count, kv_index, (size_t)B * H * nqb, nkb, kv_stride, bad, stream),
                    "check_mask");
}

size_t bsa_kmeans_workspace(int B, int H, int N, int C, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || C <= 0) return 0;
  return bsa::kmeans_ws_bytes(B * H, N, C, d);
}

int bsa_kmeans(const void* x, int B, int H, int N, int d, int n_valid, int C, int iters, const float* uniforms,
               float* centroids, int32_t* assign, int32_t* sizes, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (C < 1 || C > 1024) return fail(BSA_EUNSUPPORTED, "kmeans: C must be in [1, 1024] (got %d)", C);
  if (C > n_valid) return fail(BSA_EINVAL, "kmeans: C=%d exceeds n_valid=%d", C, n_valid);
  if (iters < 0) return fail(BSA_EINVAL, "kmeans: iters must be >= 0");
  if (!x || !uniforms || !centroids || !assign || !sizes) return fail(BSA_EINVAL, "kmeans: null pointer");
  if (!aligned16(x)) return fail(BSA_EINVAL, "kmeans: x must be 16-byte aligned");
  const size_t need = bsa_kmeans_workspace(B, H, N, C, d);
  if (ws == nullptr || ws_bytes < need) return fail(BSA_ENOSPC, "kmeans: workspace %zu bytes < %zu", ws_bytes, need);
  return hip_status(bsa::launch_kmeans(static_cast<const uint16_t*>(x), B * H, N, d, n_valid, C, iters, uniforms,
                                       centroids, assign, sizes, nullptr, 0, ws, stream),
                    "kmeans");
}

int bsa_kmeans_warm(const void* x, int B, int H, int N, int d, int n_valid, int C, int max_iters, int tol_moves,
                    float* centroids, int32_t* assign, int32_t* sizes, int32_t* changes, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  g_msg[0] = 0;
  if (int e = check_shape(B, H, N, d, n_valid)) return e;
  if (C < 1 || C > 1024) return fail(BSA_EUNSUPPORTED, "kmeans_warm: C must be in [1, 1024] (got %d)", C);
  if (C > n_valid) return fail(BSA_EINVAL, "kmeans_warm: C=%d exceeds n_valid=%d", C, n_valid);
  if (max_iters < 1) return fail(BSA_EINVAL, "kmeans_warm: max_iters must be >= 1");
  if (tol_moves < 0) return fail(BSA_EINVAL, "kmeans_warm: tol_moves must be >= 0");
  if (!x || !centroids || !assign || !sizes || !changes) return fail(BSA_EINVAL, "kmeans_warm: null pointer");
  if (!aligned16(x)) return fail(BSA_EINVAL, "kmeans_warm: x must be 16-byte aligned");
  const size_t need = bsa_kmeans_workspace(B, H, N, C, d);
  if (ws == nullptr || ws_bytes < need)
    return fail(BSA_ENOSPC, "kmeans_warm: workspace %zu bytes < %zu", ws_bytes, need);
  return hip_status(bsa::launch_kmeans(static_cast<const uint16_t*>(x), B * H, N, d, n_valid, C, max_iters,
                                       nullptr, centroids, assign, sizes, changes, tol_moves, ws, stream),
                    "kmeans_warm");
}

size_t bsa_cluster_order_workspace(int B, int H, int N, int C) {
  if (B <= 0 || H <= 0 || N <= 0 || C <= 0) return 0;
  return bsa::cluster_order_ws_bytes(B * H, N, C);
}

int bsa_cluster_order(const int32_t* assign, int B, int H, int N, int n_valid, int C, int32_t* perm, int32_t* start,
                      int32_t* len, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (B <= 0 || H <= 0 || N <= 0) return fail(BSA_EINVAL, "cluster_order: B, H, N must be positive");
  if ((long long)B * H > 65535) return fail(BSA_EUNSUPPORTED, "B*H must be <= 65535");
  if (n_valid <= 0 || n_valid > N) return fail(BSA_EINVAL, "cluster_order: n_valid must be in [1, N]");
  if (C < 1 || C > 1024) return fail(BSA_EUNSUPPORTED, "cluster_order: C must be in [1, 1024]");
  if (!assign || !perm || !start || !len) return fail(BSA_EINVAL, "cluster_order: null pointer");
  const size_t need = bsa_cluster_order_workspace(B, H, N, C);
  if (ws == nullptr || ws_bytes < need) return fail(BSA_ENOSPC, "cluster_order: workspace %zu bytes < %zu", ws_bytes, need);
  return hip_status(bsa::launch_cluster_order(assign, B * H, N, n_valid, C, perm, start, len, ws, stream),
                    "cluster_order");
}

}  // extern "C"

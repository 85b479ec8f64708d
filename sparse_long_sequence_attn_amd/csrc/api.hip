// C ABI of the dilated-attention library: argument validation, the launch
// plan (pattern geometry, tile order, workspace layout) and the launches.
// Every check runs before the first launch, so a failing call launches and
// writes nothing. The library keeps no state between calls.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "da_common.hpp"
#include "dilated_attn.h"
#include "kernels.hpp"

namespace {

using da::kDh;
using da::kMaxPat;
using da::PatDev;

constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr float kLog2e = 1.44269504088896340736f;

// Order of the tiles of all patterns in one launch (see AttnArgs).
struct TileOrder {
  int32_t ntile[kMaxPat];  // tiles per unit, caller's pattern order
  int order[kMaxPat];      // pattern indices sorted by ntile, descending
  int64_t unit_start[kMaxPat + 1];
  int64_t grid = 0;  // kXcds * (longest per-XCD tile list)
};

struct Plan {
  bool empty = false;
  bool bf16 = false;
  bool causal = true;
  int nw = 4;
  int np = 0;
  int64_t B = 0, N = 0;
  int32_t H = 0;
  float sl2 = 0.f;
  float scale = 0.f;
  PatDev pat[kMaxPat];     // caller's order
  TileOrder fwd;           // forward attention tiles
  TileOrder bwd;           // backward tiles (32 * nw rows)
  size_t ws_bytes = 0;
  size_t tensor_bytes = 0;
  size_t lse_bytes = 0;
  // backward workspace: D at float offset 0, then per pattern (two or more
  // patterns) the dq, dk, dv partial blocks at bwd_po_off[i]
  int64_t bwd_po_off[kMaxPat];
  size_t bwd_ws_bytes = 0;
};

int64_t align64(int64_t x) { return (x + 63) & ~int64_t(63); }

// Tiles of bm rows per unit, patterns sorted by tile count (descending),
// units dealt to the XCDs round-robin in that order; grid = kXcds times the
// longest per-XCD tile list.
int tile_order(const Plan* pl, int bm, TileOrder* to) {
  const int np = pl->np;
  for (int i = 0; i < np; ++i) to->ntile[i] = (pl->pat[i].lmax + bm - 1) / bm;
  for (int i = 0; i < np; ++i) to->order[i] = i;
  std::stable_sort(to->order, to->order + np,
                   [&](int x, int y) { return to->ntile[x] > to->ntile[y]; });
  to->unit_start[0] = 0;
  for (int j = 0; j < np; ++j)
    to->unit_start[j + 1] = to->unit_start[j] + pl->pat[to->order[j]].units;
  int64_t per_xcd[da::kXcds] = {0};
  for (int j = 0; j < np; ++j) {
    const int64_t u0 = to->unit_start[j], u1 = to->unit_start[j + 1];
    for (int x = 0; x < da::kXcds; ++x) {
      const int64_t first = u0 + (((x - u0) % da::kXcds) + da::kXcds) % da::kXcds;
      const int64_t cnt = first < u1 ? (u1 - first + da::kXcds - 1) / da::kXcds : 0;
      per_xcd[x] += cnt * to->ntile[to->order[j]];
    }
  }
  int64_t longest = 0;
  for (int x = 0; x < da::kXcds; ++x) longest = std::max(longest, per_xcd[x]);
  to->grid = longest * da::kXcds;
  return to->grid > kMaxGrid ? DA_ERR_SHAPE : DA_OK;
}

// Patterns in a launch's sorted order, with that launch's tile counts.
void sorted_patterns(const Plan& pl, const TileOrder& to, PatDev* dst, int64_t* unit_start) {
  for (int j = 0; j < pl.np; ++j) {
    dst[j] = pl.pat[to.order[j]];
    da::set_tile_divisors(&dst[j], to.ntile[to.order[j]], j == pl.np - 1);
  }
  for (int j = 0; j <= pl.np; ++j) unit_start[j] = to.unit_start[j];
}

// Shapes, patterns, dtype and scalars; computes everything that does not
// depend on pointers.
int make_plan(int64_t B, int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
              int32_t n_patterns, int32_t causal, int32_t dtype, float scale, Plan* pl) {
  if (dtype != DA_F32 && dtype != DA_BF16) return DA_ERR_DTYPE;
  if (Dh != DA_HEAD_DIM) return DA_ERR_HEADDIM;
  if (n_patterns < 1 || n_patterns > DA_MAX_PATTERNS) return DA_ERR_PATTERN;
  if (!patterns) return DA_ERR_NULL;
  if (B < 0 || N < 0 || H < 0) return DA_ERR_SHAPE;
  // sizes the kernels index with 32-bit positions and grid dimensions
  if (N > kMaxGrid || H > 65535 || B > 65535 || N * (int64_t)H > kMaxGrid) return DA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return DA_ERR_ARG;
  if (!isfinite(scale)) return DA_ERR_ARG;
  for (int i = 0; i < n_patterns; ++i) {
    if (patterns[i].w < 1 || patterns[i].r < 1) return DA_ERR_PATTERN;
    if (N > 0) {
      const int64_t wp = std::min<int64_t>(patterns[i].w, N);
      if (N % wp != 0) return DA_ERR_SHAPE;
      if (patterns[i].r > wp) return DA_ERR_PATTERN;
      // the attention kernel addresses one segment's rows with 32-bit byte
      // offsets (plus at most one 128-row tile of overrun)
      const int64_t esize = dtype == DA_BF16 ? 2 : 4;
      if ((wp + 128 * (int64_t)patterns[i].r) * H * Dh * esize > kMaxGrid) return DA_ERR_SHAPE;
    }
  }
  pl->bf16 = dtype == DA_BF16;
  pl->causal = causal != 0;
  pl->np = n_patterns;
  pl->B = B;
  pl->N = N;
  pl->H = H;
  const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)Dh);
  pl->sl2 = (float)(sc * (double)kLog2e);
  pl->scale = (float)sc;
  pl->tensor_bytes = (size_t)(B * N * H * Dh) * (pl->bf16 ? 2 : 4);
  pl->lse_bytes = (size_t)(B * N * H) * 4;
  pl->empty = B == 0 || N == 0 || H == 0;
  if (pl->empty) return DA_OK;

  int32_t lmax_all = 0;
  for (int i = 0; i < n_patterns; ++i) {
    PatDev& p = pl->pat[i];
    memset(&p, 0, sizeof p);
    p.wp = std::min<int64_t>(patterns[i].w, N);
    p.nseg = N / p.wp;
    p.r = patterns[i].r;
    p.lmax = da::rows_gathered(p.wp, 0, p.r);
    p.units = B * H * p.nseg;
    p.wp_div = da::make_fastdiv((uint32_t)p.wp);
    p.r_div = da::make_fastdiv((uint32_t)p.r);
    lmax_all = std::max(lmax_all, p.lmax);
  }
  // one 32-row wave per workgroup when every segment is that short
  pl->nw = lmax_all > 32 ? 4 : 1;
  int rc = tile_order(pl, da::attn_tile_rows(pl->bf16, pl->nw), &pl->fwd);
  if (rc != DA_OK) return rc;
  rc = tile_order(pl, 32 * pl->nw, &pl->bwd);
  if (rc != DA_OK) return rc;

  // partial outputs and log2-sum-exp per pattern, 256-byte aligned regions
  int64_t cur = 0;
  if (n_patterns > 1) {
    for (int i = 0; i < n_patterns; ++i) {
      PatDev& p = pl->pat[i];
      const int64_t rows = B * H * p.nseg * p.lmax;
      p.po_off = cur;
      cur += align64(rows * kDh);
      p.pl_off = cur;
      cur += align64(rows);
    }
  }
  pl->ws_bytes = (size_t)cur * 4;

  // backward: D per row, then dq, dk, dv partial blocks per pattern, in the
  // gradients' dtype (offsets and sizes here count 4-byte words)
  cur = align64(B * H * N);
  for (int i = 0; i < n_patterns; ++i) {
    pl->bwd_po_off[i] = -1;
    if (n_patterns > 1) {
      pl->bwd_po_off[i] = cur;
      const int64_t elems = 3 * B * H * pl->pat[i].nseg * pl->pat[i].lmax * kDh;
      cur += align64(pl->bf16 ? elems / 2 : elems);  // kDh is even
    }
  }
  pl->bwd_ws_bytes = (size_t)cur * 4;
  return DA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// A buffer's bytes for the alias checks: a dense range, or rows of `row`
// bytes every `stride` bytes (tensors that interleave in one buffer).
struct Region {
  const void* p;
  size_t bytes;       // first to last byte touched
  size_t stride = 0;  // 0: every byte of the range
  size_t row = 0;
};
Region dense(const void* p, size_t bytes) { return Region{p, bytes, 0, 0}; }
Region rows_of(const void* p, int64_t rows, size_t stride, size_t row) {
  return Region{p, rows > 0 ? (size_t)(rows - 1) * stride + row : 0, stride, row};
}
// Whether two regions may share a byte: two row sets with the same stride
// and row size are apart when their offset, modulo the stride, keeps every
// row of one between rows of the other.
bool collide(const Region& a, const Region& b) {
  if (!overlaps(a.p, a.bytes, b.p, b.bytes)) return false;
  if (a.stride && a.stride == b.stride && a.row == b.row && a.stride >= 2 * a.row) {
    const int64_t st = (int64_t)a.stride;
    const int64_t d = (((int64_t)((uintptr_t)b.p - (uintptr_t)a.p)) % st + st) % st;
    return d < (int64_t)a.row || d > st - (int64_t)a.row;
  }
  return true;
}

// Row stride (elements between consecutive positions) of the fused qk_norm
// entry points' q, k, v (and dq, dk, dv): 0 means H * Dh.
int qkn_row_stride(const Plan& pl, int64_t given, int64_t* rsi) {
  const int64_t hd = (int64_t)pl.H * DA_HEAD_DIM;
  const int64_t es = pl.bf16 ? 2 : 4;
  *rsi = given == 0 ? hd : given;
  if (given < 0 || (given != 0 && given < hd)) return DA_ERR_ARG;
  if ((*rsi * es) % 16 != 0) return DA_ERR_ALIGN;
  // the kernels address one segment's rows with 32-bit byte offsets
  for (int i = 0; i < pl.np; ++i)
    if ((pl.pat[i].wp + 128 * (int64_t)pl.pat[i].r) * *rsi * es > kMaxGrid) return DA_ERR_SHAPE;
  return DA_OK;
}

// with_ws false: the tensors only (the workspace is checked once it is known)
int check_buffers(const Plan& pl, const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const void* ws, size_t ws_bytes, bool with_ws = true) {
  if (!q || !k || !v || !out || !lse) return DA_ERR_NULL;
  if (!with_ws) {
    ws = nullptr;
  } else {
    if (pl.ws_bytes > 0 && !ws) return DA_ERR_WORKSPACE;
    if (ws_bytes < pl.ws_bytes) return DA_ERR_WORKSPACE;
  }
  auto mis = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; };
  if (mis(q, 16) || mis(k, 16) || mis(v, 16) || mis(out, 16) || mis(lse, 4)) return DA_ERR_ALIGN;
  if (pl.ws_bytes > 0 && mis(ws, 256)) return DA_ERR_ALIGN;
  const size_t tb = pl.tensor_bytes, lb = pl.lse_bytes, wb = pl.ws_bytes;
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (overlaps(out, tb, in, tb) || overlaps(lse, lb, in, tb) || overlaps(ws, wb, in, tb))
      return DA_ERR_ALIAS;
  if (overlaps(out, tb, lse, lb) || overlaps(out, tb, ws, wb) || overlaps(lse, lb, ws, wb))
    return DA_ERR_ALIAS;
  return DA_OK;
}

// qkn: gain_q, bias_q, gain_k, bias_k of the fused qk_norm, or null
int run_attention(const Plan& pl, const void* q, const void* k, const void* v, void* out,
                  float* lse, void* ws, hipStream_t st, const void* const* qkn = nullptr,
                  float qkn_eps = 0.f, int64_t in_rs = 0) {
  da::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.ws = reinterpret_cast<float*>(ws);
  a.B = pl.B;
  a.N = pl.N;
  a.H = pl.H;
  a.np = pl.np;
  a.sl2 = pl.sl2;
  a.h_div = da::make_fastdiv((uint32_t)pl.H);
  sorted_patterns(pl, pl.fwd, a.pat, a.unit_start);
  hipError_t e;
  a.in_rs = in_rs ? in_rs : (int64_t)pl.H * DA_HEAD_DIM;
  if (qkn) {
    for (int i = 0; i < 4; ++i) a.qkn[i] = qkn[i];
    a.qkn_eps = qkn_eps;
    e = da::launch_attention_qkn(a, pl.bf16, pl.causal, pl.fwd.grid, st);
  } else {
    e = da::launch_attention(a, pl.bf16, pl.nw, pl.causal, pl.np == 1, pl.fwd.grid, st);
  }
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int run_merge(const Plan& pl, void* out, float* lse, const void* ws, hipStream_t st) {
  if (pl.np == 1) return DA_OK;
  da::MergeArgs m;
  memset(&m, 0, sizeof m);
  m.out = out;
  m.lse = lse;
  m.ws = reinterpret_cast<const float*>(ws);
  m.B = pl.B;
  m.N = pl.N;
  m.H = pl.H;
  m.np = pl.np;
  for (int i = 0; i < pl.np; ++i) m.pat[i] = pl.pat[i];
  const hipError_t e = da::launch_merge(m, pl.bf16, st);
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// Workspace of the allocation-free forward entry point: one array per GPU,
// held by the loaded code object until the process ends. Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol); the per-device address comes from hipGetSymbolAddress.
__device__ __attribute__((aligned(256))) unsigned char scratch[DA_NOALLOC_MAX_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream), looked up once per device with that device
// current.
int scratch_address(void* stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return DA_ERR_LAUNCH;
  dev = cur;
  if (stream && hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return DA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return DA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DA_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return DA_ERR_LAUNCH;
    if (e != hipSuccess || !p) return DA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DA_OK;
}

enum Stage { kBoth = 3, kAttention = 1, kMerge = 2 };

int fwd_common(int stages, const void* q, const void* k, const void* v, void* out, float* lse,
               int64_t B, int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
               int32_t n_patterns, int32_t causal, int32_t dtype, float scale, void* workspace,
               size_t workspace_bytes, void* stream) {
  Plan pl;
  int rc = make_plan(B, N, H, Dh, patterns, n_patterns, causal, dtype, scale, &pl);
  if (rc != DA_OK || pl.empty) return rc;
  rc = check_buffers(pl, q, k, v, out, lse, workspace, workspace_bytes);
  if (rc != DA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (stages & kAttention) {
    rc = run_attention(pl, q, k, v, out, lse, workspace, st);
    if (rc != DA_OK) return rc;
  }
  if (stages & kMerge) rc = run_merge(pl, out, lse, workspace, st);
  return rc;
}

// ---------------------------------------------------------------- backward

int check_bwd_buffers(const Plan& pl, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, const void* dout, const void* dq,
                      const void* dk, const void* dv, const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return DA_ERR_NULL;
  if (!ws || ws_bytes < pl.bwd_ws_bytes) return DA_ERR_WORKSPACE;
  auto mis = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; };
  const void* t16[8] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* t : t16)
    if (mis(t, 16)) return DA_ERR_ALIGN;
  if (mis(lse, 4) || mis(ws, 256)) return DA_ERR_ALIGN;
  const size_t tb = pl.tensor_bytes, lb = pl.lse_bytes, wb = pl.bwd_ws_bytes;
  const void* outs[4] = {dq, dk, dv, ws};
  const size_t osz[4] = {tb, tb, tb, wb};
  const void* ins[6] = {q, k, v, out, dout, lse};
  const size_t isz[6] = {tb, tb, tb, tb, tb, lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return DA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return DA_ERR_ALIAS;
  }
  return DA_OK;
}

// The fused form serves one pattern whose segments gather at most 32 rows
// (the plan's one-wave case), where every output row is final.
int qkn_params_check(const Plan& pl, const void* const* gb, float eps, const void* const* outs,
                     const size_t* out_bytes, int n_outs) {
  if (!isfinite(eps) || !(eps > 0.f)) return DA_ERR_ARG;
  if (pl.empty) return DA_OK;
  if (pl.np != 1 || pl.nw != 1) return DA_ERR_PATTERN;
  const size_t pb = (size_t)DA_HEAD_DIM * (pl.bf16 ? 2 : 4);
  for (int i = 0; i < 4; ++i) {
    if (!gb[i]) return DA_ERR_NULL;
    if (((uintptr_t)gb[i] & 15) != 0) return DA_ERR_ALIGN;
    for (int j = 0; j < n_outs; ++j)
      if (overlaps(outs[j], out_bytes[j], gb[i], pb)) return DA_ERR_ALIAS;
  }
  return DA_OK;
}

// Workspace of the fused qk_norm backward: the plain backward's, then the
// per-unit gain/bias partials [2][units][2 kDh], then their folded form
// [2][groups][2 kDh] (floats, 256-byte aligned regions).
size_t qkn_part_offset(const Plan& pl) { return (pl.bwd_ws_bytes + 255) & ~(size_t)255; }
size_t qkn_fold_offset(const Plan& pl) {
  const size_t part = (size_t)2 * pl.pat[0].units * 2 * DA_HEAD_DIM * 4;
  return (qkn_part_offset(pl) + part + 255) & ~(size_t)255;
}
size_t qkn_bwd_ws_bytes(const Plan& pl) {
  return qkn_fold_offset(pl) + (size_t)2 * da::qkn_groups(pl.pat[0].units) * 2 * DA_HEAD_DIM * 4;
}

// qkn (gain_q, bias_q, gain_k, bias_k) and dparams are set for the fused
// qk_norm backward (checked by the caller), null otherwise.
int bwd_common(int stages, const void* q, const void* k, const void* v, const void* out,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t B,
               int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns, int32_t n_patterns,
               int32_t causal, int32_t dtype, float scale, void* workspace,
               size_t workspace_bytes, void* stream, const void* const* qkn = nullptr,
               float qkn_eps = 0.f, float* dparams = nullptr, int64_t row_stride = 0) {
  if (stages < 1 || stages > DA_BWD_ALL) return DA_ERR_ARG;
  Plan pl;
  int rc = make_plan(B, N, H, Dh, patterns, n_patterns, causal, dtype, scale, &pl);
  if (rc != DA_OK) return rc;
  int64_t rsi = (int64_t)pl.H * DA_HEAD_DIM;
  if (qkn) {
    const void* outs[4] = {dq, dk, dv, dparams};
    const size_t ob[4] = {pl.tensor_bytes, pl.tensor_bytes, pl.tensor_bytes,
                          (size_t)4 * DA_HEAD_DIM * 4};
    rc = qkn_params_check(pl, qkn, qkn_eps, outs, ob, 4);
    if (rc != DA_OK || pl.empty) return rc;
    const void* wsv[1] = {workspace};
    const size_t wsb[1] = {qkn_bwd_ws_bytes(pl)};
    rc = qkn_params_check(pl, qkn, qkn_eps, wsv, wsb, 1);
    if (rc != DA_OK) return rc;
    if (!dparams) return DA_ERR_NULL;
    if (((uintptr_t)dparams & 3) != 0) return DA_ERR_ALIGN;
    const size_t pb = (size_t)4 * DA_HEAD_DIM * 4;
    const void* ins[6] = {q, k, v, out, dout, lse};
    const size_t isz[6] = {pl.tensor_bytes, pl.tensor_bytes, pl.tensor_bytes, pl.tensor_bytes,
                           pl.tensor_bytes, pl.lse_bytes};
    for (int j = 0; j < 6; ++j)
      if (overlaps(dparams, pb, ins[j], isz[j])) return DA_ERR_ALIAS;
    for (int j = 0; j < 3; ++j)
      if (overlaps(dparams, pb, outs[j], pl.tensor_bytes)) return DA_ERR_ALIAS;
    if (overlaps(dparams, pb, workspace, qkn_bwd_ws_bytes(pl))) return DA_ERR_ALIAS;
    rc = qkn_row_stride(pl, row_stride, &rsi);
    if (rc != DA_OK) return rc;
  }
  if (pl.empty) return DA_OK;
  Plan chk = pl;  // the fused qk_norm backward needs room for its partials
  if (qkn) chk.bwd_ws_bytes = qkn_bwd_ws_bytes(pl);
  if (qkn && rsi != (int64_t)pl.H * DA_HEAD_DIM) {
    // q, k, v and dq, dk, dv as rows every rsi elements (they may interleave)
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return DA_ERR_NULL;
    if (!workspace || workspace_bytes < chk.bwd_ws_bytes) return DA_ERR_WORKSPACE;
    auto mis = [](const void* p, uintptr_t al) { return ((uintptr_t)p & (al - 1)) != 0; };
    const void* t16[8] = {q, k, v, out, dout, dq, dk, dv};
    for (const void* t : t16)
      if (mis(t, 16)) return DA_ERR_ALIGN;
    if (mis(lse, 4) || mis(workspace, 256)) return DA_ERR_ALIGN;
    const int64_t es = pl.bf16 ? 2 : 4, rows = pl.B * pl.N;
    const size_t rb = (size_t)(rsi * es), row = (size_t)(pl.H * DA_HEAD_DIM * es);
    const Region ins[6] = {rows_of(q, rows, rb, row),       rows_of(k, rows, rb, row),
                           rows_of(v, rows, rb, row),       dense(out, pl.tensor_bytes),
                           dense(dout, pl.tensor_bytes),    dense(lse, pl.lse_bytes)};
    const Region outs[4] = {rows_of(dq, rows, rb, row), rows_of(dk, rows, rb, row),
                            rows_of(dv, rows, rb, row), dense(workspace, chk.bwd_ws_bytes)};
    for (int i = 0; i < 4; ++i) {
      for (int j = 0; j < 6; ++j)
        if (collide(outs[i], ins[j])) return DA_ERR_ALIAS;
      for (int j = i + 1; j < 4; ++j)
        if (collide(outs[i], outs[j])) return DA_ERR_ALIAS;
    }
  } else {
    rc = check_bwd_buffers(chk, q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes);
    if (rc != DA_OK) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* ws = reinterpret_cast<float*>(workspace);

  da::BwdRowArgs ra;
  memset(&ra, 0, sizeof ra);
  ra.out = out;
  ra.dout = dout;
  ra.dvec = ws;
  ra.dq = dq;
  ra.dk = dk;
  ra.dv = dv;
  ra.ws = ws;
  ra.B = pl.B;
  ra.N = pl.N;
  ra.H = pl.H;
  ra.np = pl.np;
  ra.grad_rs = rsi;
  for (int i = 0; i < pl.np; ++i) {
    ra.pat[i] = pl.pat[i];
    ra.pat[i].po_off = pl.bwd_po_off[i];
  }

  da::BwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.out = out;
  a.lse = lse;
  a.dvec = ws;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = ws;
  a.B = pl.B;
  a.N = pl.N;
  a.H = pl.H;
  a.np = pl.np;
  a.sl2 = pl.sl2;
  a.scale = pl.scale;
  a.h_div = da::make_fastdiv((uint32_t)pl.H);
  sorted_patterns(pl, pl.bwd, a.pat, a.unit_start);
  for (int j = 0; j < pl.np; ++j) a.pat[j].po_off = pl.bwd_po_off[pl.bwd.order[j]];
  float* const qkn_part =
      reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + qkn_part_offset(pl));
  a.in_rs = rsi;
  if (qkn) {
    for (int i = 0; i < 4; ++i) a.qkn[i] = qkn[i];
    a.qkn_eps = qkn_eps;
    a.qkn_part = qkn_part;
    a.qkn_units = pl.pat[0].units;
  }

  hipError_t e = hipSuccess;
  // every segment at most 32 rows: one kernel (in the KV stage) computes D,
  // dq, dk and dv; the PREP and Q stages have nothing to do
  const bool fused = pl.nw == 1;
  if (!fused && (stages & DA_BWD_PREP)) e = da::launch_bwd_prep(ra, pl.bf16, st);
  if (e == hipSuccess && (stages & DA_BWD_KV))
    e = fused ? da::launch_bwd_short(a, pl.bf16, pl.causal, pl.bwd.grid, st)
              : da::launch_bwd_kv(a, pl.bf16, pl.causal, pl.bwd.grid, st);
  if (e == hipSuccess && !fused && (stages & DA_BWD_Q))
    e = da::launch_bwd_q(a, pl.bf16, pl.causal, pl.bwd.grid, st);
  if (e == hipSuccess && (stages & DA_BWD_MERGE)) e = da::launch_bwd_merge(ra, pl.bf16, st);
  if (e == hipSuccess && qkn && (stages & DA_BWD_MERGE)) {
    float* const folded =
        reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + qkn_fold_offset(pl));
    e = da::launch_qkn_fold(qkn_part, pl.pat[0].units, folded, st);
    if (e == hipSuccess)
      e = da::launch_qk_norm_reduce(folded, da::qkn_groups(pl.pat[0].units), dparams, st);
  }
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

// ---------------------------------------------------------------- qk_norm

int qk_norm_check(int64_t rows, int32_t Dh, int32_t dtype, float eps) {
  if (dtype != DA_F32 && dtype != DA_BF16) return DA_ERR_DTYPE;
  if (Dh != DA_HEAD_DIM) return DA_ERR_HEADDIM;
  if (rows < 0 || rows > ((int64_t)1 << 40)) return DA_ERR_SHAPE;
  if (!isfinite(eps) || !(eps > 0.f)) return DA_ERR_ARG;
  return DA_OK;
}

// Geometry of one pattern for the map hooks.
int map_pattern(int64_t N, int32_t H, da_pattern p, int32_t h, PatDev* out) {
  if (N < 1 || N > kMaxGrid || H < 1) return DA_ERR_SHAPE;
  if (h < 0 || h >= H) return DA_ERR_ARG;
  if (p.w < 1 || p.r < 1) return DA_ERR_PATTERN;
  const int64_t wp = std::min<int64_t>(p.w, N);
  if (N % wp != 0) return DA_ERR_SHAPE;
  if (p.r > wp) return DA_ERR_PATTERN;
  memset(out, 0, sizeof *out);
  out->wp = wp;
  out->nseg = N / wp;
  out->r = p.r;
  out->lmax = da::rows_gathered(wp, 0, p.r);
  out->wp_div = da::make_fastdiv((uint32_t)wp);
  out->r_div = da::make_fastdiv((uint32_t)p.r);
  return DA_OK;
}

}  // namespace

extern "C" {

int dilated_attn_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                 const da_pattern* patterns, int32_t n_patterns, int32_t dtype,
                                 size_t* bytes) {
  if (!bytes) return DA_ERR_NULL;
  Plan pl;
  const int rc = make_plan(B, N, H, Dh, patterns, n_patterns, 1, dtype, 0.f, &pl);
  if (rc != DA_OK) return rc;
  *bytes = pl.empty ? 0 : pl.ws_bytes;
  return DA_OK;
}

int dilated_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
                     int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_common(kBoth, q, k, v, out, lse, B, N, H, Dh, patterns, n_patterns, causal, dtype,
                    scale, workspace, workspace_bytes, stream);
}

// One-pass geometry: L = lcm of the dilation rates, W = gcd of the
// effective segment lengths; DA_ERR_PATTERN where the one-pass form does not
// apply (L above W: fewer than one row per residue and window).
int onepass_geometry(const Plan& pl, da::OnePassArgs* a, int64_t* grid) {
  int64_t L = 1, W = 0;
  for (int i = 0; i < pl.np; ++i) {
    const int64_t r = pl.pat[i].r;
    L = L / std::__gcd(L, r) * r;
    if (L > (int64_t)1 << 20) return DA_ERR_PATTERN;
    W = std::__gcd(W, pl.pat[i].wp);
  }
  if (L > W) return DA_ERR_PATTERN;
  const int64_t per_res = (W + L - 1) / L;  // rows of the fullest residue in a window
  a->L = (int32_t)L;
  a->W = (int32_t)W;
  constexpr int64_t bm = 32 * da::kOnePassWaves;
  a->nblk = (int32_t)((per_res + bm - 1) / bm);
  a->nwin = pl.N / W;
  const int64_t groups = pl.B * pl.H * a->nwin;
  *grid = (groups + da::kXcds - 1) / da::kXcds * da::kXcds * L * a->nblk;
  return *grid > kMaxGrid ? DA_ERR_SHAPE : DA_OK;
}

int dilated_attn_fwd_onepass(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t N, int32_t H, int32_t Dh,
                             const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                             int32_t dtype, float scale, void* stream) {
  Plan pl;
  int rc = make_plan(B, N, H, Dh, patterns, n_patterns, causal, dtype, scale, &pl);
  if (rc != DA_OK) return rc;
  if (!pl.bf16) return DA_ERR_DTYPE;
  if (pl.empty) return DA_OK;
  da::OnePassArgs a;
  memset(&a, 0, sizeof a);
  int64_t grid = 0;
  rc = onepass_geometry(pl, &a, &grid);
  if (rc != DA_OK) return rc;
  Plan chk = pl;  // no workspace
  chk.ws_bytes = 0;
  rc = check_buffers(chk, q, k, v, out, lse, nullptr, 0);
  if (rc != DA_OK) return rc;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = pl.B;
  a.N = pl.N;
  a.H = pl.H;
  a.np = pl.np;
  a.sl2 = pl.sl2;
  for (int i = 0; i < pl.np; ++i) a.pat[i] = pl.pat[i];
  const hipError_t e =
      da::launch_onepass(a, pl.causal, grid, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int dilated_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t N, int32_t H, int32_t Dh,
                             const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                             int32_t dtype, float scale, void* stream) {
  Plan pl;
  int rc = make_plan(B, N, H, Dh, patterns, n_patterns, causal, dtype, scale, &pl);
  if (rc != DA_OK || pl.empty) return rc;
  if (pl.ws_bytes > DA_NOALLOC_MAX_WORKSPACE_BYTES) return DA_ERR_WORKSPACE;
  rc = check_buffers(pl, q, k, v, out, lse, nullptr, 0, false);
  if (rc != DA_OK) return rc;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    rc = scratch_address(stream, &ws);
    if (rc != DA_OK) return rc;
    rc = check_buffers(pl, q, k, v, out, lse, ws, DA_NOALLOC_MAX_WORKSPACE_BYTES);
    if (rc != DA_OK) return rc;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = run_attention(pl, q, k, v, out, lse, ws, st);
  if (rc != DA_OK) return rc;
  return run_merge(pl, out, lse, ws, st);
}

int dilated_attn_fwd_qknorm(const void* xq, const void* xk, const void* v, const void* gain_q,
                            const void* bias_q, const void* gain_k, const void* bias_k,
                            float eps, void* out, float* lse, int64_t B, int64_t N, int32_t H,
                            int32_t Dh, int64_t row_stride, const da_pattern* patterns,
                            int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                            void* stream) {
  Plan pl;
  int rc = make_plan(B, N, H, Dh, patterns, n_patterns, causal, dtype, scale, &pl);
  if (rc != DA_OK) return rc;
  const void* gb[4] = {gain_q, bias_q, gain_k, bias_k};
  const void* outs[2] = {out, lse};
  const size_t ob[2] = {pl.tensor_bytes, pl.lse_bytes};
  rc = qkn_params_check(pl, gb, eps, outs, ob, 2);
  if (rc != DA_OK || pl.empty) return rc;
  int64_t rsi = 0;
  rc = qkn_row_stride(pl, row_stride, &rsi);
  if (rc != DA_OK) return rc;
  if (rsi == (int64_t)pl.H * DA_HEAD_DIM) {
    rc = check_buffers(pl, xq, xk, v, out, lse, nullptr, 0);
  } else {
    if (!xq || !xk || !v || !out || !lse) return DA_ERR_NULL;
    auto mis = [](const void* p, uintptr_t al) { return ((uintptr_t)p & (al - 1)) != 0; };
    if (mis(xq, 16) || mis(xk, 16) || mis(v, 16) || mis(out, 16) || mis(lse, 4))
      return DA_ERR_ALIGN;
    const int64_t es = pl.bf16 ? 2 : 4, rows = pl.B * pl.N;
    const size_t rb = (size_t)(rsi * es), row = (size_t)(pl.H * DA_HEAD_DIM * es);
    const Region ins[3] = {rows_of(xq, rows, rb, row), rows_of(xk, rows, rb, row),
                           rows_of(v, rows, rb, row)};
    const Region o[2] = {dense(out, pl.tensor_bytes), dense(lse, pl.lse_bytes)};
    for (const Region& x : o)
      for (const Region& y : ins)
        if (collide(x, y)) return DA_ERR_ALIAS;
    if (collide(o[0], o[1])) return DA_ERR_ALIAS;
  }
  if (rc != DA_OK) return rc;
  return run_attention(pl, xq, xk, v, out, lse, nullptr, reinterpret_cast<hipStream_t>(stream),
                       gb, eps, rsi);
}

int dilated_attn_bwd_qknorm_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                            const da_pattern* patterns, int32_t n_patterns,
                                            int32_t dtype, size_t* bytes) {
  if (!bytes) return DA_ERR_NULL;
  Plan pl;
  const int rc = make_plan(B, N, H, Dh, patterns, n_patterns, 1, dtype, 0.f, &pl);
  if (rc != DA_OK) return rc;
  if (pl.empty) {
    *bytes = 0;
    return DA_OK;
  }
  if (pl.np != 1 || pl.nw != 1) return DA_ERR_PATTERN;
  *bytes = qkn_bwd_ws_bytes(pl);
  return DA_OK;
}

int dilated_attn_bwd_qknorm(const void* xq, const void* xk, const void* v, const void* gain_q,
                            const void* bias_q, const void* gain_k, const void* bias_k,
                            float eps, const void* out, const float* lse, const void* dout,
                            void* dxq, void* dxk, void* dv, float* dparams, int64_t B, int64_t N,
                            int32_t H, int32_t Dh, int64_t row_stride, const da_pattern* patterns,
                            int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const void* gb[4] = {gain_q, bias_q, gain_k, bias_k};
  return bwd_common(DA_BWD_ALL, xq, xk, v, out, lse, dout, dxq, dxk, dv, B, N, H, Dh, patterns,
                    n_patterns, causal, dtype, scale, workspace, workspace_bytes, stream, gb, eps,
                    dparams, row_stride);
}

int dilated_attn_fwd_attention(const void* q, const void* k, const void* v, void* out, float* lse,
                               int64_t B, int64_t N, int32_t H, int32_t Dh,
                               const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                               int32_t dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return fwd_common(kAttention, q, k, v, out, lse, B, N, H, Dh, patterns, n_patterns, causal,
                    dtype, scale, workspace, workspace_bytes, stream);
}

int dilated_attn_fwd_merge(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t B, int64_t N, int32_t H, int32_t Dh,
                           const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                           int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return fwd_common(kMerge, q, k, v, out, lse, B, N, H, Dh, patterns, n_patterns, causal, dtype,
                    scale, workspace, workspace_bytes, stream);
}

int dilated_attn_bwd_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t Dh,
                                     const da_pattern* patterns, int32_t n_patterns,
                                     int32_t dtype, size_t* bytes) {
  if (!bytes) return DA_ERR_NULL;
  Plan pl;
  const int rc = make_plan(B, N, H, Dh, patterns, n_patterns, 1, dtype, 0.f, &pl);
  if (rc != DA_OK) return rc;
  *bytes = pl.empty ? 0 : pl.bwd_ws_bytes;
  return DA_OK;
}

int dilated_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t B,
                     int64_t N, int32_t H, int32_t Dh, const da_pattern* patterns,
                     int32_t n_patterns, int32_t causal, int32_t dtype, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(DA_BWD_ALL, q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Dh, patterns,
                    n_patterns, causal, dtype, scale, workspace, workspace_bytes, stream);
}

int dilated_attn_bwd_stages(int32_t stages, const void* q, const void* k, const void* v,
                            const void* out, const float* lse, const void* dout, void* dq,
                            void* dk, void* dv, int64_t B, int64_t N, int32_t H, int32_t Dh,
                            const da_pattern* patterns, int32_t n_patterns, int32_t causal,
                            int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return bwd_common(stages, q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Dh, patterns,
                    n_patterns, causal, dtype, scale, workspace, workspace_bytes, stream);
}

int dilated_attn_qk_norm_workspace_bytes(int64_t rows, size_t* bytes) {
  if (!bytes) return DA_ERR_NULL;
  if (rows < 0) return DA_ERR_SHAPE;
  *bytes = rows == 0 ? 0 : (size_t)(2 * da::qk_norm_blocks(rows) * 2 * kDh) * sizeof(float);
  return DA_OK;
}

int dilated_attn_qk_norm_fwd(const void* xq, const void* xk, const void* gain_q,
                             const void* bias_q, const void* gain_k, const void* bias_k, void* yq,
                             void* yk, int64_t rows, int32_t Dh, int32_t dtype, float eps,
                             void* stream) {
  int rc = qk_norm_check(rows, Dh, dtype, eps);
  if (rc != DA_OK || rows == 0) return rc;
  const void* ptrs[8] = {xq, xk, gain_q, bias_q, gain_k, bias_k, yq, yk};
  for (const void* p : ptrs) {
    if (!p) return DA_ERR_NULL;
    if (((uintptr_t)p & 15) != 0) return DA_ERR_ALIGN;
  }
  const size_t tb = (size_t)rows * kDh * (dtype == DA_BF16 ? 2 : 4);
  const size_t pb = (size_t)kDh * (dtype == DA_BF16 ? 2 : 4);
  const void* ins[6] = {xq, xk, gain_q, bias_q, gain_k, bias_k};
  const size_t isz[6] = {tb, tb, pb, pb, pb, pb};
  for (const void* o : {(const void*)yq, (const void*)yk})
    for (int j = 0; j < 6; ++j)
      if (overlaps(o, tb, ins[j], isz[j])) return DA_ERR_ALIAS;
  if (overlaps(yq, tb, yk, tb)) return DA_ERR_ALIAS;
  da::QkNormArgs a;
  memset(&a, 0, sizeof a);
  a.xq = xq;
  a.xk = xk;
  a.yq = yq;
  a.yk = yk;
  a.gq = gain_q;
  a.bq = bias_q;
  a.gk = gain_k;
  a.bk = bias_k;
  a.rows = rows;
  a.eps = eps;
  const hipError_t e =
      da::launch_qk_norm_fwd(a, dtype == DA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int dilated_attn_qk_norm_bwd(const void* xq, const void* xk, const void* dyq, const void* dyk,
                             const void* gain_q, const void* gain_k, void* dxq, void* dxk,
                             float* dparams, int64_t rows, int32_t Dh, int32_t dtype, float eps,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int rc = qk_norm_check(rows, Dh, dtype, eps);
  if (rc != DA_OK || rows == 0) return rc;
  const void* ptrs[8] = {xq, xk, dyq, dyk, gain_q, gain_k, dxq, dxk};
  for (const void* p : ptrs) {
    if (!p) return DA_ERR_NULL;
    if (((uintptr_t)p & 15) != 0) return DA_ERR_ALIGN;
  }
  if (!dparams) return DA_ERR_NULL;
  if (((uintptr_t)dparams & 3) != 0) return DA_ERR_ALIGN;
  size_t need = 0;
  dilated_attn_qk_norm_workspace_bytes(rows, &need);
  if (!workspace || workspace_bytes < need) return DA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return DA_ERR_ALIGN;
  const size_t tb = (size_t)rows * kDh * (dtype == DA_BF16 ? 2 : 4);
  const size_t pb = (size_t)kDh * (dtype == DA_BF16 ? 2 : 4);
  const size_t db = 4 * kDh * sizeof(float);
  const void* ins[6] = {xq, xk, dyq, dyk, gain_q, gain_k};
  const size_t isz[6] = {tb, tb, tb, tb, pb, pb};
  const void* outs[4] = {dxq, dxk, dparams, workspace};
  const size_t osz[4] = {tb, tb, db, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return DA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return DA_ERR_ALIAS;
  }
  da::QkNormArgs a;
  memset(&a, 0, sizeof a);
  a.xq = xq;
  a.xk = xk;
  a.dyq = dyq;
  a.dyk = dyk;
  a.dxq = dxq;
  a.dxk = dxk;
  a.gq = gain_q;
  a.gk = gain_k;
  a.partials = reinterpret_cast<float*>(workspace);
  a.dparams = dparams;
  a.rows = rows;
  a.eps = eps;
  const hipError_t e =
      da::launch_qk_norm_bwd(a, dtype == DA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int dilated_attn_gather_map(int64_t N, int32_t H, da_pattern pattern, int32_t h, int64_t* dev_out,
                            int64_t cap, int64_t* shape, void* stream) {
  PatDev p;
  int rc = map_pattern(N, H, pattern, h, &p);
  if (rc != DA_OK) return rc;
  if (shape) {
    shape[0] = p.nseg;
    shape[1] = p.lmax;
  }
  if (!dev_out) return shape ? DA_OK : DA_ERR_NULL;
  if (cap < p.nseg * p.lmax) return DA_ERR_ARG;
  if (((uintptr_t)dev_out & 7) != 0) return DA_ERR_ALIGN;
  const hipError_t e =
      da::launch_gather_map(p, h, dev_out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

int dilated_attn_coverage_map(int64_t N, int32_t H, da_pattern pattern, int32_t h,
                              int64_t* dev_out, int64_t cap, void* stream) {
  PatDev p;
  int rc = map_pattern(N, H, pattern, h, &p);
  if (rc != DA_OK) return rc;
  if (!dev_out) return DA_ERR_NULL;
  if (cap < N) return DA_ERR_ARG;
  if (((uintptr_t)dev_out & 7) != 0) return DA_ERR_ALIGN;
  const hipError_t e =
      da::launch_coverage_map(p, h, N, dev_out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

const char* dilated_attn_strerror(int code) {
  switch (code) {
    case DA_OK: return "success";
    case DA_ERR_NULL: return "a required pointer is NULL";
    case DA_ERR_SHAPE: return "invalid or unsupported shape (B, N, H, or N not a multiple of min(w, N))";
    case DA_ERR_PATTERN: return "invalid pattern list (count, w < 1, r < 1 or r > min(w, N))";
    case DA_ERR_DTYPE: return "unsupported dtype (DA_F32 or DA_BF16)";
    case DA_ERR_HEADDIM: return "unsupported head dimension (must be 64)";
    case DA_ERR_WORKSPACE: return "workspace missing or too small";
    case DA_ERR_ALIGN: return "misaligned pointer";
    case DA_ERR_ALIAS: return "an output or the workspace overlaps another buffer";
    case DA_ERR_ARG: return "invalid argument";
    case DA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

int dilated_attn_version(void) { return DA_VERSION; }

}  // extern "C"

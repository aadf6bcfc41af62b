// C ABI of the MoE layer: argument validation, workspace carving and the
// launch sequence.  Every check runs on the host before any HIP call, so a
// rejected call enqueues nothing.
#include "../../include/moe.h"
#include "bwd.h"
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

// Scratch of moe_layer_fwd_noalloc: a fixed array that every device the
// library runs on holds from the code object's load until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up per device (scratch_on_device) and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::kRouteTok;
using moe::kTileM;

struct Dims {
  int64_t T;
  int d, d_ff, n, k, K_s, esize;
};

moe_status check_problem(const moe_problem* p, Dims* out) {
  if (!p) return MOE_ERR_NULL;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (p->T < 1 || p->d < 32 || p->d % 32 != 0 || p->d_ff < 32 || p->d_ff % 32 != 0)
    return MOE_ERR_SHAPE;
  if (p->N < 1 || p->m < 1 || p->K < 1 || p->K_s < 0) return MOE_ERR_SHAPE;
  const int64_t n = (int64_t)p->m * p->N;
  const int64_t k = (int64_t)p->m * p->K - p->K_s;
  if (n > MOE_MAX_EXPERTS || k < 1 || k > n || k > MOE_MAX_TOPK) return MOE_ERR_SHAPE;
  if (p->T * k >= (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  // Kernels index rows with 32-bit element offsets: every activation tensor
  // (u, x_perm, y_perm, h and the SwiGLU intermediates) stays below 2^31
  // elements.
  const int64_t big = (int64_t)1 << 31;
  if (p->T * k * p->d >= big || p->T * k * p->d_ff >= big ||
      p->T * (int64_t)p->K_s * p->d_ff >= big)
    return MOE_ERR_SHAPE;
  if ((int64_t)p->K_s * p->d_ff > INT32_MAX / 2) return MOE_ERR_SHAPE;
  // ... and so does every weight matrix: one expert's [d_ff][d] and the
  // shared experts' dense view [K_s*d_ff][d].
  if ((int64_t)p->d * p->d_ff >= big || (int64_t)p->K_s * p->d_ff * p->d >= big)
    return MOE_ERR_SHAPE;
  out->T = p->T;
  out->d = p->d;
  out->d_ff = p->d_ff;
  out->n = (int)n;
  out->k = (int)k;
  out->K_s = p->K_s;
  out->esize = p->dtype == MOE_BF16 ? 2 : 4;
  return MOE_OK;
}

bool aligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Workspace regions, each 256-byte aligned.
struct Layout {
  size_t blk_cnt, blk_P, blk_base, lrank, offsets, perm_token, slot_of;
  size_t t_row0, t_rows, t_off, t_count, lg;
  size_t hbuf, ybuf, hsbuf, sbuf;
  size_t total;
  // kept for the backward (MOE_SAVE_FOR_BACKWARD): pre-activations W1 x | W3 x
  // of the routed rows [T*k][2 d_ff] and of the shared experts [T][2 K_s d_ff]
  size_t pre, pres;
  size_t lgs;  // and the router's logits [T][n rounded up to 8] fp32 (batches the
               // small-batch router does not cover: that one keeps them in lg)
  size_t total_train;
  int max_tiles;
  size_t hcap;  // elements of hbuf
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(const Dims& d) {
  Layout L{};
  const size_t B = (size_t)((d.T + kRouteTok - 1) / kRouteTok);
  const size_t R = (size_t)d.T * d.k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  const size_t ldn = (size_t)moe::blk_ld(d.n);
  L.blk_cnt = take(B * ldn * 4);
  L.blk_P = take(B * ldn * 4);
  L.blk_base = take(B * ldn * 4);
  L.lrank = take(R * 4);
  L.offsets = take((size_t)(d.n + 1) * 4);
  L.perm_token = take(R * 4);
  L.slot_of = take(R * 4);
  L.max_tiles = (int)(R / kTileM) + MOE_MAX_EXPERTS;
  L.t_row0 = take((size_t)L.max_tiles * 4);
  L.t_rows = take((size_t)L.max_tiles * 4);
  L.t_off = take((size_t)(MOE_MAX_EXPERTS + 1) * 4);
  L.t_count = take(4 + 64);  // the count, then 16 claim counters at int 16
  L.lg = take((size_t)(d.T < moe::kSmallBatch ? d.T : moe::kSmallBatch) * d.n * 4);
  const size_t hs_el = (size_t)d.T * d.K_s * d.d_ff;
  L.hcap = R * d.d_ff > hs_el ? R * d.d_ff : hs_el;
  L.hbuf = take(L.hcap * d.esize);
  L.ybuf = take(R * d.d * d.esize);
  L.hsbuf = take(hs_el * d.esize);
  L.sbuf = take((size_t)d.T * d.d * d.esize);
  L.total = o;
  L.pre = take(R * 2 * d.d_ff * 2);
  L.pres = take(hs_el * 2 * 2);
  L.lgs = take((size_t)d.T * ((d.n + 7) & ~7) * 4);
  L.total_train = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// The tile count's 256-byte region also holds the 16 claim counters of the
// two grouped-GEMM launches (ints 16 .. 31).
moe::TileList tiles_of(void* ws, const Layout& L) {
  return moe::TileList{at<int32_t>(ws, L.t_row0), at<int32_t>(ws, L.t_rows),
                       at<int32_t>(ws, L.t_off),  at<int32_t>(ws, L.t_count),
                       L.max_tiles,               at<int32_t>(ws, L.t_count) + 16};
}

// Last HIP error an entry point hit on this host thread.
thread_local hipError_t g_last_hip = hipSuccess;

// Few rows per group (the decode regime): the weight-streaming kernels.
// The layer also needs few tokens, since the shared experts' weights are
// streamed once per 32 tokens there.
bool use_skinny(bool packed, int64_t rows, int n_groups) {
  return packed && rows <= 16 * (int64_t)n_groups;
}

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_ERR_HIP;
}

#define MOE_TRY(expr)                                  \
  do {                                                 \
    const moe_status st_ = hip_status(expr);           \
    if (st_ != MOE_OK) return st_;                     \
  } while (0)

moe_status check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Backward-pass workspace: the grouping of the forward (rebuilt from
// topk_idx), per-row gates and the rows of u and dh in grouped order, the
// SwiGLU backward's intermediates (q = dh W2
// per row, da, db, gate * hid, gate-gradient partials), the input gradients
// of the routed and shared experts, the router's logits and softmax
// gradient, and per-chunk partial sums of the centroid gradient.
struct BwdLayout {
  size_t blk_cnt, blk_base, lrank, offsets, perm_token, slot_of;
  size_t t_row0, t_rows, t_off, t_count;
  size_t gperm, xp, dhp, q, da, db, gh, dgp, dxp;
  size_t qs, das, dbs, ghs, dxs;
  size_t lg, dl, slabs;
  size_t wctr;  // the weight-gradient kernel's work queues
  size_t total;
  int max_tiles, ldl, ldgp, kchunk, G;
};

BwdLayout bwd_layout(const Dims& d) {
  BwdLayout L{};
  const size_t B = (size_t)((d.T + kRouteTok - 1) / kRouteTok);
  const size_t R = (size_t)d.T * d.k;
  const size_t fs = (size_t)d.K_s * d.d_ff;
  L.ldl = (d.n + 7) & ~7;
  L.ldgp = 2 * ((d.d_ff + moe::kBgTile - 1) / moe::kBgTile);
  // token chunks of the centroid gradient: at least 256 tokens, at most 64 chunks
  const int64_t per = (d.T + 63) / 64;
  L.kchunk = (int)(per > 256 ? (per + 63) & ~(int64_t)63 : 256);
  L.G = (int)((d.T + L.kchunk - 1) / L.kchunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  const size_t ldn = (size_t)moe::blk_ld(d.n);
  L.blk_cnt = take(B * ldn * 4);
  L.blk_base = take(B * ldn * 4);
  L.lrank = take(R * 4);
  L.offsets = take((size_t)(d.n + 1) * 4);
  L.perm_token = take(R * 4);
  L.slot_of = take(R * 4);
  L.max_tiles = (int)(R / kTileM) + MOE_MAX_EXPERTS;
  L.t_row0 = take((size_t)L.max_tiles * 4);
  L.t_rows = take((size_t)L.max_tiles * 4);
  L.t_off = take((size_t)(MOE_MAX_EXPERTS + 1) * 4);
  L.t_count = take(4 + 64);  // the count, then 16 claim counters at int 16
  L.wctr = take(moe::kWgQueues * 4);
  L.gperm = take(R * 4);
  L.xp = take(R * d.d * 2);
  L.dhp = take(R * d.d * 2);
  L.q = take(R * d.d_ff * 2);
  L.da = take(R * d.d_ff * 2);
  L.db = take(R * d.d_ff * 2);
  L.gh = take(R * d.d_ff * 2);
  L.dgp = take(R * L.ldgp * 4);
  L.dxp = take(R * d.d * 2);
  L.qs = take((size_t)d.T * fs * 2);
  L.das = take((size_t)d.T * fs * 2);
  L.dbs = take((size_t)d.T * fs * 2);
  L.ghs = take((size_t)d.T * fs * 2);
  L.dxs = take((size_t)d.T * d.d * 2);
  L.lg = take((size_t)d.T * L.ldl * 4);
  L.dl = take((size_t)d.T * L.ldl * 2);
  L.slabs = take((size_t)L.G * d.n * d.d * 4);
  L.total = o;
  return L;
}

// Device address of `scratch` on the device that owns `stream` (the
// calling thread's current device for the null stream; a stream of another
// device is refused, since the address is looked up with that device
// current), found once per device with hipGetSymbolAddress and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

moe_status scratch_on_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    if ((int)sdev != dev) return MOE_ERR_UNSUPPORTED;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!ptr || !aligned(ptr)) return MOE_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_problem* p) {
  Dims d;
  if (check_problem(p, &d) != MOE_OK) return 0;
  return layout(d).total;
}

size_t moe_train_workspace_bytes(const moe_problem* p) {
  Dims d;
  if (check_problem(p, &d) != MOE_OK || p->dtype != MOE_BF16) return 0;
  return layout(d).total_train;
}

const char* moe_status_str(moe_status s) {
  // A C caller may pass any int; reading an out-of-range value as the enum
  // type is undefined in C++, so the bits are taken as an int.
  int v = 0;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "problem sizes out of range";
    case MOE_ERR_DTYPE: return "unknown element type";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "request not supported by this build";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int moe_last_hip_error(const char** text) {
  if (text) *text = hipGetErrorString(g_last_hip);
  return (int)g_last_hip;
}

moe_status moe_route(const moe_problem* p, const void* u, const void* centroids,
                     int32_t* topk_idx, float* topk_gate, int32_t* counts, float* f, float* P,
                     void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!u || !centroids || !topk_idx || !topk_gate || !counts || !f || !P) return MOE_ERR_NULL;
  if (!aligned(u) || !aligned(centroids) || !aligned(topk_idx) || !aligned(topk_gate) ||
      !aligned(counts) || !aligned(f) || !aligned(P))
    return MOE_ERR_ALIGN;
  const Layout L = layout(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(moe::launch_route(p->dtype, u, centroids, d.T, d.d, d.n, d.k, topk_idx, topk_gate,
                            at<int32_t>(ws, L.blk_cnt), at<float>(ws, L.blk_P),
                            at<int32_t>(ws, L.lrank), s));
  MOE_TRY(moe::launch_scan(at<int32_t>(ws, L.blk_cnt), at<float>(ws, L.blk_P), d.T, d.n, d.k,
                           counts, f, P, at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.blk_base),
                           nullptr, s));
  return MOE_OK;
}

moe_status moe_permute(const moe_problem* p, const void* u, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* perm_token, int32_t* slot_of, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!topk_idx || !offsets || !perm_token || !slot_of || (x_perm && !u)) return MOE_ERR_NULL;
  if (!aligned(topk_idx) || !aligned(offsets) || !aligned(perm_token) || !aligned(slot_of) ||
      (x_perm && (!aligned(x_perm) || !aligned(u))))
    return MOE_ERR_ALIGN;
  const Layout L = layout(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(moe::launch_hist(topk_idx, d.T, d.n, d.k, at<int32_t>(ws, L.blk_cnt),
                           at<int32_t>(ws, L.lrank), s));
  MOE_TRY(moe::launch_scan(at<int32_t>(ws, L.blk_cnt), nullptr, d.T, d.n, d.k, nullptr, nullptr,
                           nullptr, offsets, at<int32_t>(ws, L.blk_base), nullptr, s));
  MOE_TRY(moe::launch_scatter(topk_idx, at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.blk_base),
                              d.T, d.n, d.k, perm_token, slot_of, u, x_perm, d.d * d.esize, s));
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_problem* p, int32_t n_groups, int64_t rows,
                           const int32_t* offsets, const void* x, const void* w1,
                           const void* w3, const void* w2, int32_t d_ff_group, int flags,
                           void* y, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (flags & ~MOE_PACKED_WEIGHTS) return MOE_ERR_SHAPE;
  const bool packed = (flags & MOE_PACKED_WEIGHTS) != 0;
  if (packed && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (n_groups < 1 || n_groups > MOE_MAX_EXPERTS || rows < 1 || d_ff_group < 32 ||
      d_ff_group % 32 != 0 || (int64_t)d_ff_group * d.d >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (!offsets || !x || !w1 || !w3 || !w2 || !y) return MOE_ERR_NULL;
  if (!aligned(offsets) || !aligned(x) || !aligned(w1) || !aligned(w3) || !aligned(w2) ||
      !aligned(y))
    return MOE_ERR_ALIGN;
  const Layout L = layout(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  if (rows > d.T * d.k || (size_t)rows * d_ff_group > L.hcap) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::TileList tl = tiles_of(ws, L);
  const bool skinny = use_skinny(packed, rows, n_groups);
  if (p->dtype == MOE_BF16 && !skinny)
    MOE_TRY(moe::launch_tiles(offsets, n_groups, rows, tl, s));
  moe::FfnArgs a{};
  a.dtype = p->dtype;
  a.x = x;
  a.x_rows = nullptr;
  a.ldx = d.d;
  a.w1 = w1;
  a.w3 = w3;
  a.w2 = w2;
  a.n_groups = n_groups;
  a.d = d.d;
  a.d_ff_g = d_ff_group;
  a.rows = rows;
  a.offsets = offsets;
  a.tiles = &tl;
  a.hbuf = at<char>(ws, L.hbuf);
  a.y = y;
  a.packed = packed;
  if (skinny) {
    MOE_TRY(moe::launch_ffn_skinny(&a, 1, true, s));
    MOE_TRY(moe::launch_ffn_skinny(&a, 1, false, s));
  } else {
    MOE_TRY(moe::launch_grouped_ffn(a, s));
  }
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_problem* p, int64_t rows, int32_t K, const void* src,
                            void* dst, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows < 32 || rows % 32 != 0 || K < 32 || K % 32 != 0) return MOE_ERR_SHAPE;
  if (rows * (int64_t)K >= ((int64_t)1 << 33)) return MOE_ERR_SHAPE;
  if (!src || !dst) return MOE_ERR_NULL;
  if (!aligned(src) || !aligned(dst)) return MOE_ERR_ALIGN;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const int64_t nb = rows * K * 2;
  if (s0 < d0 + nb && d0 < s0 + nb) return MOE_ERR_SHAPE;  // overlapping buffers
  MOE_TRY(moe::launch_pack(src, dst, rows, K, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_combine(const moe_problem* p, const void* residual, const void* shared_out,
                       const void* y_perm, const int32_t* slot_of, const float* topk_gate,
                       void* h, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!y_perm || !slot_of || !topk_gate || !h) return MOE_ERR_NULL;
  if (!aligned(y_perm) || !aligned(slot_of) || !aligned(topk_gate) || !aligned(h) ||
      (residual && !aligned(residual)) || (shared_out && !aligned(shared_out)))
    return MOE_ERR_ALIGN;
  MOE_TRY(moe::launch_combine(p->dtype, residual, shared_out, y_perm, slot_of, topk_gate, h, d.T,
                              d.d, d.k, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_balance_loss(const moe_problem* p, const float* f, const float* P, float alpha,
                            float* loss, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!f || !P || !loss) return MOE_ERR_NULL;
  if (!aligned(f) || !aligned(P) || !aligned(loss)) return MOE_ERR_ALIGN;
  MOE_TRY(moe::launch_balance_loss(f, P, d.n, alpha, loss, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_fwd(const moe_problem* p, const void* u, const void* centroids,
                         const void* w1, const void* w3, const void* w2, const void* ws1,
                         const void* ws3, const void* ws2, void* h, int32_t* topk_idx,
                         float* topk_gate, int32_t* counts, float* f, float* P, int flags,
                         void* ws, size_t ws_bytes, void* stream) {
  return moe_layer_fwd_marked(p, u, centroids, w1, w3, w2, ws1, ws3, ws2, h, topk_idx, topk_gate,
                              counts, f, P, flags, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_fwd_noalloc(const moe_problem* p, const void* u, const void* centroids,
                                 const void* w1, const void* w3, const void* w2,
                                 const void* ws1, const void* ws3, const void* ws2, void* h,
                                 int32_t* topk_idx, float* topk_gate, int32_t* counts, float* f,
                                 float* P, int flags, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  // the backward would need the scratch's address as its fwd_ws
  if (flags & MOE_SAVE_FOR_BACKWARD) return MOE_ERR_UNSUPPORTED;
  if (layout(d).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_on_device(static_cast<hipStream_t>(stream), &ws)) != MOE_OK) return st;
  return moe_layer_fwd_marked(p, u, centroids, w1, w3, w2, ws1, ws3, ws2, h, topk_idx, topk_gate,
                              counts, f, P, flags, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream,
                              nullptr);
}

int moe_layer_kernels(const moe_problem* p, int flags, const char** names, int max_names) {
  Dims d;
  if (check_problem(p, &d) != MOE_OK) return -1;
  const bool shared = d.K_s > 0 && !(flags & MOE_NO_SHARED);
  const bool tiled = p->dtype == MOE_BF16;
  const char* seq[10];
  int c = 0;
  if (moe::route_small(p->dtype, d.T)) {
    seq[c++] = "logits";
    seq[c++] = "route_group";
  } else if (moe::group_in_one_pass(d.T, d.n)) {
    seq[c++] = "route";
    seq[c++] = "group";
  } else {
    seq[c++] = "route";
    seq[c++] = "scan";
    seq[c++] = "scatter";
  }
  // bf16: one launch per projection covers routed and shared experts; fp32
  // runs the two groups back to back inside the same mark.
  seq[c++] = tiled ? "up_swiglu" : "up_swiglu_f32";
  seq[c++] = tiled ? "down" : "down_f32";
  (void)shared;
  seq[c++] = "combine";
  for (int i = 0; names && i < c && i < max_names; ++i) names[i] = seq[i];
  return c;
}

moe_status moe_layer_fwd_marked(const moe_problem* p, const void* u, const void* centroids,
                                const void* w1, const void* w3, const void* w2,
                                const void* ws1, const void* ws3, const void* ws2, void* h,
                                int32_t* topk_idx, float* topk_gate, int32_t* counts, float* f,
                                float* P, int flags, void* ws, size_t ws_bytes, void* stream,
                                void* const* marks) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (flags & ~(MOE_NO_RESIDUAL | MOE_NO_SHARED | MOE_PACKED_WEIGHTS | MOE_SAVE_FOR_BACKWARD))
    return MOE_ERR_SHAPE;
  const bool shared = d.K_s > 0 && !(flags & MOE_NO_SHARED);
  const bool packed = (flags & MOE_PACKED_WEIGHTS) != 0;
  const bool save = (flags & MOE_SAVE_FOR_BACKWARD) != 0;
  if ((packed || save) && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!u || !centroids || !w1 || !w3 || !w2 || !h || !topk_idx || !topk_gate || !counts || !f ||
      !P)
    return MOE_ERR_NULL;
  if (shared && (!ws1 || !ws3 || !ws2)) return MOE_ERR_NULL;
  if (!aligned(u) || !aligned(centroids) || !aligned(w1) || !aligned(w3) || !aligned(w2) ||
      !aligned(h) || !aligned(topk_idx) || !aligned(topk_gate) || !aligned(counts) ||
      !aligned(f) || !aligned(P))
    return MOE_ERR_ALIGN;
  if (shared && (!aligned(ws1) || !aligned(ws3) || !aligned(ws2))) return MOE_ERR_ALIGN;
  const Layout L = layout(d);
  if ((st = check_ws(L, ws, ws_bytes)) != MOE_OK) return st;
  if (save && ws_bytes < L.total_train) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::TileList tl = tiles_of(ws, L);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm_token = at<int32_t>(ws, L.perm_token);
  int32_t* slot_of = at<int32_t>(ws, L.slot_of);
  // Few rows per expert: the weight-streaming FFN (which keeps no
  // pre-activations, so a forward saving for the backward tiles instead).
  const bool skinny = !save && d.T <= 64 && use_skinny(packed, d.T * d.k, d.n);
  int mark_i = 0;
  auto mark = [&]() -> hipError_t {
    if (!marks) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(marks[mark_i++]), s);
  };
  MOE_TRY(mark());

  if (moe::route_small(p->dtype, d.T)) {
    // Small batch: logits spread over the GPU, then one workgroup routes and
    // groups the whole batch.
    float* lg = at<float>(ws, L.lg);
    MOE_TRY(moe::launch_logits_small(u, centroids, d.T, d.d, d.n, lg, s));
    MOE_TRY(mark());
    // (the weight-streaming FFN reads no tile list)
    MOE_TRY(moe::launch_route_small(lg, d.T, d.n, d.k, topk_idx, topk_gate, counts, f, P, offsets,
                                    perm_token, slot_of, skinny ? nullptr : &tl, s));
    MOE_TRY(mark());
  } else {
    MOE_TRY(moe::launch_route(p->dtype, u, centroids, d.T, d.d, d.n, d.k, topk_idx, topk_gate,
                              at<int32_t>(ws, L.blk_cnt), at<float>(ws, L.blk_P),
                              at<int32_t>(ws, L.lrank), s, save ? at<float>(ws, L.lgs) : nullptr,
                              (d.n + 7) & ~7));
    MOE_TRY(mark());
    if (moe::group_in_one_pass(d.T, d.n)) {
      MOE_TRY(moe::launch_group(at<int32_t>(ws, L.blk_cnt), at<float>(ws, L.blk_P), d.T, d.n,
                                d.k, topk_idx, at<int32_t>(ws, L.lrank), counts, f, P, offsets,
                                perm_token, slot_of, &tl, s));
      MOE_TRY(mark());
    } else {
      MOE_TRY(moe::launch_scan(at<int32_t>(ws, L.blk_cnt), at<float>(ws, L.blk_P), d.T, d.n,
                               d.k, counts, f, P, offsets, at<int32_t>(ws, L.blk_base), &tl, s));
      MOE_TRY(mark());
      MOE_TRY(moe::launch_scatter(topk_idx, at<int32_t>(ws, L.lrank),
                                  at<int32_t>(ws, L.blk_base), d.T, d.n, d.k, perm_token,
                                  slot_of, nullptr, nullptr, 0, s));
      MOE_TRY(mark());
    }
  }
  // Routed experts (rows gathered from u through perm_token) and the shared
  // experts (one dense SwiGLU of width K_s*d_ff over all tokens) go through
  // the same launches so their tiles fill the GPU together.
  moe::FfnArgs segs[2] = {};
  moe::FfnArgs& a = segs[0];
  a.dtype = p->dtype;
  a.x = u;
  a.x_rows = perm_token;
  a.ldx = d.d;
  a.w1 = w1;
  a.w3 = w3;
  a.w2 = w2;
  a.n_groups = d.n;
  a.d = d.d;
  a.d_ff_g = d.d_ff;
  a.rows = d.T * d.k;
  a.offsets = offsets;
  a.tiles = &tl;
  a.hbuf = at<char>(ws, L.hbuf);
  a.y = at<char>(ws, L.ybuf);
  a.packed = packed;
  a.preact = save ? at<char>(ws, L.pre) : nullptr;
  void* sbuf = nullptr;
  int nseg = 1;
  if (shared) {
    moe::FfnArgs& b = segs[1];
    b.dtype = p->dtype;
    b.x = u;
    b.x_rows = nullptr;
    b.ldx = d.d;
    b.w1 = ws1;
    b.w3 = ws3;
    b.w2 = ws2;
    b.n_groups = 1;
    b.d = d.d;
    b.d_ff_g = d.K_s * d.d_ff;
    b.rows = d.T;
    b.offsets = nullptr;
    b.tiles = nullptr;
    b.hbuf = at<char>(ws, L.hsbuf);
    b.y = at<char>(ws, L.sbuf);
    b.packed = packed;
    b.preact = save ? at<char>(ws, L.pres) : nullptr;
    sbuf = b.y;
    nseg = 2;
  }
  if (skinny) {
    MOE_TRY(moe::launch_ffn_skinny(segs, nseg, true, s));
    MOE_TRY(mark());
    MOE_TRY(moe::launch_ffn_skinny(segs, nseg, false, s));
  } else {
    MOE_TRY(moe::launch_ffn_up(segs, nseg, s));
    MOE_TRY(mark());
    MOE_TRY(moe::launch_ffn_down(segs, nseg, s));
  }
  MOE_TRY(mark());
  MOE_TRY(moe::launch_combine(p->dtype, (flags & MOE_NO_RESIDUAL) ? nullptr : u, sbuf,
                              at<char>(ws, L.ybuf), slot_of, topk_gate, h, d.T, d.d, d.k, s));
  MOE_TRY(mark());
  return MOE_OK;
}

}  // extern "C"

extern "C" {

size_t moe_bwd_workspace_bytes(const moe_problem* p) {
  Dims d;
  if (check_problem(p, &d) != MOE_OK || p->dtype != MOE_BF16) return 0;
  return bwd_layout(d).total;
}

int moe_layer_bwd_kernels(const moe_problem* p, int flags, const char** names, int max_names) {
  Dims d;
  if (check_problem(p, &d) != MOE_OK) return -1;
  static const char* recompute[] = {"hist", "scan",        "scatter", "gather", "logits",
                                    "q",    "ab_swiglu",   "dx",      "softmax_bwd", "du",
                                    "wgrad", "dcent_sum"};
  // with the forward's saved grouping and pre-activations
  static const char* saved[] = {"gather", "q", "swiglu_bwd", "dx", "softmax_bwd",
                                "du", "wgrad", "dcent_sum"};
  const bool sv = (flags & MOE_SAVE_FOR_BACKWARD) != 0;
  const char** seq = sv ? saved : recompute;
  const int c = sv ? 8 : 12;
  for (int i = 0; names && i < c && i < max_names; ++i) names[i] = seq[i];
  return c;
}

moe_status moe_layer_bwd_marked(const moe_problem* p, const void* u, const void* centroids,
                                const void* w1, const void* w3, const void* w2,
                                const void* ws1, const void* ws3, const void* ws2,
                                const int32_t* topk_idx, const float* topk_gate, const float* f,
                                const void* fwd_ws, const void* dh, float alpha, float* du,
                                float* dcentroids, float* dw1, float* dw3, float* dw2,
                                float* dws1, float* dws3, float* dws2, int flags, void* ws,
                                size_t ws_bytes, void* stream, void* const* marks) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (flags & ~(MOE_NO_RESIDUAL | MOE_NO_SHARED | MOE_PACKED_WEIGHTS | MOE_SAVE_FOR_BACKWARD))
    return MOE_ERR_SHAPE;
  if (p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // the forward's saved grouping and pre-activations: flag and pointer together
  const bool saved = (flags & MOE_SAVE_FOR_BACKWARD) != 0;
  if (saved != (fwd_ws != nullptr)) return saved ? MOE_ERR_NULL : MOE_ERR_SHAPE;
  if (fwd_ws && !aligned(fwd_ws)) return MOE_ERR_ALIGN;
  const bool shared = d.K_s > 0 && !(flags & MOE_NO_SHARED);
  // packed weights: the layout of moe_pack_weights, read by the same kernels
  const bool packed = (flags & MOE_PACKED_WEIGHTS) != 0;
  if (!u || !centroids || !w1 || !w3 || !w2 || !topk_idx || !topk_gate || !f || !dh || !du ||
      !dcentroids || !dw1 || !dw3 || !dw2)
    return MOE_ERR_NULL;
  if (shared && (!ws1 || !ws3 || !ws2 || !dws1 || !dws3 || !dws2)) return MOE_ERR_NULL;
  if (!aligned(u) || !aligned(centroids) || !aligned(w1) || !aligned(w3) || !aligned(w2) ||
      !aligned(topk_idx) || !aligned(topk_gate) || !aligned(f) || !aligned(dh) || !aligned(du) ||
      !aligned(dcentroids) || !aligned(dw1) || !aligned(dw3) || !aligned(dw2))
    return MOE_ERR_ALIGN;
  if (shared && (!aligned(ws1) || !aligned(ws3) || !aligned(ws2) || !aligned(dws1) ||
                 !aligned(dws3) || !aligned(dws2)))
    return MOE_ERR_ALIGN;
  const BwdLayout L = bwd_layout(d);
  // Sizes the backward's kernels address with 32-bit offsets, checked here so
  // that nothing is enqueued on error: the softmax gradient [T][ldl] bf16 is
  // read with byte offsets, and every gradient output (fp32 [d_ff][d] per
  // expert, the shared experts' [K_s*d_ff][d], the centroids' [n][d] per
  // token chunk) through a buffer resource of fewer than 2^31 bytes.
  const int64_t out_lim = moe::kBwdOutBytes;
  if (d.T * L.ldl >= ((int64_t)1 << 31) || (int64_t)d.d_ff * d.d * 4 >= out_lim ||
      (int64_t)d.K_s * d.d_ff * d.d * 4 >= out_lim || (int64_t)d.n * d.d * 4 >= out_lim)
    return MOE_ERR_SHAPE;
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(ws)) return MOE_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int mark_i = 0;
  auto mark = [&]() -> hipError_t {
    if (!marks) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(marks[mark_i++]), s);
  };
  const int fs = d.K_s * d.d_ff;
  // The grouping: the forward's (in its workspace) when it saved for the
  // backward, else rebuilt from topk_idx (stable counting sort by expert).
  void* gws = saved ? const_cast<void*>(fwd_ws) : ws;
  const Layout FL = layout(d);
  int32_t* offsets = at<int32_t>(gws, saved ? FL.offsets : L.offsets);
  int32_t* perm = at<int32_t>(gws, saved ? FL.perm_token : L.perm_token);
  int32_t* slot_of = at<int32_t>(gws, saved ? FL.slot_of : L.slot_of);
  const moe::TileList tl =
      saved ? tiles_of(gws, FL)
            : moe::TileList{at<int32_t>(ws, L.t_row0), at<int32_t>(ws, L.t_rows),
                            at<int32_t>(ws, L.t_off), at<int32_t>(ws, L.t_count), L.max_tiles};
  MOE_TRY(mark());
  if (!saved) {
    MOE_TRY(moe::launch_hist(topk_idx, d.T, d.n, d.k, at<int32_t>(ws, L.blk_cnt),
                             at<int32_t>(ws, L.lrank), s));
    MOE_TRY(mark());
    MOE_TRY(moe::launch_scan(at<int32_t>(ws, L.blk_cnt), nullptr, d.T, d.n, d.k, nullptr,
                             nullptr, nullptr, offsets, at<int32_t>(ws, L.blk_base), &tl, s));
    MOE_TRY(mark());
    MOE_TRY(moe::launch_scatter(topk_idx, at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.blk_base),
                                d.T, d.n, d.k, perm, slot_of, nullptr, nullptr, 0, s));
    MOE_TRY(mark());
  }
  float* gperm = at<float>(ws, L.gperm);
  uint16_t* xp = at<uint16_t>(ws, L.xp);
  uint16_t* dhp = at<uint16_t>(ws, L.dhp);
  // (also zeroes the weight-gradient launch's work queues)
  int32_t* wctr = at<int32_t>(ws, L.wctr);
  MOE_TRY(moe::launch_gather_rows(slot_of, topk_gate, u, dh, d.T, d.k, d.d, xp, dhp, gperm, wctr,
                                  s));
  MOE_TRY(mark());

  // Router logits again (fp32 accumulation of bf16 products).
  auto rows_seg = [&](moe::BgSeg& g) {
    g.t_row0 = tl.row0;
    g.t_rows = tl.rows;
    g.t_off = tl.off;
    g.t_count = tl.count;
    g.n_groups = d.n;
    g.max_tiles = tl.max_tiles;
  };
  // The router's logits: kept by a forward that saved for the backward
  // (its small-batch router keeps them at pitch n), else computed again.
  const float* lg = at<float>(ws, L.lg);
  int ldlg = L.ldl;
  if (saved) {
    const bool small = moe::route_small(p->dtype, d.T);
    lg = at<float>(gws, small ? FL.lg : FL.lgs);
    ldlg = small ? d.n : L.ldl;
  } else {
    moe::BgSeg g{};
    g.A[0] = u;
    g.lda = d.d;
    g.B[0] = centroids;
    g.ldb = d.d;
    g.npass = 1;
    g.N = d.n;
    g.K = d.d;
    g.rows = d.T;
    g.C = at<float>(ws, L.lg);
    g.ldc = L.ldl;
    MOE_TRY(moe::launch_bg(moe::BG_LOGITS, &g, 1, s));
    MOE_TRY(mark());
  }

  // q = dh W2 for every grouped row (ungated), and for the shared experts.
  uint16_t* q = at<uint16_t>(ws, L.q);
  uint16_t* qs = at<uint16_t>(ws, L.qs);
  {
    moe::BgSeg g[2] = {};
    rows_seg(g[0]);
    g[0].A[0] = dhp;
    g[0].lda = d.d;
    g[0].B[0] = w2;
    g[0].ldb = d.d_ff;
    g[0].b_gstride = (int64_t)d.d * d.d_ff;
    g[0].npass = 1;
    g[0].N = d.d_ff;
    g[0].K = d.d;
    g[0].bk_lim = d.d;
    g[0].b_lim = d.d_ff;
    g[0].C = q;
    g[0].ldc = d.d_ff;
    if (shared) {
      g[1].A[0] = dh;
      g[1].lda = d.d;
      g[1].B[0] = ws2;
      g[1].ldb = fs;
      g[1].npass = 1;
      g[1].N = fs;
      g[1].K = d.d;
      g[1].bk_lim = d.d;
      g[1].b_lim = fs;
      g[1].rows = d.T;
      g[1].C = qs;
      g[1].ldc = fs;
    }
    MOE_TRY(moe::launch_bg(packed ? moe::BG_PROJ_PACKED : moe::BG_PROJ, g, shared ? 2 : 1, s));
  }
  MOE_TRY(mark());

  // SwiGLU backward: from the forward's kept pre-activations, or with a and b
  // computed again (and the SwiGLU backward in the GEMM's epilogue).
  uint16_t* da = at<uint16_t>(ws, L.da);
  uint16_t* db = at<uint16_t>(ws, L.db);
  uint16_t* gh = at<uint16_t>(ws, L.gh);
  uint16_t* das = at<uint16_t>(ws, L.das);
  uint16_t* dbs = at<uint16_t>(ws, L.dbs);
  uint16_t* ghs = at<uint16_t>(ws, L.ghs);
  float* dgp = at<float>(ws, L.dgp);
  if (saved) {
    MOE_TRY(moe::launch_swiglu_bwd(q, at<uint16_t>(gws, FL.pre), gperm, offsets + d.n,
                                   d.T * d.k, d.d_ff, da, db, gh, dgp, L.ldgp, s));
    if (shared)
      MOE_TRY(moe::launch_swiglu_bwd(qs, at<uint16_t>(gws, FL.pres), nullptr, nullptr, d.T, fs,
                                     das, dbs, ghs, nullptr, 0, s));
  } else {
    {
      moe::BgSeg g[2] = {};
      rows_seg(g[0]);
      g[0].A[0] = xp;
      g[0].lda = d.d;
      g[0].B[0] = w1;
      g[0].B2 = w3;
      g[0].ldb = d.d;
      g[0].b_gstride = (int64_t)d.d_ff * d.d;
      g[0].npass = 1;
      g[0].N = d.d_ff;
      g[0].K = d.d;
      g[0].ldc = d.d_ff;
      g[0].q = q;
      g[0].gate = gperm;
      g[0].da = da;
      g[0].db = db;
      g[0].gh = gh;
      g[0].dgp = dgp;
      g[0].ldgp = L.ldgp;
      if (shared) {
        g[1].A[0] = u;
        g[1].lda = d.d;
        g[1].B[0] = ws1;
        g[1].B2 = ws3;
        g[1].ldb = d.d;
        g[1].npass = 1;
        g[1].N = fs;
        g[1].K = d.d;
        g[1].rows = d.T;
        g[1].ldc = fs;
        g[1].q = qs;
        g[1].da = das;
        g[1].db = dbs;
        g[1].gh = ghs;
      }
      MOE_TRY(moe::launch_bg(packed ? moe::BG_SWIGLU_PACKED : moe::BG_SWIGLU, g, shared ? 2 : 1,
                             s));
    }
  }
  MOE_TRY(mark());

  // Input gradients of the experts: dx = da W1 + db W3.
  uint16_t* dxp = at<uint16_t>(ws, L.dxp);
  uint16_t* dxs = at<uint16_t>(ws, L.dxs);
  {
    moe::BgSeg g[2] = {};
    rows_seg(g[0]);
    g[0].A[0] = da;
    g[0].A[1] = db;
    g[0].lda = d.d_ff;
    g[0].B[0] = w1;
    g[0].B[1] = w3;
    g[0].ldb = d.d;
    g[0].b_gstride = (int64_t)d.d_ff * d.d;
    g[0].npass = 2;
    g[0].N = d.d;
    g[0].K = d.d_ff;
    g[0].bk_lim = d.d_ff;
    g[0].b_lim = d.d;
    g[0].C = dxp;
    g[0].ldc = d.d;
    if (shared) {
      g[1].A[0] = das;
      g[1].A[1] = dbs;
      g[1].lda = fs;
      g[1].B[0] = ws1;
      g[1].B[1] = ws3;
      g[1].ldb = d.d;
      g[1].npass = 2;
      g[1].N = d.d;
      g[1].K = fs;
      g[1].bk_lim = fs;
      g[1].b_lim = d.d;
      g[1].rows = d.T;
      g[1].C = dxs;
      g[1].ldc = d.d;
    }
    MOE_TRY(moe::launch_bg(packed ? moe::BG_PROJ_PACKED : moe::BG_PROJ, g, shared ? 2 : 1, s));
  }
  MOE_TRY(mark());

  // Softmax backward with the gate gradients and the balance term.
  uint16_t* dl = at<uint16_t>(ws, L.dl);
  MOE_TRY(moe::launch_softmax_bwd(lg, ldlg, L.ldl, d.T, d.n, d.k, topk_idx, slot_of, dgp, L.ldgp, f,
                                  alpha, dl, s));
  MOE_TRY(mark());

  // du = dl E + residual + shared + sum of the kept experts' dx.
  {
    moe::BgSeg g{};
    g.A[0] = dl;
    g.lda = L.ldl;
    g.B[0] = centroids;
    g.ldb = d.d;
    g.npass = 1;
    g.N = d.d;
    g.K = L.ldl;
    g.bk_lim = d.n;
    g.b_lim = d.d;
    g.rows = d.T;
    g.C = du;
    g.ldc = d.d;
    g.resid = (flags & MOE_NO_RESIDUAL) ? nullptr : dh;
    g.dxs = shared ? dxs : nullptr;
    g.dxp = dxp;
    g.slot_of = slot_of;
    g.k = d.k;
    MOE_TRY(moe::launch_bg(moe::BG_DU, &g, 1, s));
  }
  MOE_TRY(mark());

  // Weight gradients (one output per expert, reduced over its rows) and the
  // centroid gradient's per-chunk partial sums, in one launch.
  float* slabs = at<float>(ws, L.slabs);
  auto wseg = [&](moe::BgSeg& x, const void* A, int64_t lda, const void* B, int64_t ldb, int M,
                  int N, const int32_t* koff, int kchunk, int K, int G, float* C, int64_t ldc) {
    x.A[0] = A;
    x.lda = lda;
    x.a_lim = (int)lda;
    x.B[0] = B;
    x.ldb = ldb;
    x.b_lim = (int)ldb;
    x.npass = 1;
    x.M = M;
    x.N = N;
    x.koff = koff;
    x.kchunk = kchunk;
    x.K = K;
    x.G = G;
    x.C = C;
    x.ldc = ldc;
    x.c_gstride = (int64_t)M * N;
    x.c_stream = 1;
  };
  {
    moe::BgSeg g[7] = {};
    int c = 0;
    // The shared experts' tiles reduce over all T tokens (the routed ones
    // over one expert's rows): dealt first, so they do not end the launch.
    if (shared) {
      wseg(g[c++], das, fs, u, d.d, fs, d.d, nullptr, (int)d.T, (int)d.T, 1, dws1, d.d);
      wseg(g[c++], dbs, fs, u, d.d, fs, d.d, nullptr, (int)d.T, (int)d.T, 1, dws3, d.d);
      wseg(g[c++], dh, d.d, ghs, fs, d.d, fs, nullptr, (int)d.T, (int)d.T, 1, dws2, fs);
    }
    // dW1 = da^T x, dW3 = db^T x, dW2 = (g dh)^T hid per expert
    wseg(g[c++], da, d.d_ff, xp, d.d, d.d_ff, d.d, offsets, 0, 0, d.n, dw1, d.d);
    wseg(g[c++], db, d.d_ff, xp, d.d, d.d_ff, d.d, offsets, 0, 0, d.n, dw3, d.d);
    wseg(g[c++], dhp, d.d, gh, d.d_ff, d.d, d.d_ff, offsets, 0, 0, d.n, dw2, d.d_ff);
    // dE = dl^T u over token chunks: M = n, N = d
    wseg(g[c++], dl, L.ldl, u, d.d, d.n, d.d, nullptr, L.kchunk, (int)d.T, L.G, slabs, d.d);
    g[c - 1].c_stream = 0;  // the slab sum reads these partials next
    MOE_TRY(moe::launch_bg(moe::BG_WGRAD, g, c, s, wctr));
  }
  MOE_TRY(mark());
  MOE_TRY(moe::launch_slab_sum(slabs, L.G, (int64_t)d.n * d.d, dcentroids, s));
  MOE_TRY(mark());
  return MOE_OK;
}

moe_status moe_layer_bwd(const moe_problem* p, const void* u, const void* centroids,
                         const void* w1, const void* w3, const void* w2, const void* ws1,
                         const void* ws3, const void* ws2, const int32_t* topk_idx,
                         const float* topk_gate, const float* f, const void* fwd_ws,
                         const void* dh, float alpha, float* du, float* dcentroids, float* dw1,
                         float* dw3, float* dw2, float* dws1, float* dws3, float* dws2, int flags,
                         void* ws, size_t ws_bytes, void* stream) {
  return moe_layer_bwd_marked(p, u, centroids, w1, w3, w2, ws1, ws3, ws2, topk_idx, topk_gate, f,
                              fwd_ws, dh, alpha, du, dcentroids, dw1, dw3, dw2, dws1, dws3, dws2,
                              flags, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"

// C ABI of the MoE layer: argument validation, workspace layout and the
// launch sequence router -> gate/up GEMM -> down GEMM -> combine.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_mi355x.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
// done counter at [0]; expert e's cursor at 64 + CURSOR_STRIDE * e and token
// block b's K-split counter at 64 + CURSOR_STRIDE * (256 + b), one cache line
// each so that atomics on different counters do not serialize
constexpr int kCursor0 = 64;
constexpr int kTbDone0 = kCursor0 + CURSOR_STRIDE * 256;
constexpr int kHeaderInts = kTbDone0 + CURSOR_STRIDE * ROUTE_MAX_TB;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t topk_id, topk_w, rel_pos, counts, offsets, n_tiles, tiles, expert_rows, part, xq, hq, y, fold, pair_row, total;
  int max_tiles;
};

constexpr int kWide64Rows = 48;

int max_tiles_for(int P, int E, int mt) { return (P + mt - 1) / mt + (E < P ? E : P); }

Layout layout(int T, int d, int I, int E, int k) {
  Layout L;
  const size_t P = (size_t)T * k;
  L.max_tiles = max_tiles_for((int)P, E, MT_SMALL);
  size_t o = up(kHeaderInts * sizeof(int));
  L.topk_id = o; o = up(o + P * 4);
  L.topk_w = o; o = up(o + P * 4);
  L.rel_pos = o; o = up(o + P * 4);
  L.counts = o; o = up(o + (size_t)E * 4);
  L.offsets = o; o = up(o + (size_t)(E + 1) * 4);
  L.n_tiles = o; o = up(o + 4);
  L.tiles = o; o = up(o + (size_t)L.max_tiles * 8);
  L.expert_rows = o; o = up(o + (size_t)E * T * 4);
  L.part = o; o = up(o + route_partial_bytes(T, E));
  L.xq = o; o = up(o + (size_t)T * mx6_row_bytes(d / 32));
  L.hq = o; o = up(o + P * mx6_row_bytes(I / 32));
  L.y = o; o = up(o + P * d * 4);
  L.fold = o; o = up(o + (size_t)T * ((d + 63) / 64) * 4);
  L.pair_row = o; o = up(o + P * 4);
  L.total = o;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int T, int d, int I, int E, int k) {
  if (T < 0 || d <= 0 || I <= 0 || (d % 32) || (I % 32)) return MOE_ERR_BAD_SHAPE;
  if (E < 1 || E > 256 || k < 1 || k > 8 || k > E) return MOE_ERR_BAD_SHAPE;
  const long long big = (long long)T * (k > E ? k : E);
  if (big >= (long long)INT_MAX) return MOE_ERR_BAD_SHAPE;
  if ((long long)d * 2 * I >= (long long)INT_MAX * 16) return MOE_ERR_BAD_SHAPE;
  // operands are addressed with 32-bit byte offsets (MX6x3 activations:
  // 80 bytes per 32 elements)
  const long long w = d > I ? d : I;
  if ((long long)T * k * mx6_row_bytes((int)(w / 32)) >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long long)E * I * d >= (1ll << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_UNSUPPORTED;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct LayerArgs {
  const void* x; const void* router_w; const float* router_b;
  const uint8_t* w13c; const uint8_t* w13s; const float* b13;
  const uint8_t* w2c; const uint8_t* w2s; const float* b2;
  int T, d, I, E, k; float clamp;
  int terms = 3;  // FP6 terms of the expert GEMMs' activations: 3 (exact path), 2 or 1 (fast mode)
  int alt = 0;    // 1: the variant gate/up layout and activation
  int packed = 0; // 1: expert weights in the packed layout of moe_pack_weights
};

size_t packed_scale_bytes(int E, int N, int K) { return (size_t)E * N * 4 * (size_t)(((K >> 5) + 3) >> 2); }

int check_layer(const LayerArgs& a, const void* out) {
  int st = check_shape(a.T, a.d, a.I, a.E, a.k);
  if (st) return st;
  if (!(a.clamp > 0.0f)) return MOE_ERR_BAD_SHAPE;
  if (a.T == 0) return MOE_OK;  // no-op: nothing is read or written
  if (!a.x || !a.router_w || !a.router_b || !a.w13c || !a.w13s || !a.b13 || !a.w2c || !a.w2s || !a.b2)
    return MOE_ERR_NULL_PTR;
  if (!aligned(a.x, 16) || !aligned(a.router_w, 16) || !aligned(a.w13c, 16) || !aligned(a.w2c, 16) ||
      !aligned(a.w13s, 16) || !aligned(a.w2s, 16) ||
      !aligned(a.router_b, 4) || !aligned(a.b13, 4) || !aligned(a.b2, 4))
    return MOE_ERR_MISALIGNED;
  // the packed layout pairs weight rows and keeps an even number of
  // 32-element blocks per row: d and I multiples of 64
  if (a.packed && ((a.d % 64) || (a.I % 64))) return MOE_ERR_UNSUPPORTED;
  if (out) {
    if (!aligned(out, 16)) return MOE_ERR_MISALIGNED;
    const size_t no = (size_t)a.T * a.d * 2;
    const size_t E = a.E, d = a.d, I = a.I;
    const size_t s13 = a.packed ? packed_scale_bytes(a.E, 2 * a.I, a.d) : E * 2 * I * d / 32;
    const size_t s2 = a.packed ? packed_scale_bytes(a.E, a.d, a.I) : E * d * I / 32;
    if (overlap(out, no, a.x, no) || overlap(out, no, a.router_w, E * d * 2) ||
        overlap(out, no, a.router_b, E * 4) || overlap(out, no, a.w13c, E * 2 * I * d / 2) ||
        overlap(out, no, a.w13s, s13) || overlap(out, no, a.b13, E * 2 * I * 4) ||
        overlap(out, no, a.w2c, E * d * I / 2) || overlap(out, no, a.w2s, s2) ||
        overlap(out, no, a.b2, E * d * 4))
      return MOE_ERR_ALIAS;
  }
  return MOE_OK;
}

// library-owned workspaces, one per device
struct OwnedWs { void* p = nullptr; size_t n = 0; };
std::mutex g_mu;
OwnedWs g_ws[64];

int owned_workspace(size_t need, hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  OwnedWs& w = g_ws[dev];
  if (w.n < need) {
    if (w.p) {
      if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
      (void)hipFree(w.p);
      w.p = nullptr;
      w.n = 0;
    }
    void* p = nullptr;
    const size_t n = need + need / 8;  // headroom against small growths
    if (hipMalloc(&p, n) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERR_NOMEM;
    }
    if (launch_zero_ints((int*)p, kHeaderInts, s)) return MOE_ERR_HIP;
    w.p = p;
    w.n = n;
  }
  *out = w.p;
  return MOE_OK;
}

// optional per-kernel event timing
struct Timing {
  int mask = 0;  // bit i: time kernel kind i
  std::vector<hipEvent_t> pool;
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> pending;
  double ms[5] = {0, 0, 0, 0, 0};
  int n[5] = {0, 0, 0, 0, 0};
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
} g_t;

// ext: the events are handed to the one launch inside the region, which
// records them when its kernel starts and ends; otherwise they are recorded
// on the stream around the region (and include the dispatch).
struct Timed {
  int kind; hipStream_t s; bool ext; hipEvent_t a = nullptr, b = nullptr;
  Timed(int k, hipStream_t st, bool ext_ = false) : kind(k), s(st), ext(ext_) {
    if (!((g_t.mask >> k) & 1)) return;
    a = g_t.get(); b = g_t.get();
    if (a && b && !ext) (void)hipEventRecord(a, s);
  }
  LaunchEvents events() const { return ext && a && b ? LaunchEvents{a, b} : LaunchEvents{}; }
  ~Timed() {
    if (!a || !b) return;
    if (!ext) (void)hipEventRecord(b, s);
    g_t.pending.push_back({kind, a, b});
  }
};

// Enqueues the layer on `s` using workspace `ws` (layout L).  Optional
// debug outputs replace the workspace copies of the routing results.
int run_layer(const LayerArgs& a, const Layout& L, uint8_t* ws, void* out, float* out_f32,
              int32_t* topk_id, float* topk_w, int32_t* counts, bool route_only, hipStream_t s,
              const uint16_t* resid_in = nullptr, uint16_t* resid_out = nullptr,
              uint16_t* norm_out = nullptr, float eps = 0.f) {
  const int P = a.T * a.k;
  // 16-row decode tiles up to 32 rows per expert on average: they read an
  // expert's weights once per tile, and still beat the 64-row tiles there
  // (20b shapes: 160 tokens 189 vs 245 us, 256 tokens 241 vs 284 us; from
  // 36 rows per expert on they lose)
  const bool small_m = (long long)P <= 32LL * a.E;
  // 128-row tiles above the decode sizes whenever both projections copy
  // their scale bytes in pairs (K/32 even): measured faster than 64-row
  // tiles from 33 rows per expert on, partly filled tiles included (20b
  // shapes: 264 tokens 233 vs 256 us, 384 tokens 242 vs 296 us)
  const bool wide = !small_m && (a.d / 32) % 2 == 0 && (a.I / 32) % 2 == 0;
  // up to kWide64Rows rows per expert on average, 64-row wide tiles with
  // three weight stages: twice the weight bytes in flight and half the idle
  // MFMA rows (20b shapes: 288 tokens 177 vs 208 us, 384 tokens 186 vs 211
  // us; even from 56 rows on, where experts start to need a second 64-row
  // tile that reads the weights again)
  const bool wide64 = wide && (long long)P <= (long long)kWide64Rows * a.E;
  const int mode = small_m ? GEMM_DECODE : wide64 ? GEMM_WIDE64 : wide ? GEMM_WIDE : GEMM_PREFILL;
  // decode sizes above 16 rows per expert: 32-row tiles (two row blocks),
  // which read an expert's weights once
  const bool mb2 = small_m && (long long)P > 16LL * a.E;
  const int mt = small_m ? (mb2 ? MT_SMALL2 : MT_SMALL) : (wide && !wide64) ? MT_WIDE : MT_LARGE;
  const int max_tiles = max_tiles_for(P, a.E, mt);
  int* hdr = (int*)ws;

  RouteParams rp;
  rp.x = (const uint16_t*)a.x;
  rp.router_w = (const uint16_t*)a.router_w;
  rp.router_b = a.router_b;
  rp.T = a.T; rp.d = a.d; rp.E = a.E; rp.k = a.k; rp.mt = mt;
  rp.topk_id = topk_id ? topk_id : (int*)(ws + L.topk_id);
  rp.topk_w = topk_w ? topk_w : (float*)(ws + L.topk_w);
  rp.rel_pos = (int*)(ws + L.rel_pos);
  rp.expert_rows = (int*)(ws + L.expert_rows);
  rp.cursor = hdr + kCursor0;
  rp.done = hdr;
  rp.tb_done = hdr + kTbDone0;
  rp.part = (float*)(ws + L.part);
  rp.xq = route_only ? nullptr : ws + L.xq;
  rp.n_tb = rp.ks = 0;  // set by launch_route
  rp.counts = counts ? counts : (int*)(ws + L.counts);
  rp.offsets = (int*)(ws + L.offsets);
  rp.n_tiles = (int*)(ws + L.n_tiles);
  rp.tiles = (int2*)(ws + L.tiles);
  // decode-sized single layers fold the combine into the down GEMM (the
  // stack's combine also adds the residual and stays a kernel of its own)
  const bool fold = small_m && !mb2 && !route_only && resid_out == nullptr && out != nullptr;
  rp.fold_cnt = fold ? (int*)(ws + L.fold) : nullptr;
  rp.n_fold = a.T * ((a.d + 63) / 64);
  {
    Timed tm(0, s);
    if (launch_route(rp, s)) return MOE_ERR_HIP;
  }
  if (route_only) return MOE_OK;

  GemmParams gp;
  gp.n_tiles = rp.n_tiles;
  gp.tiles = rp.tiles;
  gp.counts = rp.counts;
  gp.offsets = rp.offsets;
  gp.expert_rows = rp.expert_rows;
  gp.T = a.T; gp.k = a.k;
  gp.a = ws + L.xq;
  gp.b_codes = a.w13c; gp.b_scales = a.w13s; gp.bias = a.b13;
  gp.N = 2 * a.I; gp.K = a.d; gp.I = a.I; gp.E = a.E;
  gp.clamp = a.clamp;
  gp.terms = a.terms;
  gp.alt = a.alt;
  gp.packed = a.packed;
  gp.hq = ws + L.hq;
  gp.y = nullptr;
  gp.fold_cnt = nullptr;
  gp.mb = mb2 ? 2 : 1;
  gp.pair_row = fold ? (int*)(ws + L.pair_row) : nullptr;
  gp.topk_w = rp.topk_w;
  gp.out = (uint16_t*)out;
  gp.out_f32 = out_f32;
  {
    Timed tm(1, s, true);
    if (launch_gemm_gateup(gp, max_tiles, mode, s, tm.events())) return MOE_ERR_HIP;
  }

  gp.a = gp.hq;
  gp.b_codes = a.w2c; gp.b_scales = a.w2s; gp.bias = a.b2;
  gp.N = a.d; gp.K = a.I;
  gp.hq = nullptr;
  gp.y = (float*)(ws + L.y);
  gp.alt = 0;  // (the down projection has no gate/up rows)
  gp.fold_cnt = rp.fold_cnt;
  {
    Timed tm(2, s, true);
    if (launch_gemm_down(gp, max_tiles, mode, s, tm.events())) return MOE_ERR_HIP;
  }

  if (fold) return MOE_OK;

  CombineParams cp;
  cp.y = gp.y;
  cp.topk_id = rp.topk_id;
  cp.topk_w = rp.topk_w;
  cp.rel_pos = rp.rel_pos;
  cp.offsets = rp.offsets;
  cp.T = a.T; cp.d = a.d; cp.k = a.k;
  cp.out = (uint16_t*)out;
  cp.out_f32 = out_f32;
  cp.resid_in = resid_in;
  cp.resid_out = resid_out;
  cp.norm_out = norm_out;
  cp.eps = eps;
  {
    Timed tm(3, s);
    if (launch_combine(cp, s)) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: its scratch is this file-scope device array,
// one copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` only names the symbol; its device address on each GPU
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[64] = {};

int scratch_for_current_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return MOE_ERR_HIP;
    }
    g_scratch_ptr[dev] = (uint8_t*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_version(void) { return MOE_MI355X_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "the current device is not gfx950";
    case MOE_ERR_MISALIGNED: return "a pointer breaks the alignment rules";
    case MOE_ERR_NOMEM: return "workspace allocation failed";
    case MOE_ERR_HIP: return "a HIP launch or runtime call failed";
    case MOE_ERR_ALIAS: return "the output overlaps an input";
    case MOE_ERR_WORKSPACE: return "the workspace is too small";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(int T, int d, int I, int E, int k) {
  if (check_shape(T, d, I, E, k)) return 0;
  return layout(T, d, I, E, k).total;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_ERR_NULL_PTR;
  if (!aligned(ws, kAlign)) return MOE_ERR_MISALIGNED;
  if (ws_bytes < kHeaderInts * sizeof(int)) return MOE_ERR_WORKSPACE;
  if (int st = check_device()) return st;
  return launch_zero_ints((int*)ws, kHeaderInts, (hipStream_t)stream) ? MOE_ERR_HIP : MOE_OK;
}

int moe_layer_forward_ws(const void* x, const void* router_w, const float* router_b,
                         const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2, int T, int d,
                         int I, int E, int k, float clamp, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  if (int st = check_layer(a, out)) return st;
  if (T == 0) return MOE_OK;
  if (!out || !ws) return MOE_ERR_NULL_PTR;
  if (!aligned(ws, kAlign)) return MOE_ERR_MISALIGNED;
  const Layout L = layout(T, d, I, E, k);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (int st = check_device()) return st;
  return run_layer(a, L, (uint8_t*)ws, out, nullptr, nullptr, nullptr, nullptr, false, (hipStream_t)stream);
}

static int forward_owned(const LayerArgs& a, void* out, void* stream) {
  if (int st = check_layer(a, out)) return st;
  if (a.T == 0) return MOE_OK;
  if (!out) return MOE_ERR_NULL_PTR;
  if (int st = check_device()) return st;
  const Layout L = layout(a.T, a.d, a.I, a.E, a.k);
  void* ws = nullptr;
  if (int st = owned_workspace(L.total, (hipStream_t)stream, &ws)) return st;
  return run_layer(a, L, (uint8_t*)ws, out, nullptr, nullptr, nullptr, nullptr, false, (hipStream_t)stream);
}

static int forward_dbg(const LayerArgs& a, void* out, float* out_f32, int32_t* topk_id, float* topk_w,
                       int32_t* counts, void* stream) {
  if (int st = check_layer(a, out)) return st;
  if (a.T == 0) return MOE_OK;
  if (!topk_id || !topk_w || !counts) return MOE_ERR_NULL_PTR;
  if (!aligned(topk_id, 4) || !aligned(topk_w, 4) || !aligned(counts, 4) || (out_f32 && !aligned(out_f32, 16)))
    return MOE_ERR_MISALIGNED;
  if (int st = check_device()) return st;
  const Layout L = layout(a.T, a.d, a.I, a.E, a.k);
  void* ws = nullptr;
  if (int st = owned_workspace(L.total, (hipStream_t)stream, &ws)) return st;
  return run_layer(a, L, (uint8_t*)ws, out, out_f32, topk_id, topk_w, counts, false, (hipStream_t)stream);
}

int moe_layer_forward(const void* x, const void* router_w, const float* router_b, const uint8_t* w13_codes,
                      const uint8_t* w13_scales, const float* b13, const uint8_t* w2_codes,
                      const uint8_t* w2_scales, const float* b2, int T, int d, int I, int E, int k, float clamp,
                      void* out, void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  return forward_owned(a, out, stream);
}

int moe_layer_forward_noalloc(const void* x, const void* router_w, const float* router_b,
                              const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                              const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2, int T, int d, int I,
                              int E, int k, float clamp, void* out, void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  if (int st = check_layer(a, out)) return st;
  if (T == 0) return MOE_OK;
  if (!out) return MOE_ERR_NULL_PTR;
  const Layout L = layout(T, d, I, E, k);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (int st = check_device()) return st;
  uint8_t* ws = nullptr;
  if (int st = scratch_for_current_device(&ws)) return st;
  hipStream_t s = (hipStream_t)stream;
  // the counters the kernels expect at zero, cleared by a kernel (not a
  // memset) so that the call can be captured into a graph; the rest of the
  // scratch is written before it is read within the call
  if (launch_zero_ints((int*)ws, kHeaderInts, s)) return MOE_ERR_HIP;
  return run_layer(a, L, ws, out, nullptr, nullptr, nullptr, nullptr, false, s);
}

int moe_layer_forward_dbg(const void* x, const void* router_w, const float* router_b, const uint8_t* w13_codes,
                          const uint8_t* w13_scales, const float* b13, const uint8_t* w2_codes,
                          const uint8_t* w2_scales, const float* b2, int T, int d, int I, int E, int k,
                          float clamp, void* out, float* out_f32, int32_t* topk_id, float* topk_w,
                          int32_t* counts, void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  return forward_dbg(a, out, out_f32, topk_id, topk_w, counts, stream);
}

int moe_layer_forward_ex(const void* x, const void* router_w, const float* router_b, const uint8_t* w13_codes,
                         const uint8_t* w13_scales, const float* b13, const uint8_t* w2_codes,
                         const uint8_t* w2_scales, const float* b2, int T, int d, int I, int E, int k, float clamp,
                         int flags, void* out, float* out_f32, int32_t* topk_id, float* topk_w, int32_t* counts,
                         void* stream) {
  if (flags & ~(MOE_LAYER_MXFP6 | MOE_LAYER_ALT_ACT | MOE_LAYER_PACKED | MOE_LAYER_MX6X2)) return MOE_ERR_BAD_SHAPE;
  if ((flags & MOE_LAYER_MXFP6) && (flags & MOE_LAYER_MX6X2)) return MOE_ERR_BAD_SHAPE;
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  a.terms = (flags & MOE_LAYER_MXFP6) ? 1 : (flags & MOE_LAYER_MX6X2) ? 2 : 3;
  a.alt = (flags & MOE_LAYER_ALT_ACT) ? 1 : 0;
  a.packed = (flags & MOE_LAYER_PACKED) ? 1 : 0;
  const bool any = topk_id || topk_w || counts, all = topk_id && topk_w && counts;
  if (any && !all) return MOE_ERR_NULL_PTR;
  if (!all && !out_f32) return forward_owned(a, out, stream);
  if (!all) return MOE_ERR_NULL_PTR;  // (the fp32 output comes with the routing outputs)
  return forward_dbg(a, out, out_f32, topk_id, topk_w, counts, stream);
}

int moe_layer_forward_mx6(const void* x, const void* router_w, const float* router_b, const uint8_t* w13_codes,
                          const uint8_t* w13_scales, const float* b13, const uint8_t* w2_codes,
                          const uint8_t* w2_scales, const float* b2, int T, int d, int I, int E, int k,
                          float clamp, void* out, void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  a.terms = 1;
  return forward_owned(a, out, stream);
}

int moe_layer_forward_mx6_dbg(const void* x, const void* router_w, const float* router_b,
                              const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                              const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2, int T, int d,
                              int I, int E, int k, float clamp, void* out, float* out_f32, int32_t* topk_id,
                              float* topk_w, int32_t* counts, void* stream) {
  LayerArgs a{x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d, I, E, k, clamp};
  a.terms = 1;
  return forward_dbg(a, out, out_f32, topk_id, topk_w, counts, stream);
}

int moe_route(const void* x, const void* router_w, const float* router_b, int T, int d, int E, int k,
              int32_t* topk_id, float* topk_w, int32_t* counts, void* stream) {
  if (int st = check_shape(T, d, 32, E, k)) return st;
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !router_b || !topk_id || !topk_w || !counts) return MOE_ERR_NULL_PTR;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(router_b, 4) || !aligned(topk_id, 4) ||
      !aligned(topk_w, 4) || !aligned(counts, 4))
    return MOE_ERR_MISALIGNED;
  if (T == 0) return MOE_OK;
  if (int st = check_device()) return st;
  const Layout L = layout(T, d, 32, E, k);
  void* ws = nullptr;
  if (int st = owned_workspace(L.total, (hipStream_t)stream, &ws)) return st;
  LayerArgs a{x, router_w, router_b, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, T, d, 32, E, k, 1.0f};
  return run_layer(a, L, (uint8_t*)ws, nullptr, nullptr, topk_id, topk_w, counts, true, (hipStream_t)stream);
}

int moe_rmsnorm(const void* x, void* out, int T, int d, float eps, void* stream) {
  if (T < 0 || d <= 0 || (d % 32) || !(eps >= 0.0f)) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !out) return MOE_ERR_NULL_PTR;
  if (!aligned(x, 16) || !aligned(out, 16)) return MOE_ERR_MISALIGNED;
  if (T == 0) return MOE_OK;
  if (int st = check_device()) return st;
  return launch_rmsnorm((const uint16_t*)x, (uint16_t*)out, T, d, eps, (hipStream_t)stream) ? MOE_ERR_HIP : MOE_OK;
}

int moe_rmsnorm_residual(const void* x, const void* y_bf16, const float* y_f32, void* x_out, void* n_out, int T,
                         int d, float eps, void* stream) {
  if (T < 0 || d <= 0 || (d % 32) || !(eps >= 0.0f)) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !x_out || (!y_bf16 == !y_f32)) return MOE_ERR_NULL_PTR;
  const void* y = y_f32 ? (const void*)y_f32 : y_bf16;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(x_out, 16) || (n_out && !aligned(n_out, 16)))
    return MOE_ERR_MISALIGNED;
  const size_t nb = (size_t)T * d * 2, ny = (size_t)T * d * (y_f32 ? 4 : 2);
  if ((x_out != x && overlap(x_out, nb, x, nb)) || overlap(x_out, nb, y, ny)) return MOE_ERR_ALIAS;
  if (n_out && (overlap(n_out, nb, x, nb) || overlap(n_out, nb, y, ny) || overlap(n_out, nb, x_out, nb)))
    return MOE_ERR_ALIAS;
  if (int st = check_device()) return st;
  return launch_residual_rmsnorm((const uint16_t*)x, y, y_f32 != nullptr, (uint16_t*)x_out, (uint16_t*)n_out, T, d,
                                 eps, (hipStream_t)stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

int moe_attn_rope(const void* x, void* out, int n, int H, int D, int pos0, float theta, void* stream) {
  if (n < 0 || H < 0 || D < 2 || D > 256 || (D & 1) || pos0 < 0 || (long long)pos0 + n >= (1ll << 31) ||
      !(theta > 1.0f) || theta == INFINITY)
    return MOE_ERR_BAD_SHAPE;
  if (n == 0 || H == 0) return MOE_OK;
  if (!x || !out) return MOE_ERR_NULL_PTR;
  if (!aligned(x, 16) || !aligned(out, 16)) return MOE_ERR_MISALIGNED;
  const size_t nb = (size_t)n * H * D * 2;
  if (out != x && overlap(out, nb, x, nb)) return MOE_ERR_ALIAS;
  if (int st = check_device()) return st;
  return launch_rope((const uint16_t*)x, (uint16_t*)out, n, H, D, pos0, theta, (hipStream_t)stream) ? MOE_ERR_HIP
                                                                                                      : MOE_OK;
}

int moe_attn_forward(const void* q, const void* k, const void* v, const float* sinks, void* out, int B, int Tq,
                     int S, int q_pos0, int Hq, int Hkv, int D, int window, void* stream) {
  if (B < 0 || Tq < 0 || S < 1 || q_pos0 < 0 || (long long)q_pos0 + Tq > S || Hq < 1 || Hkv < 1 || window < 0)
    return MOE_ERR_BAD_SHAPE;
  if (D != 64 || Hq % Hkv || B > 65535 || Hkv > 65535) return MOE_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return MOE_ERR_UNSUPPORTED;
  const size_t nq = (size_t)B * Tq * Hq * D * 2, nk = (size_t)B * S * Hkv * D * 2;
  if (nq / 2 >= (1ull << 40) || nk / 2 >= (1ull << 40)) return MOE_ERR_UNSUPPORTED;
  if (B == 0 || Tq == 0) return MOE_OK;
  if (!q || !k || !v || !sinks || !out) return MOE_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(sinks, 4))
    return MOE_ERR_MISALIGNED;
  if (overlap(out, nq, q, nq) || overlap(out, nq, k, nk) || overlap(out, nq, v, nk) ||
      overlap(out, nq, sinks, (size_t)Hq * 4))
    return MOE_ERR_ALIAS;
  if (int st = check_device()) return st;
  AttnParams p{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks, (uint16_t*)out,
               B, Tq, S, q_pos0, Hq, Hkv, window, (float)(1.4426950408889634 / sqrt((double)D))};
  return launch_attention(p, (hipStream_t)stream) ? MOE_ERR_HIP : MOE_OK;
}

static int stack_forward(const void* x0, int n_layers, const void* const* router_w, const float* const* router_b,
                         const uint8_t* const* w13_codes, const uint8_t* const* w13_scales, const float* const* b13,
                         const uint8_t* const* w2_codes, const uint8_t* const* w2_scales, const float* const* b2,
                         int T, int d, int I, int E, int k, float clamp, float eps, int flags, void* out,
                         void* stream) {
  if (n_layers < 1 || (flags & ~(MOE_LAYER_ALT_ACT | MOE_LAYER_PACKED))) return MOE_ERR_BAD_SHAPE;
  if (!x0 || !out || !router_w || !router_b || !w13_codes || !w13_scales || !b13 || !w2_codes || !w2_scales || !b2)
    return MOE_ERR_NULL_PTR;
  if (!(eps >= 0.0f)) return MOE_ERR_BAD_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    LayerArgs a{x0, router_w[l], router_b[l], w13_codes[l], w13_scales[l], b13[l], w2_codes[l], w2_scales[l],
                b2[l], T, d, I, E, k, clamp};
    a.alt = (flags & MOE_LAYER_ALT_ACT) ? 1 : 0;
    a.packed = (flags & MOE_LAYER_PACKED) ? 1 : 0;
    if (int st = check_layer(a, out)) return st;
  }
  if (T == 0) return MOE_OK;
  if (int st = check_device()) return st;
  const Layout L = layout(T, d, I, E, k);
  const size_t act = up((size_t)T * d * 2);
  void* wsv = nullptr;
  if (int st = owned_workspace(L.total + 2 * act, (hipStream_t)stream, &wsv)) return st;
  uint8_t* ws = (uint8_t*)wsv;
  uint16_t* norm = (uint16_t*)(ws + L.total);
  uint16_t* spare = (uint16_t*)(ws + L.total + act);
  hipStream_t s = (hipStream_t)stream;
  if (launch_rmsnorm((const uint16_t*)x0, norm, T, d, eps, s)) return MOE_ERR_HIP;
  // ping-pong the residual stream so that the last layer writes `out`
  uint16_t* bufs[2] = {(uint16_t*)out, spare};
  int cur = (n_layers % 2 == 1) ? 0 : 1;
  const uint16_t* resid = (const uint16_t*)x0;
  for (int l = 0; l < n_layers; ++l) {
    LayerArgs a{norm, router_w[l], router_b[l], w13_codes[l], w13_scales[l], b13[l], w2_codes[l], w2_scales[l],
                b2[l], T, d, I, E, k, clamp};
    a.alt = (flags & MOE_LAYER_ALT_ACT) ? 1 : 0;
    a.packed = (flags & MOE_LAYER_PACKED) ? 1 : 0;
    uint16_t* dst = bufs[cur];
    const bool last = (l == n_layers - 1);
    if (int st = run_layer(a, L, ws, nullptr, nullptr, nullptr, nullptr, nullptr, false, s, resid, dst,
                           last ? nullptr : norm, eps))
      return st;
    resid = dst;
    cur ^= 1;
  }
  return MOE_OK;
}

int moe_stack_forward(const void* x0, int n_layers, const void* const* router_w, const float* const* router_b,
                      const uint8_t* const* w13_codes, const uint8_t* const* w13_scales, const float* const* b13,
                      const uint8_t* const* w2_codes, const uint8_t* const* w2_scales, const float* const* b2,
                      int T, int d, int I, int E, int k, float clamp, float eps, void* out, void* stream) {
  return stack_forward(x0, n_layers, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d,
                       I, E, k, clamp, eps, 0, out, stream);
}

int moe_stack_forward_ex(const void* x0, int n_layers, const void* const* router_w, const float* const* router_b,
                         const uint8_t* const* w13_codes, const uint8_t* const* w13_scales, const float* const* b13,
                         const uint8_t* const* w2_codes, const uint8_t* const* w2_scales, const float* const* b2,
                         int T, int d, int I, int E, int k, float clamp, float eps, int flags, void* out,
                         void* stream) {
  return stack_forward(x0, n_layers, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, T, d,
                       I, E, k, clamp, eps, flags, out, stream);
}

size_t moe_packed_scale_bytes(int E, int N, int K) {
  if (E < 1 || N < 2 || (N & 1) || K < 64 || (K % 64)) return 0;
  return packed_scale_bytes(E, N, K);
}

int moe_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* codes_out,
                     uint8_t* scales_out, void* stream) {
  if (E < 1 || N < 2 || (N & 1) || K < 64 || (K % 64)) return MOE_ERR_BAD_SHAPE;
  const size_t nc = (size_t)E * N * (K / 2), ns = (size_t)E * N * (K / 32), nsp = packed_scale_bytes(E, N, K);
  if (nc >= (1ull << 40)) return MOE_ERR_UNSUPPORTED;
  if (!codes || !scales || !codes_out || !scales_out) return MOE_ERR_NULL_PTR;
  if (!aligned(codes, 16) || !aligned(codes_out, 16) || !aligned(scales_out, 4)) return MOE_ERR_MISALIGNED;
  if (overlap(codes_out, nc, codes, nc) || overlap(codes_out, nc, scales, ns) || overlap(scales_out, nsp, codes, nc) ||
      overlap(scales_out, nsp, scales, ns) || overlap(codes_out, nc, scales_out, nsp))
    return MOE_ERR_ALIAS;
  if (int st = check_device()) return st;
  return launch_pack_weights(codes, scales, E, N, K, codes_out, scales_out, (hipStream_t)stream) ? MOE_ERR_HIP
                                                                                                   : MOE_OK;
}

int moe_timing_enable(int mask) {
  g_t.mask = mask & 0x1f;
  return MOE_OK;
}

int moe_timing_read(double* ms, int* launches, int reset) {
  for (auto& r : g_t.pending) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return MOE_ERR_HIP;
    g_t.ms[r.kind] += t;
    g_t.n[r.kind] += 1;
    g_t.pool.push_back(r.a);
    g_t.pool.push_back(r.b);
  }
  g_t.pending.clear();
  for (int i = 0; i < 5; ++i) {
    if (ms) ms[i] = g_t.ms[i];
    if (launches) launches[i] = g_t.n[i];
    if (reset) { g_t.ms[i] = 0; g_t.n[i] = 0; }
  }
  return MOE_OK;
}

void moe_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (int dev = 0; dev < 64; ++dev) {
    OwnedWs& w = g_ws[dev];
    if (!w.p) continue;
    (void)hipSetDevice(dev);
    (void)hipDeviceSynchronize();
    (void)hipFree(w.p);
    w.p = nullptr;
    w.n = 0;
  }
  (void)hipSetDevice(cur);
}

}  // extern "C"

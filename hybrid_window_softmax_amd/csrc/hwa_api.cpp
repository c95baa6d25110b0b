// C ABI of libhwa: argument validation, workspace layouts and the launch
// sequences of the hybrid attention forward and of the backward of both
// branches. Declarations and semantics are
// in include/hwa.h.

#include <math.h>
#include <stddef.h>
#include <string.h>

#include "linear_bwd.h"

using hwa::bf16_t;
using hwa::Geom;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_dim_ok(int d, int dtype) {
  if (dtype == HWA_BF16) return d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64 || d == 128;
}

// The struct as first published ended at stage_events; fields after it are
// read only when the caller's struct_size covers them.
constexpr size_t kParamsV1 = offsetof(hwa_params, softmax_lse);

template <typename T>
T field_or_null(const hwa_params* p, T hwa_params::*f, size_t off) {
  return p->struct_size >= off + sizeof(T) ? p->*f : nullptr;
}
float* lse_out_of(const hwa_params* p) {
  return field_or_null(p, &hwa_params::softmax_lse, offsetof(hwa_params, softmax_lse));
}
void* sm_out_of(const hwa_params* p) {
  return field_or_null(p, &hwa_params::softmax_out, offsetof(hwa_params, softmax_out));
}
bool has_route_tau(const hwa_params* p) {
  return p->struct_size >= offsetof(hwa_params, route_tau) + sizeof(float);
}

// Basic checks on the params struct shared by every entry point.
hwa_status check_params(const hwa_params* p) {
  if (!p || p->struct_size < kParamsV1) return HWA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1) return HWA_ERR_INVALID_ARG;
  if (p->dtype != HWA_F32 && p->dtype != HWA_BF16) return HWA_ERR_INVALID_ARG;
  if (p->head_dim < 1) return HWA_ERR_INVALID_ARG;
  if (!head_dim_ok(p->head_dim, p->dtype)) return HWA_ERR_UNSUPPORTED;
  return HWA_OK;
}

bool make_geom(int32_t frames, int32_t tokens_per_frame, int32_t chunk,
               int32_t radius, const hwa_params* p, Geom& g) {
  if (frames < 1 || tokens_per_frame < 1 || chunk < 1 || radius < 0)
    return false;
  g.B = p->batch;
  g.H = p->heads;
  g.d = p->head_dim;
  g.F = frames;
  g.S = tokens_per_frame;
  g.chunk = chunk;
  g.radius = radius;
  g.nch = (frames + chunk - 1) / chunk;
  g.N = (long long)frames * tokens_per_frame;
  // grid dimensions and 32-bit launch parameters stay in range
  if (g.N > (1LL << 31) / 2 || (long long)g.B * g.H > 65535) return false;
  // bf16 softmax tiles are fetched with 32-bit byte offsets inside one head
  if (p->dtype == HWA_BF16 && ((g.N + 63) / 64 * 64) * g.d * 2 > (1LL << 31) - 1) return false;
  // one-dimensional softmax grid: query tiles x chunks x heads x batch
  if ((long long)((g.chunk * (long long)g.S + 127) / 128) * g.nch * g.B * g.H >
      (1LL << 31) - 1)
    return false;
  return true;
}

// Workspace regions the launch sequence needs besides the layout's fields:
// S_t and its eps (also in the layout) and the softmax kernel's work-queue
// counters (internal, the last region inside L.total).
struct Internal {
  size_t st16 = 0, st_eps = 0, sched = 0;
  size_t rq = 0, rk = 0, rcount = 0, rlist = 0;  // routing (HWA_FLAG_ROUTED)
};

hwa_workspace_layout compute_layout(const Geom& g, int dtype, Internal* in = nullptr,
                                    bool routed = false) {
  hwa_workspace_layout L;
  const size_t bh = (size_t)g.B * g.H;
  const size_t dd = (size_t)g.d * g.d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.lohi = take(2 * (size_t)g.F * sizeof(int32_t));
  L.stat_a = take(bh * g.F * dd * sizeof(float));
  L.stat_b = take(bh * g.F * dd * sizeof(float));
  L.map_m = take(bh * g.F * dd * sizeof(float));
  L.bank_p = take(bh * (g.nch + 1) * dd * sizeof(float));
  L.bank_q = take(bh * (g.nch + 1) * dd * sizeof(float));
  L.decay = take(bh * g.F * 2 * g.d * sizeof(float));
  L.bank_e = take(2 * bh * (g.nch + 1) * g.d * sizeof(int32_t));
  const size_t Np = (size_t)((g.N + 63) / 64 * 64);
  L.v_t = take(dtype == HWA_BF16 ? bh * g.d * Np * sizeof(bf16_t) : 0);
  Internal x;
  x.st16 = L.st16 = take(dtype == HWA_BF16 ? bh * g.F * dd * sizeof(_Float16) : 0);
  x.st_eps = L.st_eps = take(dtype == HWA_BF16 ? bh * g.F * sizeof(float) : 0);
  x.sched = take(hwa::HWA_SCHED_WORDS * sizeof(unsigned));
  if (routed) {
    const size_t units = bh * g.nch;
    const size_t nt = (size_t)hwa::route_tiles(g);
    x.rq = take(units * nt * g.d * sizeof(float));
    x.rk = take(units * (size_t)hwa::route_pieces(g) * g.d * sizeof(float));
    x.rcount = take(units * nt * sizeof(int32_t));
    x.rlist = take(units * nt * (size_t)hwa::route_blocks_max(g) * sizeof(uint16_t));
  }
  if (in) *in = x;
  L.total = off;
  return L;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x0 = (uintptr_t)a, x1 = x0 + na;
  uintptr_t y0 = (uintptr_t)b, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace

extern "C" {

const char* hwa_status_string(hwa_status s) {
  switch (s) {
    case HWA_OK: return "HWA_OK: success";
    case HWA_ERR_INVALID_ARG: return "HWA_ERR_INVALID_ARG: invalid argument";
    case HWA_ERR_UNSUPPORTED: return "HWA_ERR_UNSUPPORTED: unsupported head_dim or dtype";
    case HWA_ERR_WORKSPACE: return "HWA_ERR_WORKSPACE: workspace missing or too small";
    case HWA_ERR_HIP: return "HWA_ERR_HIP: HIP launch error";
  }
  return "unknown hwa_status";
}

hwa_status hwa_window_bounds(int32_t frames, int32_t chunk, int32_t radius,
                             int32_t* lo, int32_t* hi) {
  if (frames < 1 || chunk < 1 || radius < 0 || !lo || !hi)
    return HWA_ERR_INVALID_ARG;
  for (int32_t t = 0; t < frames; ++t) {
    const int64_t c = t / chunk;
    const int64_t l = (c - radius) * (int64_t)chunk;
    const int64_t h = (c + radius + 1) * (int64_t)chunk - 1;
    lo[t] = (int32_t)(l < 0 ? 0 : l);
    hi[t] = (int32_t)(h > frames - 1 ? frames - 1 : h);
  }
  return HWA_OK;
}

hwa_status hwa_get_workspace_layout(int32_t frames, int32_t tokens_per_frame,
                                    int32_t chunk, const hwa_params* p,
                                    hwa_workspace_layout* layout) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!layout || !make_geom(frames, tokens_per_frame, chunk, 0, p, g))
    return HWA_ERR_INVALID_ARG;
  *layout = compute_layout(g, p->dtype, nullptr, (p->flags & HWA_FLAG_ROUTED) != 0);
  return HWA_OK;
}

hwa_status hwa_get_route_layout(int32_t frames, int32_t tokens_per_frame, int32_t chunk,
                                const hwa_params* p, size_t* count_offset,
                                size_t* list_offset, int32_t* tiles_per_chunk,
                                int32_t* list_stride) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!count_offset || !list_offset || !tiles_per_chunk || !list_stride ||
      !make_geom(frames, tokens_per_frame, chunk, 0, p, g))
    return HWA_ERR_INVALID_ARG;
  Internal X;
  compute_layout(g, p->dtype, &X, true);
  *count_offset = X.rcount;
  *list_offset = X.rlist;
  *tiles_per_chunk = hwa::route_tiles(g);
  *list_stride = hwa::route_blocks_max(g);
  return HWA_OK;
}

size_t hwa_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, const hwa_params* p) {
  hwa_workspace_layout L;
  if (hwa_get_workspace_layout(frames, tokens_per_frame, chunk, p, &L) != HWA_OK)
    return 0;
  return L.total;
}

hwa_status hybrid_attn_fwd(const void* q, const void* k, const void* v,
                           const float* beta, const float* alpha,
                           const void* gate, const float* text_state,
                           int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, int32_t radius, int32_t rule,
                           void* out, hipStream_t stream, const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, radius, p, g))
    return HWA_ERR_INVALID_ARG;
  if (rule < HWA_RULE_VDN_SOLVE || rule > HWA_RULE_VDN_SCALED)
    return HWA_ERR_INVALID_ARG;
  const uint32_t known = HWA_FLAG_SOFTMAX_ONLY | HWA_FLAG_LINEAR_ONLY | HWA_FLAG_ROUTED;
  if (p->flags & ~known) return HWA_ERR_INVALID_ARG;
  const bool do_sm = !(p->flags & HWA_FLAG_LINEAR_ONLY);
  const bool do_lin = !(p->flags & HWA_FLAG_SOFTMAX_ONLY);
  if (!do_sm && !do_lin) return HWA_ERR_INVALID_ARG;
  const bool routed = (p->flags & HWA_FLAG_ROUTED) != 0;
  if (routed) {
    if (!do_sm || !has_route_tau(p) || isnan(p->route_tau)) return HWA_ERR_INVALID_ARG;
    if (p->dtype != HWA_BF16) return HWA_ERR_UNSUPPORTED;
    // the softmax kernel's list of kept 64-key tiles holds at most 4096
    const long long wkeys = (2LL * radius + 1) * chunk * (long long)tokens_per_frame;
    if (wkeys / 64 + 4 > 4096) return HWA_ERR_UNSUPPORTED;
  }
  if (!q || !k || !v || !out) return HWA_ERR_INVALID_ARG;
  if (do_lin && (!beta || !alpha || !gate || !p->conv_k || !p->conv_v))
    return HWA_ERR_INVALID_ARG;
  float* lse_out = lse_out_of(p);
  void* sm_out = sm_out_of(p);
  if (!do_sm && (lse_out || sm_out)) return HWA_ERR_INVALID_ARG;
  if (!isfinite(p->c) || !isfinite(p->text_scale) || !(p->rms_eps > 0.0f) ||
      !isfinite(p->rms_eps))
    return HWA_ERR_INVALID_ARG;

  const size_t es = p->dtype == HWA_BF16 ? 2 : 4;
  const size_t bh = (size_t)g.B * g.H;
  const size_t io_bytes = bh * (size_t)g.N * g.d * es;
  const void* qs = p->q_rope ? p->q_rope : q;
  const void* ks = p->k_rope ? p->k_rope : k;
  const size_t va = p->dtype == HWA_BF16 ? 16 : 4;
  if (!aligned(q, va) || !aligned(k, va) || !aligned(v, va) ||
      !aligned(out, va) || !aligned(qs, va) || !aligned(ks, va) ||
      (gate && !aligned(gate, va)) || (beta && !aligned(beta, 4)) ||
      (alpha && !aligned(alpha, 4)) || (text_state && !aligned(text_state, 4)) ||
      (lse_out && !aligned(lse_out, 4)) || (sm_out && !aligned(sm_out, va)))
    return HWA_ERR_INVALID_ARG;

  Internal X;
  const hwa_workspace_layout L = compute_layout(g, p->dtype, &X, routed);
  if (!p->workspace || p->workspace_bytes < L.total ||
      !aligned(p->workspace, kAlign))
    return HWA_ERR_WORKSPACE;

  // out must not alias any input or the workspace
  const struct { const void* ptr; size_t n; } ins[] = {
      {q, io_bytes},
      {k, io_bytes},
      {v, io_bytes},
      {gate, io_bytes},
      {p->q_rope, io_bytes},
      {p->k_rope, io_bytes},
      {beta, bh * (size_t)g.N * sizeof(float)},
      {alpha, bh * (size_t)g.F * g.d * sizeof(float)},
      {text_state, bh * (size_t)g.d * g.d * sizeof(float)},
      {p->workspace, p->workspace_bytes},
  };
  const size_t lse_bytes = bh * (size_t)g.N * sizeof(float);
  for (const auto& in : ins)
    if (overlaps(out, io_bytes, in.ptr, in.n) || overlaps(sm_out, io_bytes, in.ptr, in.n) ||
        overlaps(lse_out, lse_bytes, in.ptr, in.n))
      return HWA_ERR_INVALID_ARG;
  if (overlaps(sm_out, io_bytes, out, io_bytes) || overlaps(lse_out, lse_bytes, out, io_bytes) ||
      overlaps(lse_out, lse_bytes, sm_out, io_bytes))
    return HWA_ERR_INVALID_ARG;

  hipStream_t st = stream;
  char* ws = (char*)p->workspace;
  int32_t* lohi = (int32_t*)(ws + L.lohi);
  float* A = (float*)(ws + L.stat_a);
  float* Bm = (float*)(ws + L.stat_b);
  float* M = (float*)(ws + L.map_m);
  float* bank_p = (float*)(ws + L.bank_p);
  float* bank_q = (float*)(ws + L.bank_q);
  int32_t* bank_e = (int32_t*)(ws + L.bank_e);
  float* decay = (float*)(ws + L.decay);
  bf16_t* v_t = (bf16_t*)(ws + L.v_t);
  _Float16* st16 = (_Float16*)(ws + X.st16);
  float* st_eps = (float*)(ws + X.st_eps);
  unsigned* sched = (unsigned*)(ws + X.sched);

  void* const* ev = p->stage_events;
  auto mark = [&](int i) {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  // the linear branch first, so that on bf16 the softmax kernel can add its
  // readout in the epilogue (reading the raw q itself when the softmax runs
  // on q_rope)
  const bool fuse = do_sm && do_lin && p->dtype == HWA_BF16;
  if (mark(0) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_window_table(g, lohi, st, sched) != hipSuccess) return HWA_ERR_HIP;
  if (mark(1) != hipSuccess) return HWA_ERR_HIP;
  // on bf16 calls whose frames hold a multiple of 4 tokens the statistics
  // kernel also writes the softmax's transposed v
  const bool vt_fused = do_lin && do_sm && p->dtype == HWA_BF16 && g.S % 4 == 0;
  if (do_lin && hwa::launch_stats(g, p->dtype, k, v, beta, p->conv_k, p->conv_v, true, A, Bm,
                                  st, vt_fused ? v_t : nullptr) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(2) != hipSuccess) return HWA_ERR_HIP;
  const bool bf = p->dtype == HWA_BF16;
  if (do_lin && bf) {
    // M_f = (I + c~^2 A_f)^-1, or I - c^2 A_f for sana_scaled, written as the
    // bf16 scan's packed (hi, lo) operands into the map_m region
    const bool sana = rule == HWA_RULE_SANA_SCALED;
    const float cc = rule == HWA_RULE_VDN_SOLVE ? 1.0f : p->c * p->c;
    if (hwa::launch_update_packed(g, !sana, cc, A, (bf16_t*)M, st) != hipSuccess)
      return HWA_ERR_HIP;
  } else if (do_lin && rule != HWA_RULE_SANA_SCALED) {
    const float cc = rule == HWA_RULE_VDN_SCALED ? p->c : 1.0f;
    if (hwa::launch_inverse(g, cc * cc, A, M, st) != hipSuccess)
      return HWA_ERR_HIP;
  }
  if (mark(3) != hipSuccess) return HWA_ERR_HIP;
  if (do_lin && bf &&
      hwa::launch_scan_packed(g, rule, p->c, (const bf16_t*)M, Bm, alpha, text_state,
                              p->text_scale, bank_p, bank_q, bank_e, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (do_lin && !bf &&
      hwa::launch_scan(g, p->dtype, rule, p->c, A, Bm, M, alpha, text_state, p->text_scale,
                       bank_p, bank_q, bank_e, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(4) != hipSuccess) return HWA_ERR_HIP;
  if (do_lin && hwa::launch_decay(g, alpha, lohi, decay, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (do_lin && p->dtype == HWA_BF16 &&
      hwa::launch_state(g, decay, bank_p, bank_q, bank_e, p->rms_eps, st16, st_eps,
                        st) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(5) != hipSuccess) return HWA_ERR_HIP;
  if (do_sm && p->dtype == HWA_BF16 && !vt_fused &&
      hwa::launch_vtranspose(g, (const bf16_t*)v, v_t, st) != hipSuccess)
    return HWA_ERR_HIP;
  hwa::RouteArgs rt{(const int*)(ws + X.rcount), (const uint16_t*)(ws + X.rlist),
                    hwa::route_blocks_max(g)};
  if (routed &&
      hwa::launch_route(g, (const bf16_t*)qs, (const bf16_t*)ks, lohi, p->route_tau,
                        (float*)(ws + X.rq), (float*)(ws + X.rk), (int*)(ws + X.rcount),
                        (uint16_t*)(ws + X.rlist), rt.nkb_max, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(6) != hipSuccess) return HWA_ERR_HIP;
  const hwa::ReadoutArgs ra{(const bf16_t*)gate, st16, st_eps, p->rms_weight, g.F,
                            qs == q ? nullptr : (const bf16_t*)q};
  if (do_sm && hwa::launch_softmax(g, p->dtype, qs, ks, v, v_t, lohi, out, st,
                                   fuse ? &ra : nullptr, sched, lse_out, sm_out,
                                   routed ? &rt : nullptr) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(7) != hipSuccess) return HWA_ERR_HIP;
  if (do_lin && !fuse &&
      hwa::launch_readout(g, p->dtype, q, gate, decay, lohi, bank_p, bank_q,
                          bank_e, st16, st_eps, p->rms_weight, p->rms_eps, do_sm, out,
                          st) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(8) != hipSuccess) return HWA_ERR_HIP;
  return HWA_OK;
}

}  // extern "C"

namespace {

// Workspace of hwa_softmax_bwd: window table, delta and lse2 [B*H, Np] fp32.
struct BwdLayout {
  size_t lohi, delta, lse2, total;
};

BwdLayout bwd_layout(const Geom& g, int dtype) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  (void)dtype;
  const size_t bh = (size_t)g.B * g.H;
  const size_t Np = (size_t)((g.N + 63) / 64 * 64);
  L.lohi = take(2 * (size_t)g.F * sizeof(int32_t));
  L.delta = take(bh * Np * sizeof(float));
  L.lse2 = take(bh * Np * sizeof(float));
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t hwa_softmax_bwd_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                                       int32_t chunk, const hwa_params* p) {
  if (check_params(p) != HWA_OK) return 0;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, 0, p, g)) return 0;
  return bwd_layout(g, p->dtype).total;
}

hwa_status hwa_softmax_bwd(const void* q, const void* k, const void* v,
                           const void* o_sm, const float* lse, const void* d_o,
                           int32_t frames, int32_t tokens_per_frame,
                           int32_t chunk, int32_t radius, void* dq, void* dk,
                           void* dv, hipStream_t stream, const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, radius, p, g))
    return HWA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o_sm || !lse || !d_o || !dq || !dk || !dv)
    return HWA_ERR_INVALID_ARG;
  const size_t va = 16;  // 16-byte row loads on both dtypes
  if (!aligned(q, va) || !aligned(k, va) || !aligned(v, va) || !aligned(o_sm, va) ||
      !aligned(d_o, va) || !aligned(dq, va) || !aligned(dk, va) || !aligned(dv, va) ||
      !aligned(lse, 4))
    return HWA_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(g, p->dtype);
  if (!p->workspace || p->workspace_bytes < L.total || !aligned(p->workspace, kAlign))
    return HWA_ERR_WORKSPACE;
  const size_t es = p->dtype == HWA_BF16 ? 2 : 4;
  const size_t bh = (size_t)g.B * g.H;
  const size_t io_bytes = bh * (size_t)g.N * g.d * es;
  const struct { const void* ptr; size_t n; } ins[] = {
      {q, io_bytes}, {k, io_bytes}, {v, io_bytes}, {o_sm, io_bytes}, {d_o, io_bytes},
      {lse, bh * (size_t)g.N * sizeof(float)}, {p->workspace, p->workspace_bytes},
  };
  void* outs[] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i], io_bytes, in.ptr, in.n)) return HWA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], io_bytes, outs[j], io_bytes)) return HWA_ERR_INVALID_ARG;
  }

  hipStream_t st = stream;
  char* ws = (char*)p->workspace;
  int32_t* lohi = (int32_t*)(ws + L.lohi);
  float* delta = (float*)(ws + L.delta);
  float* lse2 = (float*)(ws + L.lse2);
  void* const* ev = p->stage_events;
  auto mark = [&](int i) {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  if (mark(0) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_window_table(g, lohi, st) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_bwd_prep(g, p->dtype, o_sm, d_o, lse, delta, lse2, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(1) != hipSuccess) return HWA_ERR_HIP;
  for (int part = 0; part < 2; ++part) {
    if (hwa::launch_softmax_bwd(g, p->dtype, part, q, k, v, d_o, lse2, delta, lohi, dq, dk,
                                dv, st) != hipSuccess)
      return HWA_ERR_HIP;
    if (mark(2 + part) != hipSuccess) return HWA_ERR_HIP;
  }
  return HWA_OK;
}

}  // extern "C"

namespace {

// Workspace of hwa_linear_bwd (see hwa::LinBwdArgs for what each holds).
struct LinBwdLayout {
  size_t A, Bm, M, Pst, Qst, E, dSt, dXQ, dbank, lam0, gab, dal, dwpart, dkc, dvc, cpart;
  size_t total;
};

LinBwdLayout lin_bwd_layout(const Geom& g) {
  LinBwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t bh = (size_t)g.B * g.H;
  const size_t dd = (size_t)g.d * g.d * sizeof(float);
  const size_t rowf = (size_t)g.d * sizeof(float);
  L.A = take(bh * g.F * dd);
  L.Bm = take(bh * g.F * dd);
  L.M = take(bh * g.F * dd);
  L.Pst = take(bh * (g.F + 1) * dd);
  L.Qst = take(bh * (g.F + 1) * dd);
  L.E = take(2 * bh * (g.F + 1) * g.d * sizeof(int32_t));
  L.dSt = take(bh * g.F * dd);
  L.dXQ = take(bh * g.F * dd);
  L.dbank = take(2 * bh * (g.nch + 1) * dd);
  L.lam0 = take(2 * bh * dd);
  L.gab = take(2 * bh * g.F * rowf);
  L.dal = take(bh * g.F * rowf);
  L.dwpart = take(bh * g.F * rowf);
  L.dkc = take(bh * (size_t)g.N * rowf);
  L.dvc = take(bh * (size_t)g.N * rowf);
  L.cpart = take(bh * g.F * 8 * rowf);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t hwa_linear_bwd_workspace_bytes(int32_t frames, int32_t tokens_per_frame,
                                      int32_t chunk, const hwa_params* p) {
  if (check_params(p) != HWA_OK) return 0;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, 0, p, g)) return 0;
  return lin_bwd_layout(g).total;
}

hwa_status hwa_linear_bwd(const void* q, const void* k, const void* v, const float* beta,
                          const float* alpha, const void* gate, const float* text_state,
                          const void* d_o, int32_t frames, int32_t tokens_per_frame,
                          int32_t chunk, int32_t radius, int32_t rule, void* dq, void* dk,
                          void* dv, float* dbeta, float* dalpha, void* dgate,
                          float* dtext_state, float* dconv_k, float* dconv_v,
                          float* drms_weight, hipStream_t stream, const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, radius, p, g)) return HWA_ERR_INVALID_ARG;
  if (rule < HWA_RULE_VDN_SOLVE || rule > HWA_RULE_VDN_SCALED) return HWA_ERR_INVALID_ARG;
  if (!q || !k || !v || !beta || !alpha || !gate || !d_o || !p->conv_k || !p->conv_v ||
      !dq || !dk || !dv || !dbeta || !dalpha || !dgate || !dconv_k || !dconv_v)
    return HWA_ERR_INVALID_ARG;
  if (!isfinite(p->c) || !isfinite(p->text_scale) || !(p->rms_eps > 0.0f) ||
      !isfinite(p->rms_eps))
    return HWA_ERR_INVALID_ARG;
  if (p->flags & ~(uint32_t)HWA_FLAG_ACCUMULATE) return HWA_ERR_INVALID_ARG;
  const size_t va = p->dtype == HWA_BF16 ? 16 : 4;
  const void* io_ptrs[] = {q, k, v, gate, d_o, dq, dk, dv, dgate};
  for (const void* x : io_ptrs)
    if (!aligned(x, va)) return HWA_ERR_INVALID_ARG;
  const void* f32_ptrs[] = {beta, alpha, text_state, p->conv_k, p->conv_v, p->rms_weight,
                            dbeta, dalpha, dtext_state, dconv_k, dconv_v, drms_weight};
  for (const void* x : f32_ptrs)
    if (x && !aligned(x, 4)) return HWA_ERR_INVALID_ARG;
  const LinBwdLayout L = lin_bwd_layout(g);
  if (!p->workspace || p->workspace_bytes < L.total || !aligned(p->workspace, kAlign))
    return HWA_ERR_WORKSPACE;

  const size_t es = p->dtype == HWA_BF16 ? 2 : 4;
  const size_t bh = (size_t)g.B * g.H;
  const size_t io_bytes = bh * (size_t)g.N * g.d * es;
  const size_t tok_bytes = bh * (size_t)g.N * sizeof(float);
  const size_t alpha_bytes = bh * (size_t)g.F * g.d * sizeof(float);
  const size_t mat_bytes = bh * (size_t)g.d * g.d * sizeof(float);
  const size_t conv_bytes = (size_t)g.H * g.d * 4 * sizeof(float);
  const struct { const void* ptr; size_t n; } ins[] = {
      {q, io_bytes}, {k, io_bytes}, {v, io_bytes}, {gate, io_bytes}, {d_o, io_bytes},
      {beta, tok_bytes}, {alpha, alpha_bytes}, {text_state, mat_bytes},
      {p->conv_k, conv_bytes}, {p->conv_v, conv_bytes},
      {p->rms_weight, (size_t)g.d * sizeof(float)}, {p->workspace, p->workspace_bytes},
  };
  const struct { const void* ptr; size_t n; } outs[] = {
      {dq, io_bytes}, {dk, io_bytes}, {dv, io_bytes}, {dgate, io_bytes},
      {dbeta, tok_bytes}, {dalpha, alpha_bytes}, {dtext_state, mat_bytes},
      {dconv_k, conv_bytes}, {dconv_v, conv_bytes},
      {drms_weight, (size_t)g.d * sizeof(float)},
  };
  const int n_outs = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < n_outs; ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i].ptr, outs[i].n, in.ptr, in.n)) return HWA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i].ptr, outs[i].n, outs[j].ptr, outs[j].n)) return HWA_ERR_INVALID_ARG;
  }

  char* ws = (char*)p->workspace;
  hwa::LinBwdArgs a;
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.d_o = d_o;
  a.beta = beta; a.alpha = alpha; a.text_state = text_state;
  a.conv_k = p->conv_k; a.conv_v = p->conv_v; a.rms_w = p->rms_weight;
  a.rule = rule; a.c = p->c; a.text_scale = p->text_scale; a.eps = p->rms_eps;
  a.acc = (p->flags & HWA_FLAG_ACCUMULATE) ? 1 : 0;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dgate = dgate;
  a.dbeta = dbeta; a.dalpha = dalpha; a.dtext = dtext_state;
  a.dconv_k = dconv_k; a.dconv_v = dconv_v; a.drms = drms_weight;
  a.A = (float*)(ws + L.A); a.Bm = (float*)(ws + L.Bm); a.M = (float*)(ws + L.M);
  a.Pst = (float*)(ws + L.Pst); a.Qst = (float*)(ws + L.Qst);
  a.E = (int32_t*)(ws + L.E);
  a.dSt = (float*)(ws + L.dSt);
  a.dXP = a.dSt;  // dS_t is consumed by the gather before the prefix adjoint writes
  a.dXQ = (float*)(ws + L.dXQ);
  a.dbank = (float*)(ws + L.dbank); a.lam0 = (float*)(ws + L.lam0);
  a.gab = (float*)(ws + L.gab); a.dal = (float*)(ws + L.dal);
  a.dwpart = (float*)(ws + L.dwpart);
  a.dkc = (float*)(ws + L.dkc); a.dvc = (float*)(ws + L.dvc);
  a.cpart = (float*)(ws + L.cpart);

  hipStream_t st = stream;
  void* const* ev = p->stage_events;
  auto mark = [&](int i) {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  if (mark(0) != hipSuccess) return HWA_ERR_HIP;
  for (int stage = 0; stage < 5; ++stage) {
    if (hwa::launch_linear_bwd(g, p->dtype, stage, a, st) != hipSuccess) return HWA_ERR_HIP;
    if (mark(stage + 1) != hipSuccess) return HWA_ERR_HIP;
  }
  return HWA_OK;
}

size_t hwa_text_state_workspace_bytes(int32_t text_tokens,
                                      const hwa_params* p) {
  if (check_params(p) != HWA_OK || text_tokens < 1) return 0;
  const size_t mat = (size_t)p->batch * p->heads * p->head_dim * p->head_dim *
                     sizeof(float);
  return 3 * align_up(mat);
}

hwa_status hwa_text_state(const void* k_txt, const void* v_txt,
                          const float* beta_txt, int32_t text_tokens,
                          float* state_out, hipStream_t stream,
                          const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  if (!k_txt || !v_txt || !beta_txt || !state_out || text_tokens < 1)
    return HWA_ERR_INVALID_ARG;
  Geom g;
  if (!make_geom(1, text_tokens, 1, 0, p, g)) return HWA_ERR_INVALID_ARG;
  const size_t need = hwa_text_state_workspace_bytes(text_tokens, p);
  if (!p->workspace || p->workspace_bytes < need ||
      !aligned(p->workspace, kAlign))
    return HWA_ERR_WORKSPACE;
  const size_t es = p->dtype == HWA_BF16 ? 2 : 4;
  const size_t bh = (size_t)g.B * g.H;
  const size_t io_bytes = bh * (size_t)text_tokens * g.d * es;
  const size_t st_bytes = bh * (size_t)g.d * g.d * sizeof(float);
  if (overlaps(state_out, st_bytes, k_txt, io_bytes) ||
      overlaps(state_out, st_bytes, v_txt, io_bytes) ||
      overlaps(state_out, st_bytes, beta_txt, bh * text_tokens * sizeof(float)) ||
      overlaps(state_out, st_bytes, p->workspace, p->workspace_bytes))
    return HWA_ERR_INVALID_ARG;
  // the forward's rules: 16 bytes for bf16 token rows (the statistics kernel
  // reads them 8 bytes at a time), 4 bytes for fp32 arrays
  const size_t va = p->dtype == HWA_BF16 ? 16 : 4;
  if (!aligned(k_txt, va) || !aligned(v_txt, va) || !aligned(beta_txt, 4) ||
      !aligned(state_out, 16))
    return HWA_ERR_INVALID_ARG;
  hipStream_t st = stream;
  float* A = (float*)p->workspace;
  float* Bm = (float*)((char*)p->workspace + need / 3);
  float* M = (float*)((char*)p->workspace + 2 * (need / 3));
  if (hwa::launch_stats(g, p->dtype, k_txt, v_txt, beta_txt, nullptr, nullptr,
                        false, A, Bm, st) != hipSuccess)
    return HWA_ERR_HIP;
  if (hwa::launch_inverse(g, 1.0f, A, M, st) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_matmul_bm(g, Bm, M, state_out, st) != hipSuccess)
    return HWA_ERR_HIP;
  return HWA_OK;
}

hwa_status hwa_frame_alpha(const void* k, const float* w, const float* bias,
                           const float* a_log, int32_t frames, int32_t tokens_per_frame,
                           float* alpha, hipStream_t stream, const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, 1, 0, p, g)) return HWA_ERR_INVALID_ARG;
  if (!k || !w || !bias || !a_log || !alpha) return HWA_ERR_INVALID_ARG;
  // 16-byte row loads of k; fp32 arrays on 4 bytes
  if (!aligned(k, 16) || !aligned(w, 4) || !aligned(bias, 4) || !aligned(a_log, 4) ||
      !aligned(alpha, 4))
    return HWA_ERR_INVALID_ARG;
  const size_t es = p->dtype == HWA_BF16 ? 2 : 4;
  const size_t bh = (size_t)g.B * g.H;
  const size_t a_bytes = bh * (size_t)g.F * g.d * sizeof(float);
  const struct { const void* ptr; size_t n; } ins[] = {
      {k, bh * (size_t)g.N * g.d * es},
      {w, (size_t)g.H * g.d * g.d * sizeof(float)},
      {bias, (size_t)g.H * g.d * sizeof(float)},
      {a_log, (size_t)g.H * g.d * sizeof(float)},
  };
  for (const auto& in : ins)
    if (overlaps(alpha, a_bytes, in.ptr, in.n)) return HWA_ERR_INVALID_ARG;
  if (hwa::launch_frame_alpha(g, p->dtype, k, w, bias, a_log, alpha, stream) != hipSuccess)
    return HWA_ERR_HIP;
  return HWA_OK;
}

namespace {

// The block's own regions (q, k, v, q_rope, k_rope, the attention output)
// before the attention's workspace.
size_t block_io_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * g.N * g.d * sizeof(bf16_t));
}

}  // namespace

size_t hwa_block_workspace_bytes(int32_t frames, int32_t tokens_per_frame, int32_t chunk,
                                 const hwa_params* p) {
  if (check_params(p) != HWA_OK || p->dtype != HWA_BF16) return 0;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, 0, p, g)) return 0;
  const size_t att = hwa_workspace_bytes(frames, tokens_per_frame, chunk, p);
  return att ? 6 * block_io_bytes(g) + att : 0;
}

hwa_status hwa_block_fwd(const void* x, const void* w_qkv, const void* w_o, const float* beta,
                         const float* alpha, const void* gate, const float* text_state,
                         int32_t frames, int32_t tokens_per_frame, int32_t grid_w,
                         float rope_theta, int32_t chunk, int32_t radius, int32_t rule, void* y,
                         hipStream_t stream, const hwa_params* p) {
  hwa_status s = check_params(p);
  if (s != HWA_OK) return s;
  if (p->dtype != HWA_BF16) return HWA_ERR_UNSUPPORTED;
  Geom g;
  if (!make_geom(frames, tokens_per_frame, chunk, radius, p, g)) return HWA_ERR_INVALID_ARG;
  if (!x || !w_qkv || !w_o || !y || grid_w < 1 || tokens_per_frame % grid_w != 0 ||
      !(rope_theta > 0.0f) || !isfinite(rope_theta))
    return HWA_ERR_INVALID_ARG;
  if (p->flags || p->q_rope || p->k_rope || lse_out_of(p) || sm_out_of(p))
    return HWA_ERR_INVALID_ARG;
  const size_t D = (size_t)g.H * g.d;
  const size_t M = (size_t)g.B * g.N;
  // 32-bit byte offsets of the projections' direct loads
  if (M * D * 2 >= (1ull << 31)) return HWA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(y, 16))
    return HWA_ERR_INVALID_ARG;
  const size_t need = hwa_block_workspace_bytes(frames, tokens_per_frame, chunk, p);
  if (!need || !p->workspace || p->workspace_bytes < need || !aligned(p->workspace, kAlign))
    return HWA_ERR_WORKSPACE;
  const size_t io = M * D * sizeof(bf16_t);
  const struct { const void* ptr; size_t n; } ins[] = {
      {x, io}, {w_qkv, 3 * D * D * sizeof(bf16_t)}, {w_o, D * D * sizeof(bf16_t)},
      {p->workspace, p->workspace_bytes},
  };
  for (const auto& in : ins)
    if (overlaps(y, io, in.ptr, in.n)) return HWA_ERR_INVALID_ARG;

  char* ws = (char*)p->workspace;
  const size_t r = block_io_bytes(g);
  bf16_t* q = (bf16_t*)ws;
  bf16_t* k = (bf16_t*)(ws + r);
  bf16_t* v = (bf16_t*)(ws + 2 * r);
  bf16_t* qr = (bf16_t*)(ws + 3 * r);
  bf16_t* kr = (bf16_t*)(ws + 4 * r);
  bf16_t* att = (bf16_t*)(ws + 5 * r);
  hwa_params pa = *p;
  pa.q_rope = qr;
  pa.k_rope = kr;
  pa.workspace = ws + 6 * r;
  pa.workspace_bytes = p->workspace_bytes - 6 * r;
  pa.stage_events = nullptr;
  // the attention's own checks, before anything is enqueued: with a NULL
  // workspace it stops at the workspace check (HWA_ERR_WORKSPACE) when every
  // other argument is valid
  {
    hwa_params pv = pa;
    pv.workspace = nullptr;
    pv.workspace_bytes = 0;
    const hwa_status sv = hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, frames,
                                          tokens_per_frame, chunk, radius, rule, att, stream, &pv);
    if (sv != HWA_ERR_WORKSPACE) return sv;
  }
  void* const* ev = p->stage_events;
  auto mark = [&](int i) { return ev ? hipEventRecord((hipEvent_t)ev[i], stream) : hipSuccess; };
  if (mark(0) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_gemm_qkv((const bf16_t*)x, (const bf16_t*)w_qkv, (int)M, (int)g.N, g.H, g.d,
                           g.S, grid_w, rope_theta, q, k, v, qr, kr, stream) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(1) != hipSuccess) return HWA_ERR_HIP;
  s = hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, frames, tokens_per_frame, chunk,
                      radius, rule, att, stream, &pa);
  if (s != HWA_OK) return s;
  if (mark(2) != hipSuccess) return HWA_ERR_HIP;
  if (hwa::launch_gemm_out(att, (const bf16_t*)w_o, (int)M, (int)g.N, g.H, g.d, (bf16_t*)y,
                           stream) != hipSuccess)
    return HWA_ERR_HIP;
  if (mark(3) != hipSuccess) return HWA_ERR_HIP;
  return HWA_OK;
}

}  // extern "C"

// C ABI of the low-rank bottleneck block: host-side argument checks, workspace
// carving and launch sequencing.  The operations are documented in lr_block.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "lr_block.h"
#include "lr_kernels.h"

namespace {

using lr::bf16;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t esize(int32_t dt) { return dt == LR_BF16 ? 2 : 4; }
inline int n_up_of(const lr_dims* d) { return d->act == LR_ACT_SWIGLU ? 1 : (int)d->g; }

// Shape checks shared by every entry point.
lr_status check_dims(const lr_dims* d) {
  if (!d) return LR_EINVAL;
  if (d->dtype != LR_F32 && d->dtype != LR_BF16) return LR_EINVAL;
  if (d->act < LR_ACT_IDENTITY || d->act > LR_ACT_SWIGLU) return LR_EINVAL;
  if (d->T < 0 || d->d <= 0 || d->r <= 0 || d->g <= 0 || d->d_norm < 0) return LR_EINVAL;
  if (!(d->eps >= 0.f) || !isfinite(d->eps)) return LR_EINVAL;
  if (d->d % 64 || d->r % 64) return LR_EUNSUPPORTED;
  if (d->g > lr::MAX_G) return LR_EUNSUPPORTED;
  if (d->act == LR_ACT_SWIGLU && d->g != 2) return LR_EUNSUPPORTED;
  // every index below is formed in 64 bits; tile coordinates in 32 bits
  if (d->T > (1ll << 30) || d->d > (1 << 20) || d->r * d->g > (1 << 20)) return LR_EUNSUPPORTED;
  return LR_OK;
}

inline float inv_width(const lr_dims* d) { return 1.0f / (float)(d->d_norm ? d->d_norm : d->d); }

struct Carve {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    P* p = reinterpret_cast<P*>(base + off);
    off += align_up(bytes);
    return p;
  }
};

// split count of the small-rank forward for these dims (0: not used)
int small_splits(const lr_dims* d) {
  return d->dtype == LR_BF16 ? lr::small_rank_splits<bf16>((int)d->T, (int)d->d, (int)d->r, (int)d->g, d->act)
                             : lr::small_rank_splits<float>((int)d->T, (int)d->d, (int)d->r, (int)d->g, d->act);
}

// whether the forward runs as the one-kernel small-rank path
bool fused_fwd(const lr_dims* d) {
  return d->dtype == LR_BF16 && lr::fused_fwd_supported((int)d->r, (int)d->g, d->act);
}

// A' (or A'^T), z, then for the small-rank forward the split partials and sums of
// squares.  The one-kernel path uses A'^T and the B_i in fragment order; z stays
// reserved for the shard seam (lr_up_finish), which shares this size.
size_t fwd_ws(const lr_dims* d) {
  const size_t es = esize(d->dtype), gr = (size_t)(d->g * d->r), T = (size_t)d->T;
  if (fused_fwd(d)) return 2 * align_up((size_t)d->d * gr * es) + align_up(T * gr * es);
  const size_t ns = (size_t)small_splits(d);
  return align_up((size_t)d->d * gr * es) + align_up(T * gr * es) + align_up(ns * T * gr * 4) +
         align_up(ns * T * 4);
}

template <typename E>
size_t bwd_ws_t(const lr_dims* d) {
  const size_t es = sizeof(E), gr = (size_t)(d->g * d->r), T = (size_t)d->T;
  const int nsp = n_up_of(d) * lr::dz_nparts<E>((int)d->r);
  const int ngp = lr::wgrad_nparts<E>((int)gr);
  const lr::WgradPlan wp = lr::wgrad_plan<E>((int)d->T, (int)d->d, (int)d->r, (int)d->g, n_up_of(d), (int)d->d);
  const size_t part = (size_t)wp.part_floats * 4;
  return align_up(T * 4) + align_up(T * gr * es) * 2 + align_up(T * lr::spart_stride(nsp) * 4) +
         align_up((size_t)d->d * ngp * 4) +
         align_up(part);
}

size_t bwd_ws(const lr_dims* d) { return d->dtype == LR_BF16 ? bwd_ws_t<bf16>(d) : bwd_ws_t<float>(d); }

inline lr_status hip_status(hipError_t e) { return e == hipSuccess ? LR_OK : LR_EHIP; }

// Per-thread launch trace (lr_trace_*): event pairs around matching launches.
constexpr int kMaxTraceLaunches = 1 << 16;
struct Trace {
  bool on = false;
  char filter[32] = {0};
  int cap = 0, n = 0;
  hipEvent_t* ev = nullptr;
  const char** names = nullptr;
};
thread_local Trace g_trace;

struct TraceGuard {
  hipStream_t s;
  int slot = -1;
  TraceGuard(const char* name, hipStream_t st) : s(st) {
    Trace& t = g_trace;
    if (!t.on || t.n >= t.cap || (t.filter[0] && strcmp(t.filter, name) != 0)) return;
    slot = t.n++;
    t.names[slot] = name;
    (void)hipEventRecord(t.ev[2 * slot], s);
  }
  ~TraceGuard() {
    if (slot >= 0) (void)hipEventRecord(g_trace.ev[2 * slot + 1], s);
  }
};

#define LR_LAUNCH(name, s, expr)          \
  do {                                    \
    TraceGuard tg_(name, s);              \
    hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return LR_EHIP; \
  } while (0)

template <typename E>
lr_status fwd_impl(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                   const void* const* residual, void* const* y, void* h_save, float* rstd_save, void* ws,
                   hipStream_t s) {
  const int T = (int)d->T, D = (int)d->d, r = (int)d->r, g = (int)d->g, gr = g * r, n_up = n_up_of(d);
  Carve cv{static_cast<char*>(ws)};
  void* Ap = cv.take<void>((size_t)D * gr * sizeof(E));
  // With a residual the one-kernel small-rank forward is not used: those shapes
  // run the down-projection and the up-projection (whose epilogue adds the
  // residual), which fit in the same workspace.
  const bool one_kernel = fused_fwd(d) && !residual;
  if (one_kernel) {
    // small g*r: x . A', deferred rstd, sigma and the up-projections in one
    // kernel; z stays in LDS
    void* Bf = cv.take<void>((size_t)D * gr * sizeof(E));
    LR_LAUNCH("fold_gamma", s, lr::launch_fold_fused(A, gamma, B, n_up, Ap, Bf, D, gr, r, s));
    lr::FusedArgs fa{};
    fa.x = x; fa.Apt = Ap; fa.Bf = Bf; fa.h = h_save; fa.rstd = rstd_save;
    for (int i = 0; i < n_up; ++i) fa.y[i] = y[i];
    fa.T = T; fa.d = D; fa.r = r; fa.g = g; fa.invD = inv_width(d); fa.eps = d->eps;
    LR_LAUNCH("fused", s, lr::launch_fused_fwd(fa, d->act, s));
    return LR_OK;
  }
  void* z = cv.take<void>((size_t)T * gr * sizeof(E));
  const int ns = fused_fwd(d) ? 0 : small_splits(d);
  if (ns > 0) {
    // small g*r: split-K down-projection into fp32 partials, then the finish
    // kernel (sum, deferred rstd, sigma), then the up-projection
    float* part = cv.take<float>((size_t)ns * T * gr * 4);
    float* ssp = cv.take<float>((size_t)ns * T * 4);
    LR_LAUNCH("fold_gamma", s, lr::launch_fold_gamma_t<E>(A, gamma, Ap, D, gr, s));
    lr::SplitDownArgs sa{};
    sa.x = x; sa.Apt = Ap; sa.T = T; sa.d = D; sa.gr = gr; sa.nsplit = ns; sa.partial = part; sa.sumsq = ssp;
    {
      const int BK = lr::gemm_bk<E>();
      sa.ksplit = (((D + BK - 1) / BK + ns - 1) / ns) * BK;
    }
    LR_LAUNCH("down", s, lr::launch_down_split<E>(sa, s));
    LR_LAUNCH("finish", s, lr::launch_finish<E>(part, ssp, h_save, z, rstd_save, T, r, g, d->act, inv_width(d),
                                                d->eps, ns, s));
  } else {
    LR_LAUNCH("fold_gamma", s, lr::launch_fold_gamma<E>(A, gamma, Ap, D, gr, s));
    lr::DownArgs da{};
    da.x = x; da.Ap = Ap; da.T = T; da.d = D; da.r = r; da.g = g; da.act = d->act; da.mode = lr::DOWN_BLOCK;
    da.invD = inv_width(d); da.eps = d->eps; da.h = h_save; da.z = z; da.rstd = rstd_save;
    LR_LAUNCH("down", s, lr::launch_down<E>(da, s));
  }
  lr::UpArgs ua{};
  const bool z_is_h = d->act == LR_ACT_IDENTITY && h_save;
  ua.z = z_is_h ? h_save : z;
  ua.ldz = d->act == LR_ACT_SWIGLU ? r : gr;
  for (int i = 0; i < n_up; ++i) {
    ua.B[i] = B[i];
    ua.y[i] = y[i];
    ua.res[i] = residual ? residual[i] : nullptr;
  }
  ua.T = T; ua.d = D; ua.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(ua, n_up, s));
  return LR_OK;
}

template <typename E>
lr_status bwd_impl(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                   const void* h, const float* rstd_saved, const void* const* dy, const void* dx_residual, void* dx,
                   float* dgamma, float* dA, float* const* dB, void* ws, hipStream_t s) {
  const int T = (int)d->T, D = (int)d->d, r = (int)d->r, g = (int)d->g, gr = g * r, n_up = n_up_of(d);
  const int nsp = n_up * lr::dz_nparts<E>(r);
  const int ngp = lr::wgrad_nparts<E>(gr);
  Carve cv{static_cast<char*>(ws)};
  float* rstd_ws = cv.take<float>((size_t)T * 4);
  void* dh = cv.take<void>((size_t)T * gr * sizeof(E));
  void* z = cv.take<void>((size_t)T * gr * sizeof(E));
  const int sps = lr::spart_stride(nsp);
  float* spart = cv.take<float>((size_t)T * sps * 4);
  float* gpart = cv.take<float>((size_t)D * ngp * 4);
  const lr::WgradPlan wp = lr::wgrad_plan<E>(T, D, r, g, n_up, D);
  const int ns = wp.nsplit;
  // the split-tile plan reduces only dB tiles; dA's tiles run whole and leave
  // dgamma partials, as an unsplit pass does
  const bool reduced = wp.streamk || ns > 1;
  // dgamma from the whole dA tiles' row partials: its own launch after an
  // unsplit pass, inside the reduction with split tiles
  const bool gamma_parts = !reduced;
  const int64_t pstride = (int64_t)n_up * r * D + (int64_t)D * gr;
  float* wpart = cv.take<float>((size_t)wp.part_floats * 4);

  // the forward's rstd when the caller kept it, else recomputed from x
  const float* rstd = rstd_saved;
  if (!rstd) {
    LR_LAUNCH("rms_stats", s,
              lr::launch_rms_stats<E>(x, nullptr, nullptr, nullptr, rstd_ws, T, D, inv_width(d), d->eps, s));
    rstd = rstd_ws;
  }

  lr::DzArgs za{};
  for (int i = 0; i < n_up; ++i) { za.dy[i] = dy[i]; za.B[i] = B[i]; }
  za.h = h; za.rstd = rstd; za.dh = dh; za.z = z; za.spart = spart; za.spstride = sps;
  za.T = T; za.d = D; za.r = r; za.g = g; za.act = d->act;
  LR_LAUNCH("dz", s, lr::launch_dz<E>(za, n_up, s));

  lr::WgradArgs wa{};
  wa.z = d->act == LR_ACT_IDENTITY ? h : z;
  wa.ldz = d->act == LR_ACT_SWIGLU ? r : gr;
  for (int i = 0; i < n_up; ++i) { wa.dy[i] = dy[i]; wa.dB[i] = dB[i]; }
  wa.x = x; wa.dh = dh; wa.A = A; wa.gamma = gamma; wa.dA = dA; wa.dgamma = dgamma; wa.gpart = gpart; wa.ngpart = ngp;
  wa.T = T; wa.d = D; wa.dn = D; wa.r = r; wa.g = g; wa.n_up = n_up;
  wa.nsplit = ns; wa.wpart = wpart; wa.part_stride = pstride; wa.part_offA = (int64_t)n_up * r * D;
  wa.streamk = wp.streamk; wa.sk_G = wp.G; wa.sk_Q = wp.Q; wa.sk_R = wp.R; wa.sk_KS = wp.KS;
  wa.sk_maxseg = wp.maxseg; wa.sk_S = wp.S; wa.sk_tiles = wp.tiles; wa.split_tiles = wp.split_tiles;
  wa.gparts_used = lr::wgrad_nparts_used<E>(gr, false);
  {
    const int BK = lr::gemm_bk<E>();   // split lengths are whole k steps
    const int ksteps = (T + BK - 1) / BK;
    wa.ksplit = ((ksteps + ns - 1) / ns) * BK;
  }
  LR_LAUNCH("wgrad", s, lr::launch_wgrad<E>(wa, s));
  if (reduced)  // the reduction (it also forms dgamma)
    LR_LAUNCH("wgrad_reduce", s, lr::launch_wgrad_reduce<E>(wa, s));
  if (gamma_parts)  // dA's tiles ran whole: they left per-tile dgamma partials
    LR_LAUNCH("sum_parts", s, lr::launch_sum_parts(gpart, dgamma, D, lr::wgrad_nparts_used<E>(gr, false), ngp, s));

  lr::DxArgs xa{};
  xa.dh = dh; xa.A = A; xa.x = x; xa.gamma = gamma; xa.rstd = rstd; xa.spart = spart; xa.nspart = nsp; xa.spstride = sps;
  xa.dx = dx; xa.dres = dx_residual; xa.T = T; xa.d = D; xa.r = r; xa.g = g; xa.invD = inv_width(d);
  LR_LAUNCH("dx", s, lr::launch_dx<E>(xa, s));
  return LR_OK;
}

template <typename E>
lr_status partial_impl(const lr_dims* d, const void* x, const void* gamma, const void* A, float* partial,
                       float* sumsq, void* ws, hipStream_t s) {
  const int T = (int)d->T, D = (int)d->d, r = (int)d->r, g = (int)d->g, gr = g * r;
  Carve cv{static_cast<char*>(ws)};
  void* Ap = cv.take<void>((size_t)D * gr * sizeof(E));
  LR_LAUNCH("fold_gamma", s, lr::launch_fold_gamma<E>(A, gamma, Ap, D, gr, s));
  lr::DownArgs da{};
  da.x = x; da.Ap = Ap; da.T = T; da.d = D; da.r = r; da.g = g; da.act = d->act; da.mode = lr::DOWN_PARTIAL;
  da.invD = inv_width(d); da.eps = d->eps; da.partial = partial; da.sumsq = sumsq;
  LR_LAUNCH("down", s, lr::launch_down<E>(da, s));
  return LR_OK;
}

template <typename E>
lr_status finish_impl(const lr_dims* d, const float* partial, const float* sumsq, const void* const* B,
                      void* const* y, void* h_save, void* ws, hipStream_t s) {
  const int T = (int)d->T, D = (int)d->d, r = (int)d->r, g = (int)d->g, gr = g * r, n_up = n_up_of(d);
  Carve cv{static_cast<char*>(ws)};
  cv.take<void>((size_t)D * gr * sizeof(E));  // same layout as the forward
  void* z = cv.take<void>((size_t)T * gr * sizeof(E));
  LR_LAUNCH("finish", s, lr::launch_finish<E>(partial, sumsq, h_save, z, nullptr, T, r, g, d->act, inv_width(d),
                                              d->eps, 1, s));
  lr::UpArgs ua{};
  const bool z_is_h = d->act == LR_ACT_IDENTITY && h_save;
  ua.z = z_is_h ? h_save : z;
  ua.ldz = d->act == LR_ACT_SWIGLU ? r : gr;
  for (int i = 0; i < n_up; ++i) { ua.B[i] = B[i]; ua.y[i] = y[i]; }
  ua.T = T; ua.d = D; ua.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(ua, n_up, s));
  return LR_OK;
}

lr_status check_ptrs(const void* const* arr, int n) {
  if (!arr) return LR_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!arr[i] || !aligned16(arr[i])) return LR_EINVAL;
  return LR_OK;
}
inline bool req(const void* p) { return p && aligned16(p); }
inline bool opt(const void* p) { return !p || aligned16(p); }
// a [T, ...] buffer: may be NULL when there are no rows
inline bool req_rows(const void* p, int64_t T) { return T == 0 ? opt(p) : req(p); }
lr_status check_rows_ptrs(const void* const* arr, int n, int64_t T) {
  if (!arr) return LR_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!req_rows(arr[i], T)) return LR_EINVAL;
  return LR_OK;
}

lr_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return LR_OK;
  if (!ws || !aligned16(ws) || have < need) return LR_EWORKSPACE;
  return LR_OK;
}

lr_status fwd_entry(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                    const void* const* residual, void* const* y, void* h_save, float* rstd_save, void* ws,
                    size_t ws_bytes, hipStream_t s) {
  lr_status st = check_dims(d);
  if (st != LR_OK) return st;
  if (!req_rows(x, d->T) || !req(gamma) || !req(A) || !opt(h_save) || !opt(rstd_save)) return LR_EINVAL;
  const int n_up = n_up_of(d);
  if ((st = check_ptrs(B, n_up)) != LR_OK) return st;
  if ((st = check_rows_ptrs(reinterpret_cast<const void* const*>(y), n_up, d->T)) != LR_OK) return st;
  if (residual && (st = check_rows_ptrs(residual, n_up, d->T)) != LR_OK) return st;
  if ((st = check_ws(ws, ws_bytes, fwd_ws(d))) != LR_OK) return st;
  return d->dtype == LR_BF16 ? fwd_impl<bf16>(d, x, gamma, A, B, residual, y, h_save, rstd_save, ws, s)
                             : fwd_impl<float>(d, x, gamma, A, B, residual, y, h_save, rstd_save, ws, s);
}

lr_status bwd_entry(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                    const void* h_saved, const float* rstd_saved, const void* const* dy, const void* dx_residual,
                    void* dx, float* dgamma, float* dA, float* const* dB, void* ws, size_t ws_bytes, hipStream_t s) {
  lr_status st = check_dims(d);
  if (st != LR_OK) return st;
  if (!req_rows(x, d->T) || !req(gamma) || !req(A) || !req_rows(h_saved, d->T) || !opt(rstd_saved) ||
      !req_rows(dx, d->T) || !req(dgamma) || !req(dA) || !opt(dx_residual))
    return LR_EINVAL;
  const int n_up = n_up_of(d);
  if ((st = check_ptrs(B, n_up)) != LR_OK) return st;
  if ((st = check_rows_ptrs(dy, n_up, d->T)) != LR_OK) return st;
  if ((st = check_ptrs(reinterpret_cast<const void* const*>(dB), n_up)) != LR_OK) return st;
  if ((st = check_ws(ws, ws_bytes, bwd_ws(d))) != LR_OK) return st;
  return d->dtype == LR_BF16
             ? bwd_impl<bf16>(d, x, gamma, A, B, h_saved, rstd_saved, dy, dx_residual, dx, dgamma, dA, dB, ws, s)
             : bwd_impl<float>(d, x, gamma, A, B, h_saved, rstd_saved, dy, dx_residual, dx, dgamma, dA, dB, ws, s);
}


// ---------------------------------------------------------------- per-projection low-rank SwiGLU MLP
// Input layers: the block with identity between its factors, g = 2 and
// up-projections of width f; SwiGLU at width f in the second up-projection's
// epilogue; output layer: a down factor without normalisation over width f and
// an up factor back to d.  The backward recomputes gate, up and s from h_in.
lr_status check_mlp(const lr_mlp_dims* m) {
  if (!m) return LR_EINVAL;
  if (m->dtype != LR_F32 && m->dtype != LR_BF16) return LR_EINVAL;
  if (m->T < 0 || m->d <= 0 || m->f <= 0 || m->r <= 0) return LR_EINVAL;
  if (!(m->eps >= 0.f) || !isfinite(m->eps)) return LR_EINVAL;
  if (m->d % 64 || m->f % 64 || m->r % 64) return LR_EUNSUPPORTED;
  if (m->T > (1ll << 30) || m->d > (1 << 20) || m->f > (1 << 20) || m->r > (1 << 19)) return LR_EUNSUPPORTED;
  return LR_OK;
}

// A'_in, h_in, h_out, gate, s
size_t mlp_fwd_ws(const lr_mlp_dims* m) {
  const size_t es = esize(m->dtype), T = (size_t)m->T, d = (size_t)m->d, f = (size_t)m->f, r = (size_t)m->r;
  return align_up(d * 2 * r * es) + align_up(T * 2 * r * es) + align_up(T * r * es) + 2 * align_up(T * f * es);
}

template <typename E>
lr::WgradPlan mlp_plan_in(const lr_mlp_dims* m) {
  return lr::wgrad_plan<E>((int)m->T, (int)m->d, (int)m->r, 2, 2, (int)m->f);
}
template <typename E>
lr::WgradPlan mlp_plan_out(const lr_mlp_dims* m) {
  return lr::wgrad_plan<E>((int)m->T, (int)m->f, (int)m->r, 1, 1, (int)m->d);
}

// rstd, gate, up, s, dh_out, dh_in, S' partials, dgamma partials, weight-gradient partials
template <typename E>
size_t mlp_bwd_ws_t(const lr_mlp_dims* m) {
  const size_t es = sizeof(E), T = (size_t)m->T, d = (size_t)m->d, f = (size_t)m->f, r = (size_t)m->r;
  const int nsp = 2 * lr::dz_nparts<E>((int)r);
  const int ngp = lr::wgrad_nparts<E>(2 * (int)r);
  const int64_t pf1 = mlp_plan_in<E>(m).part_floats, pf2 = mlp_plan_out<E>(m).part_floats;
  return align_up(T * 4) + 3 * align_up(T * f * es) + align_up(T * r * es) + align_up(T * 2 * r * es) +
         align_up(T * lr::spart_stride(nsp) * 4) + align_up(d * ngp * 4) +
         align_up((size_t)(pf1 > pf2 ? pf1 : pf2) * 4);
}
size_t mlp_bwd_ws(const lr_mlp_dims* m) { return m->dtype == LR_BF16 ? mlp_bwd_ws_t<bf16>(m) : mlp_bwd_ws_t<float>(m); }

template <typename E>
lr_status mlp_fwd_impl(const lr_mlp_dims* m, const void* x, const void* gamma, const void* A_in, const void* B_g,
                       const void* B_u, const void* A_o, const void* B_o, const void* residual, void* out,
                       void* h_in_save, void* h_out_save, float* rstd_save, void* ws, hipStream_t s) {
  const int T = (int)m->T, D = (int)m->d, F = (int)m->f, r = (int)m->r;
  Carve cv{static_cast<char*>(ws)};
  void* Ap = cv.take<void>((size_t)D * 2 * r * sizeof(E));
  void* h_in = cv.take<void>((size_t)T * 2 * r * sizeof(E));
  void* h_out = cv.take<void>((size_t)T * r * sizeof(E));
  void* gate = cv.take<void>((size_t)T * F * sizeof(E));
  void* sw = cv.take<void>((size_t)T * F * sizeof(E));
  if (h_in_save) h_in = h_in_save;
  if (h_out_save) h_out = h_out_save;
  // input layers' down factors: [A_g | A_u] with gamma folded in, rstd applied late
  LR_LAUNCH("fold_gamma", s, lr::launch_fold_gamma<E>(A_in, gamma, Ap, D, 2 * r, s));
  lr::DownArgs da{};
  da.x = x; da.Ap = Ap; da.T = T; da.d = D; da.r = r; da.g = 2; da.act = lr::ACT_IDENTITY; da.mode = lr::DOWN_BLOCK;
  da.invD = 1.0f / (float)D; da.eps = m->eps; da.h = h_in; da.z = h_in; da.rstd = rstd_save;
  LR_LAUNCH("down", s, lr::launch_down<E>(da, s));
  // their up factors: gate, then up with s = SiLU(gate) * up formed in the epilogue
  lr::UpArgs ug{};
  ug.z = h_in; ug.ldz = 2 * r; ug.B[0] = B_g; ug.y[0] = gate; ug.T = T; ug.d = F; ug.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(ug, 1, s));
  lr::UpArgs uu{};
  uu.z = static_cast<const E*>(h_in) + r; uu.ldz = 2 * r; uu.B[0] = B_u; uu.y[0] = sw; uu.res[0] = gate; uu.swiglu = 1;
  uu.T = T; uu.d = F; uu.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(uu, 1, s));
  // output layer: down factor over width f (no normalisation), up factor to d
  lr::DownArgs dd{};
  dd.x = sw; dd.Ap = A_o; dd.T = T; dd.d = F; dd.r = r; dd.g = 1; dd.act = lr::ACT_IDENTITY; dd.mode = lr::DOWN_PLAIN;
  dd.invD = 1.0f / (float)F; dd.eps = m->eps; dd.h = h_out; dd.z = h_out;
  LR_LAUNCH("down", s, lr::launch_down<E>(dd, s));
  lr::UpArgs uo{};
  uo.z = h_out; uo.ldz = r; uo.B[0] = B_o; uo.y[0] = out; uo.res[0] = residual; uo.T = T; uo.d = D; uo.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(uo, 1, s));
  return LR_OK;
}

// weight gradients of one layer group: the launch, then the reduction and the
// dgamma sum where the plan needs them
template <typename E>
lr_status mlp_wgrad(lr::WgradArgs wa, const lr::WgradPlan& wp, int gr, float* gpart, int ngp, hipStream_t s) {
  const int ns = wp.nsplit;
  const bool reduced = wp.streamk || ns > 1;
  const bool gamma_parts = wa.gamma && !reduced;
  wa.nsplit = ns;
  wa.part_stride = (int64_t)wa.n_up * wa.r * wa.dn + (int64_t)wa.d * gr;
  wa.part_offA = (int64_t)wa.n_up * wa.r * wa.dn;
  wa.streamk = wp.streamk; wa.sk_G = wp.G; wa.sk_Q = wp.Q; wa.sk_R = wp.R; wa.sk_KS = wp.KS;
  wa.sk_maxseg = wp.maxseg; wa.sk_S = wp.S; wa.sk_tiles = wp.tiles; wa.split_tiles = wp.split_tiles;
  wa.gparts_used = lr::wgrad_nparts_used<E>(gr, false);
  {
    const int BK = lr::gemm_bk<E>();
    const int ksteps = (wa.T + BK - 1) / BK;
    wa.ksplit = ((ksteps + ns - 1) / ns) * BK;
  }
  LR_LAUNCH("wgrad", s, lr::launch_wgrad<E>(wa, s));
  if (reduced) LR_LAUNCH("wgrad_reduce", s, lr::launch_wgrad_reduce<E>(wa, s));
  if (gamma_parts)
    LR_LAUNCH("sum_parts", s, lr::launch_sum_parts(gpart, wa.dgamma, wa.d, lr::wgrad_nparts_used<E>(gr, false), ngp, s));
  return LR_OK;
}

template <typename E>
lr_status mlp_bwd_impl(const lr_mlp_dims* m, const void* x, const void* gamma, const void* A_in, const void* B_g,
                       const void* B_u, const void* A_o, const void* B_o, const void* h_in, const void* h_out,
                       const float* rstd_saved, const void* dout, const void* dx_residual, void* dx, float* dgamma,
                       float* dA_in, float* dB_g, float* dB_u, float* dA_o, float* dB_o, void* ws, hipStream_t s) {
  const int T = (int)m->T, D = (int)m->d, F = (int)m->f, r = (int)m->r;
  const int nsp = 2 * lr::dz_nparts<E>(r), sps = lr::spart_stride(nsp);
  const int ngp = lr::wgrad_nparts<E>(2 * r);
  const lr::WgradPlan p_in = mlp_plan_in<E>(m), p_out = mlp_plan_out<E>(m);
  Carve cv{static_cast<char*>(ws)};
  float* rstd_ws = cv.take<float>((size_t)T * 4);
  void* gate = cv.take<void>((size_t)T * F * sizeof(E));
  void* up = cv.take<void>((size_t)T * F * sizeof(E));
  void* sw = cv.take<void>((size_t)T * F * sizeof(E));
  void* dh_out = cv.take<void>((size_t)T * r * sizeof(E));
  void* dh_in = cv.take<void>((size_t)T * 2 * r * sizeof(E));
  float* spart = cv.take<float>((size_t)T * sps * 4);
  float* gpart = cv.take<float>((size_t)D * ngp * 4);
  float* wpart = cv.take<float>((size_t)(p_in.part_floats > p_out.part_floats ? p_in.part_floats : p_out.part_floats) * 4);

  const float* rstd = rstd_saved;
  if (!rstd) {
    LR_LAUNCH("rms_stats", s,
              lr::launch_rms_stats<E>(x, nullptr, nullptr, nullptr, rstd_ws, T, D, 1.0f / (float)D, m->eps, s));
    rstd = rstd_ws;
  }
  // gate, up and s recomputed from the checkpoint h_in
  lr::UpArgs ug{};
  ug.z = h_in; ug.ldz = 2 * r; ug.B[0] = B_g; ug.y[0] = gate; ug.T = T; ug.d = F; ug.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(ug, 1, s));
  lr::UpArgs uu{};
  uu.z = static_cast<const E*>(h_in) + r; uu.ldz = 2 * r; uu.B[0] = B_u; uu.y[0] = sw; uu.y2[0] = up;
  uu.res[0] = gate; uu.swiglu = 1; uu.T = T; uu.d = F; uu.r = r;
  LR_LAUNCH("up", s, lr::launch_up<E>(uu, 1, s));

  // output layer: dh_out = dout . B_o^T; dB_o = h_out^T . dout and dA_o = s^T . dh_out
  lr::DzArgs zo{};
  zo.dy[0] = dout; zo.B[0] = B_o; zo.h = h_out; zo.rstd = nullptr; zo.dh = dh_out; zo.z = nullptr;
  zo.spart = nullptr; zo.spstride = 0; zo.T = T; zo.d = D; zo.r = r; zo.g = 1; zo.act = lr::ACT_IDENTITY;
  LR_LAUNCH("dz", s, lr::launch_dz<E>(zo, 1, s));
  lr::WgradArgs wo{};
  wo.z = h_out; wo.ldz = r; wo.dy[0] = dout; wo.dB[0] = dB_o; wo.x = sw; wo.dh = dh_out; wo.A = nullptr;
  wo.gamma = nullptr; wo.dA = dA_o; wo.dgamma = nullptr; wo.gpart = nullptr; wo.ngpart = 0; wo.wpart = wpart;
  wo.T = T; wo.d = F; wo.dn = D; wo.r = r; wo.g = 1; wo.n_up = 1;
  lr_status st = mlp_wgrad<E>(wo, p_out, r, nullptr, 0, s);
  if (st != LR_OK) return st;
  // ds = dh_out . A_o^T with the SwiGLU backward in the epilogue: dgate over
  // gate, dup over up (s is no longer needed)
  lr::DxArgs xo{};
  xo.dh = dh_out; xo.A = A_o; xo.x = gate; xo.dres = up; xo.dx = gate; xo.dx2 = up; xo.swiglu = 1;
  xo.T = T; xo.d = F; xo.r = r; xo.g = 1; xo.invD = 1.0f / (float)F;
  LR_LAUNCH("dx", s, lr::launch_dx<E>(xo, s));

  // input layers: the block's backward for dy = (dgate, dup)
  lr::DzArgs zi{};
  zi.dy[0] = gate; zi.dy[1] = up; zi.B[0] = B_g; zi.B[1] = B_u; zi.h = h_in; zi.rstd = rstd; zi.dh = dh_in;
  zi.z = nullptr; zi.spart = spart; zi.spstride = sps; zi.T = T; zi.d = F; zi.r = r; zi.g = 2;
  zi.act = lr::ACT_IDENTITY;
  LR_LAUNCH("dz", s, lr::launch_dz<E>(zi, 2, s));
  lr::WgradArgs wi{};
  wi.z = h_in; wi.ldz = 2 * r; wi.dy[0] = gate; wi.dy[1] = up; wi.dB[0] = dB_g; wi.dB[1] = dB_u; wi.x = x;
  wi.dh = dh_in; wi.A = A_in; wi.gamma = gamma; wi.dA = dA_in; wi.dgamma = dgamma; wi.gpart = gpart;
  wi.ngpart = ngp; wi.wpart = wpart; wi.T = T; wi.d = D; wi.dn = F; wi.r = r; wi.g = 2; wi.n_up = 2;
  if ((st = mlp_wgrad<E>(wi, p_in, 2 * r, gpart, ngp, s)) != LR_OK) return st;
  lr::DxArgs xi{};
  xi.dh = dh_in; xi.A = A_in; xi.x = x; xi.gamma = gamma; xi.rstd = rstd; xi.spart = spart; xi.nspart = nsp;
  xi.spstride = sps; xi.dx = dx; xi.dres = dx_residual; xi.T = T; xi.d = D; xi.r = r; xi.g = 2;
  xi.invD = 1.0f / (float)D;
  LR_LAUNCH("dx", s, lr::launch_dx<E>(xi, s));
  return LR_OK;
}



// Scratch of the allocation-free forward (lr_block_fwd_noalloc): a file-scope
// device array, one copy per GPU, held until the process ends.  Host code uses
// only the device address hipGetSymbolAddress returns for the current device,
// never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = (size_t)LR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// the scratch array's address on device `dev` (which is current), looked up once
lr_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return LR_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return LR_EHIP;
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return LR_OK;
}

}  // namespace

extern "C" {

const char* lr_status_str(lr_status st) {
  switch (st) {
    case LR_OK: return "LR_OK";
    case LR_EINVAL: return "LR_EINVAL";
    case LR_EUNSUPPORTED: return "LR_EUNSUPPORTED";
    case LR_EWORKSPACE: return "LR_EWORKSPACE";
    case LR_EHIP: return "LR_EHIP";
  }
  return "LR_UNKNOWN";
}

size_t lr_block_workspace_size(const lr_dims* d, int backward) {
  if (check_dims(d) != LR_OK) return 0;
  return backward ? bwd_ws(d) : fwd_ws(d);
}

lr_status rmsnorm_online(const lr_dims* d, const void* x, const void* gamma, void* y, float* sumsq, float* rstd,
                         hipStream_t s) {
  if (!d) return LR_EINVAL;
  if (d->dtype != LR_F32 && d->dtype != LR_BF16) return LR_EINVAL;
  if (d->T < 0 || d->d <= 0 || d->d_norm < 0 || !(d->eps >= 0.f) || !isfinite(d->eps)) return LR_EINVAL;
  if (d->d % 8) return LR_EUNSUPPORTED;
  if (d->T > (1ll << 30) || d->d > (1 << 24)) return LR_EUNSUPPORTED;
  if (!req_rows(x, d->T) || !opt(y) || !opt(sumsq) || !opt(rstd)) return LR_EINVAL;
  if (y && !req(gamma)) return LR_EINVAL;
  const int T = (int)d->T, D = (int)d->d;
  if (d->dtype == LR_BF16)
    LR_LAUNCH("rms_stats", s, lr::launch_rms_stats<bf16>(x, gamma, y, sumsq, rstd, T, D, inv_width(d), d->eps, s));
  else
    LR_LAUNCH("rms_stats", s, lr::launch_rms_stats<float>(x, gamma, y, sumsq, rstd, T, D, inv_width(d), d->eps, s));
  return LR_OK;
}


lr_status lr_block_fwd_rstd(const lr_dims* d, const void* x, const void* gamma, const void* A,
                            const void* const* B, void* const* y, void* h_save, float* rstd_save, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  return fwd_entry(d, x, gamma, A, B, nullptr, y, h_save, rstd_save, ws, ws_bytes, s);
}

lr_status lr_block_fwd(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                       void* const* y, void* h_save, void* ws, size_t ws_bytes, hipStream_t s) {
  return fwd_entry(d, x, gamma, A, B, nullptr, y, h_save, nullptr, ws, ws_bytes, s);
}

lr_status lr_block_fwd_residual(const lr_dims* d, const void* x, const void* gamma, const void* A,
                                const void* const* B, const void* const* residual, void* const* y, void* h_save,
                                float* rstd_save, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!residual) return LR_EINVAL;
  return fwd_entry(d, x, gamma, A, B, residual, y, h_save, rstd_save, ws, ws_bytes, s);
}

lr_status lr_block_fwd_noalloc(const lr_dims* d, const void* x, const void* gamma, const void* A,
                               const void* const* B, void* const* y, void* h_save, float* rstd_save,
                               hipStream_t s) {
  lr_status st = check_dims(d);
  if (st != LR_OK) return st;
  if (!req_rows(x, d->T) || !req(gamma) || !req(A) || !opt(h_save) || !opt(rstd_save)) return LR_EINVAL;
  const int n_up = n_up_of(d);
  if ((st = check_ptrs(B, n_up)) != LR_OK) return st;
  if ((st = check_rows_ptrs(reinterpret_cast<const void* const*>(y), n_up, d->T)) != LR_OK) return st;
  const size_t need = fwd_ws(d);
  if (need > kScratchBytes) return LR_EWORKSPACE;
  // the stream must belong to the current device, whose copy of the array the
  // kernels get
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LR_EHIP;
  if (hipStreamGetDevice(s, &sdev) != hipSuccess) return LR_EHIP;
  if (sdev != dev) return LR_EINVAL;
  void* ws = nullptr;
  if ((st = scratch_on(dev, &ws)) != LR_OK) return st;
  return d->dtype == LR_BF16 ? fwd_impl<bf16>(d, x, gamma, A, B, nullptr, y, h_save, rstd_save, ws, s)
                             : fwd_impl<float>(d, x, gamma, A, B, nullptr, y, h_save, rstd_save, ws, s);
}

lr_status lr_block_bwd_rstd(const lr_dims* d, const void* x, const void* gamma, const void* A,
                            const void* const* B, const void* h_saved, const float* rstd_saved,
                            const void* const* dy, void* dx, float* dgamma, float* dA, float* const* dB, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  return bwd_entry(d, x, gamma, A, B, h_saved, rstd_saved, dy, nullptr, dx, dgamma, dA, dB, ws, ws_bytes, s);
}

lr_status lr_block_bwd(const lr_dims* d, const void* x, const void* gamma, const void* A, const void* const* B,
                       const void* h_saved, const void* const* dy, void* dx, float* dgamma, float* dA,
                       float* const* dB, void* ws, size_t ws_bytes, hipStream_t s) {
  return bwd_entry(d, x, gamma, A, B, h_saved, nullptr, dy, nullptr, dx, dgamma, dA, dB, ws, ws_bytes, s);
}

lr_status lr_block_bwd_residual(const lr_dims* d, const void* x, const void* gamma, const void* A,
                                const void* const* B, const void* h_saved, const float* rstd_saved,
                                const void* const* dy, const void* dx_residual, void* dx, float* dgamma, float* dA,
                                float* const* dB, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dx_residual && d && d->T > 0) return LR_EINVAL;
  return bwd_entry(d, x, gamma, A, B, h_saved, rstd_saved, dy, dx_residual, dx, dgamma, dA, dB, ws, ws_bytes, s);
}

lr_status lr_down_partial(const lr_dims* d, const void* x, const void* gamma, const void* A, float* partial,
                          float* sumsq, void* ws, size_t ws_bytes, hipStream_t s) {
  lr_status st = check_dims(d);
  if (st != LR_OK) return st;
  if (!req_rows(x, d->T) || !req(gamma) || !req(A) || !req_rows(partial, d->T) || !req_rows(sumsq, d->T))
    return LR_EINVAL;
  if ((st = check_ws(ws, ws_bytes, fwd_ws(d))) != LR_OK) return st;
  return d->dtype == LR_BF16 ? partial_impl<bf16>(d, x, gamma, A, partial, sumsq, ws, s)
                             : partial_impl<float>(d, x, gamma, A, partial, sumsq, ws, s);
}

lr_status lr_up_finish(const lr_dims* d, const float* partial, const float* sumsq, const void* const* B,
                       void* const* y, void* h_save, void* ws, size_t ws_bytes, hipStream_t s) {
  lr_status st = check_dims(d);
  if (st != LR_OK) return st;
  if (!req_rows(partial, d->T) || !req_rows(sumsq, d->T) || !opt(h_save)) return LR_EINVAL;
  const int n_up = n_up_of(d);
  if ((st = check_ptrs(B, n_up)) != LR_OK) return st;
  if ((st = check_rows_ptrs(reinterpret_cast<const void* const*>(y), n_up, d->T)) != LR_OK) return st;
  if ((st = check_ws(ws, ws_bytes, fwd_ws(d))) != LR_OK) return st;
  return d->dtype == LR_BF16 ? finish_impl<bf16>(d, partial, sumsq, B, y, h_save, ws, s)
                             : finish_impl<float>(d, partial, sumsq, B, y, h_save, ws, s);
}

size_t lr_mlp_workspace_size(const lr_mlp_dims* m, int backward) {
  if (check_mlp(m) != LR_OK) return 0;
  return backward ? mlp_bwd_ws(m) : mlp_fwd_ws(m);
}

lr_status lr_mlp_fwd(const lr_mlp_dims* m, const void* x, const void* gamma, const void* A_in, const void* B_g,
                     const void* B_u, const void* A_o, const void* B_o, const void* residual, void* out,
                     void* h_in_save, void* h_out_save, float* rstd_save, void* ws, size_t ws_bytes, hipStream_t s) {
  lr_status st = check_mlp(m);
  if (st != LR_OK) return st;
  if (!req_rows(x, m->T) || !req(gamma) || !req(A_in) || !req(B_g) || !req(B_u) || !req(A_o) || !req(B_o) ||
      !opt(residual) || !req_rows(out, m->T) || !opt(h_in_save) || !opt(h_out_save) || !opt(rstd_save))
    return LR_EINVAL;
  if ((st = check_ws(ws, ws_bytes, mlp_fwd_ws(m))) != LR_OK) return st;
  return m->dtype == LR_BF16 ? mlp_fwd_impl<bf16>(m, x, gamma, A_in, B_g, B_u, A_o, B_o, residual, out, h_in_save,
                                                  h_out_save, rstd_save, ws, s)
                             : mlp_fwd_impl<float>(m, x, gamma, A_in, B_g, B_u, A_o, B_o, residual, out,
                                                   h_in_save, h_out_save, rstd_save, ws, s);
}

lr_status lr_mlp_bwd(const lr_mlp_dims* m, const void* x, const void* gamma, const void* A_in, const void* B_g,
                     const void* B_u, const void* A_o, const void* B_o, const void* h_in_saved,
                     const void* h_out_saved, const float* rstd_saved, const void* dout, const void* dx_residual,
                     void* dx, float* dgamma, float* dA_in, float* dB_g, float* dB_u, float* dA_o, float* dB_o,
                     void* ws, size_t ws_bytes, hipStream_t s) {
  lr_status st = check_mlp(m);
  if (st != LR_OK) return st;
  if (!req_rows(x, m->T) || !req(gamma) || !req(A_in) || !req(B_g) || !req(B_u) || !req(A_o) || !req(B_o) ||
      !req_rows(h_in_saved, m->T) || !req_rows(h_out_saved, m->T) || !opt(rstd_saved) || !req_rows(dout, m->T) ||
      !opt(dx_residual) || !req_rows(dx, m->T) || !req(dgamma) || !req(dA_in) || !req(dB_g) || !req(dB_u) ||
      !req(dA_o) || !req(dB_o))
    return LR_EINVAL;
  if ((st = check_ws(ws, ws_bytes, mlp_bwd_ws(m))) != LR_OK) return st;
  return m->dtype == LR_BF16
             ? mlp_bwd_impl<bf16>(m, x, gamma, A_in, B_g, B_u, A_o, B_o, h_in_saved, h_out_saved, rstd_saved, dout,
                                  dx_residual, dx, dgamma, dA_in, dB_g, dB_u, dA_o, dB_o, ws, s)
             : mlp_bwd_impl<float>(m, x, gamma, A_in, B_g, B_u, A_o, B_o, h_in_saved, h_out_saved, rstd_saved, dout,
                                   dx_residual, dx, dgamma, dA_in, dB_g, dB_u, dA_o, dB_o, ws, s);
}

lr_status lr_trace_begin(const char* kernel, int max_launches) {
  Trace& t = g_trace;
  if (t.on || max_launches < 1 || max_launches > kMaxTraceLaunches) return LR_EINVAL;
  t.ev = new (std::nothrow) hipEvent_t[2 * (size_t)max_launches];
  t.names = new (std::nothrow) const char*[max_launches];
  if (!t.ev || !t.names) {
    delete[] t.ev;
    delete[] t.names;
    t = Trace{};
    return LR_EINVAL;
  }
  for (int i = 0; i < 2 * max_launches; ++i) {
    if (hipEventCreate(&t.ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(t.ev[j]);
      delete[] t.ev;
      delete[] t.names;
      t = Trace{};
      return LR_EHIP;
    }
  }
  t.cap = max_launches;
  t.n = 0;
  t.filter[0] = 0;
  if (kernel) {
    strncpy(t.filter, kernel, sizeof(t.filter) - 1);
    t.filter[sizeof(t.filter) - 1] = 0;
  }
  t.on = true;
  return LR_OK;
}

int lr_trace_count(void) { return g_trace.on ? g_trace.n : 0; }

lr_status lr_trace_elapsed(int i, const char** kernel, float* ms) {
  Trace& t = g_trace;
  if (!t.on || i < 0 || i >= t.n || !ms) return LR_EINVAL;
  if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess) return LR_EHIP;
  if (hipEventElapsedTime(ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return LR_EHIP;
  if (kernel) *kernel = t.names[i];
  return LR_OK;
}

lr_status lr_trace_end(void) {
  Trace& t = g_trace;
  if (!t.on) return LR_EINVAL;
  for (int i = 0; i < 2 * t.cap; ++i) (void)hipEventDestroy(t.ev[i]);
  delete[] t.ev;
  delete[] t.names;
  t = Trace{};
  return LR_OK;
}

}  // extern "C"

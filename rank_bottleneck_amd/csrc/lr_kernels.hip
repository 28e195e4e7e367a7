// HIP kernels of the fused low-rank bottleneck block (gfx950).
//
// Forward  (lr_block_fwd):
//   fold_gamma : A' = diag(gamma) . A                      (weights only, d x g*r)
//   down       : acc = x . A'  with the per-token sum of squares of x accumulated
//                from the same x tiles on their way to LDS (Online-RMSNorm: the
//                statistic is local, the normalisation is applied late), then
//                h = rstd * acc, sigma(h) in fp32 registers; writes h (checkpoint),
//                rstd when kept, and z = sigma(h).  SwiGLU pairs gate/up columns in one lane.
//   up         : y_i = z_i . B_i, batched over branches (one launch).
// Backward (lr_block_bwd), with h' = rstd * dh (rstd the forward's, or recomputed):
//   stats      : rstd from x, when the forward's was not kept
//   dz         : dz_i = dy_i . B_i^T; epilogue: dh from sigma'(h_saved), writes
//                dh' = rstd*dh, z = sigma(h) and per-row partials of
//                S'_t = sum_c dh'_tc h_tc
//   wgrad_B    : dB_i = z_i^T . dy_i                       (reduced over tokens)
//   wgrad_A    : M = x^T . dh';  dA = diag(gamma) M,  dgamma partials sum_c A_jc M_jc
//   dx         : dx = gamma * (dh' . A^T) - x * rstd * S'/D
//   reduce     : dgamma_j = sum of partials
// The two rank-r identities used (sum_k gamma_k dxn_tk x_tk = S_t / rstd_t and
// dgamma_j = sum_c A_jc (xhat^T dh)_jc) move both RMSNorm-backward reductions onto
// rank-r tensors.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lr_device.h"
#include "lr_pipe.h"
#include "lr_kernels.h"

namespace lr {

constexpr int kGroupM = 4;  // row panels per scheduling group

// ------------------------------------------------------------------ small kernels
template <typename E>
__global__ __launch_bounds__(256) void k_rms_stats(const E* __restrict__ x, const E* __restrict__ gamma,
                                                   E* __restrict__ y, float* __restrict__ sumsq,
                                                   float* __restrict__ rstd, int T, int d, float invD,
                                                   float eps) {
  // one wave per row, 16-byte vectors
  constexpr int VEC = 16 / (int)sizeof(E);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const E* xr = x + (int64_t)row * d;
  // U independent 16-byte loads in flight per lane before any arithmetic
  constexpr int U = 8;
  float s = 0.f;
  for (int j0 = lane * VEC; j0 < d; j0 += 64 * VEC * U) {
    uint4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 64 * VEC;
      q[u] = j < d ? *reinterpret_cast<const uint4*>(xr + j) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += sumsq_vec(q[u], (E*)nullptr);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const float rs = 1.0f / sqrtf(s * invD + eps);
  if (lane == 0) {
    if (sumsq) sumsq[row] = s;
    if (rstd) rstd[row] = rs;
  }
  if (y) {
    E* yr = y + (int64_t)row * d;
    for (int j = lane * VEC; j < d; j += 64 * VEC) {
      uint4 q = *reinterpret_cast<const uint4*>(xr + j);
      uint4 gq = *reinterpret_cast<const uint4*>(gamma + j);
      const E* xe = reinterpret_cast<const E*>(&q);
      const E* ge = reinterpret_cast<const E*>(&gq);
      uint4 o;
      E* oe = reinterpret_cast<E*>(&o);
#pragma unroll
      for (int e = 0; e < VEC; ++e) oe[e] = from_f32<E>(to_f32(xe[e]) * rs * to_f32(ge[e]));
      *reinterpret_cast<uint4*>(yr + j) = o;
    }
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_fold_gamma(const E* __restrict__ A, const E* __restrict__ gamma,
                                                    E* __restrict__ Ap, int d, int n) {
  constexpr int VEC = 16 / (int)sizeof(E);
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
  if (i >= (int64_t)d * n) return;
  const int j = (int)(i / n);
  const float gj = to_f32(gamma[j]);
  uint4 q = *reinterpret_cast<const uint4*>(A + i);
  E* e = reinterpret_cast<E*>(&q);
#pragma unroll
  for (int k = 0; k < VEC; ++k) e[k] = from_f32<E>(to_f32(e[k]) * gj);
  *reinterpret_cast<uint4*>(Ap + i) = q;
}

// A'^T [n, d] through 64 x 16 blocks (64 rows of A, 16 of its columns) in LDS:
// the rows of A'^T are written with consecutive threads on consecutive elements
// (d is a multiple of 64, n of 16)
template <typename E>
__global__ __launch_bounds__(256) void k_fold_gamma_t(const E* __restrict__ A, const E* __restrict__ gamma,
                                                      E* __restrict__ Apt, int d, int n) {
  __shared__ float tile[64][17];
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = threadIdx.x + k * 256, jj = e / 16, cc = e % 16;
    tile[jj][cc] = to_f32(A[(int64_t)(j0 + jj) * n + c0 + cc]) * to_f32(gamma[j0 + jj]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = threadIdx.x + k * 256, cc = e / 64, jj = e % 64;
    Apt[(int64_t)(c0 + cc) * d + j0 + jj] = from_f32<E>(tile[jj][cc]);
  }
}

// seam: h = partial * rstd, z = sigma(h)
// (the partials and sums of squares of nsplit K splits are added in split order);
// one thread per 4 consecutive output columns of a row
template <typename E>
__global__ __launch_bounds__(256) void k_finish(const float* __restrict__ partial, const float* __restrict__ sumsq,
                                                E* __restrict__ h, E* __restrict__ z, float* __restrict__ rstd,
                                                int T, int r, int g, int act, float invD, float eps, int nsplit) {
  const int gr = g * r;
  const int ncols = (act == ACT_SWIGLU) ? r : gr;
  const int q4 = ncols / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * q4) return;
  const int t = (int)(i / q4), c = (int)(i % q4) * 4;
  const int64_t pstride = (int64_t)T * gr;
  float ss = 0.f;
  for (int k = 0; k < nsplit; ++k) ss += sumsq[(int64_t)k * T + t];
  const float rs = 1.0f / sqrtf(ss * invD + eps);
  if (rstd && c == 0) rstd[t] = rs;
  const float* pr = partial + (int64_t)t * gr;
  auto col4 = [&](int cc) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < nsplit; ++k) {
      const float4 p = *reinterpret_cast<const float4*>(pr + k * pstride + cc);
      v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    }
    return make_float4(v.x * rs, v.y * rs, v.z * rs, v.w * rs);
  };
  const int64_t hrow = (int64_t)t * gr;
  if (act == ACT_SWIGLU) {
    const float4 g4 = col4(c), u4 = col4(r + c);
    if (h) {
      store4(h + hrow + c, g4.x, g4.y, g4.z, g4.w);
      store4(h + hrow + r + c, u4.x, u4.y, u4.z, u4.w);
    }
    store4(z + (int64_t)t * r + c, g4.x * sigmoidf_(g4.x) * u4.x, g4.y * sigmoidf_(g4.y) * u4.y,
           g4.z * sigmoidf_(g4.z) * u4.z, g4.w * sigmoidf_(g4.w) * u4.w);
  } else {
    const float4 v = col4(c);
    if (h) store4(h + hrow + c, v.x, v.y, v.z, v.w);
    if (act == ACT_SILU)
      store4(z + hrow + c, v.x * sigmoidf_(v.x), v.y * sigmoidf_(v.y), v.z * sigmoidf_(v.z), v.w * sigmoidf_(v.w));
    else if (!h)
      store4(z + hrow + c, v.x, v.y, v.z, v.w);
  }
}

__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ parts, float* __restrict__ out,
                                                   int n, int nparts, int stride) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float* p = parts + (int64_t)i * stride;
  float s = 0.f;
  for (int k = 0; k < nparts; ++k) s += p[k];
  out[i] = s;
}

// Work-group -> tile.  A grid of T/256 x N/256 tiles whose last round would
// leave at least half of the CUs idle runs its full rounds as 256-row tiles and
// each remaining tile as two 128-row halves (HALF), which fill the CUs once;
// both in one launch, the halves' work-groups after the whole tiles'.  Work-group
// bid of nblk (of its part) takes tile tile0 + i in the grid's order (per-XCD
// ranges, groups of row panels), i its renumbered index; in the HALF part the
// renumbered pairs (2i, 2i+1) take the two halves of tile tile0 + i.
template <bool HALF>
__device__ __forceinline__ void tail_index(int tile0, int bid, int nblk, int& t, int& piece) {
  const int idx = xcd_remap(bid, nblk);
  t = tile0 + (HALF ? idx / 2 : idx);
  piece = HALF ? idx % 2 : 0;
}
// rows of tiles of the full grid: of 2*BM rows for HALF launches
template <class C, bool HALF>
__device__ __forceinline__ int tile_rows(int T) {
  constexpr int ROWS = HALF ? 2 * C::BM : C::BM;
  return (T + ROWS - 1) / ROWS;
}
template <class C, bool HALF>
__device__ __forceinline__ void tail_tile(int tile0, int bid, int nblk, int T, int tiles_n, int& tm, int& tn,
                                          int& m0) {
  int t, piece;
  tail_index<HALF>(tile0, bid, nblk, t, piece);
  grouped_tile<kGroupM>(t, tile_rows<C, HALF>(T), tiles_n, tm, tn);
  m0 = (tm * (HALF ? 2 : 1) + piece) * C::BM;
}

// LDS words a GEMM kernel needs: the mainloop ring or the epilogue staging,
// whichever is larger, plus BM floats of per-row values.
// LDS of a GEMM kernel: the mainloop's tiles, then (after the mainloop) the
// waves' epilogue staging regions followed by BM per-row floats.  The per-row
// floats are written only after the mainloop's final barrier, when every load of
// a real stage has landed (loads of stages past the end go to the sink, which
// lies beyond them).
template <class C>
struct KernLds {
  static constexpr int MAIN = RowStage<C>::UINT4;   // offset of the per-row floats
  static constexpr int STAGE_PLUS_ROWS = MAIN + C::BM / 4;
  static constexpr int TOTAL = C::LDS_UINT4 > STAGE_PLUS_ROWS ? C::LDS_UINT4 : STAGE_PLUS_ROWS;
};

// ------------------------------------------------------------------ down projection
// acc = x . A' over K = d; mode DOWN_BLOCK: h = rstd*acc, z = sigma(h);
// mode DOWN_PARTIAL: fp32 partial = acc and sumsq (tile column 0 writes it).
template <class C, bool GATEUP, bool HALF>
__device__ __forceinline__ void down_tile(const DownArgs& a, uint4* lds, int bid, int nblk, int tile0) {
  using E = typename C::E;
  float* rowss = reinterpret_cast<float*>(lds + KernLds<C>::MAIN);
  const int gr = a.g * a.r;
  constexpr int TN = GATEUP ? C::BN / 2 : C::BN;  // logical columns per tile
  const int tiles_n = ((GATEUP ? a.r : gr) + TN - 1) / TN;
  int tm, tn, m0;
  tail_tile<C, HALF>(tile0, bid, nblk, a.T, tiles_n, tm, tn, m0);
  const int n0 = tn * TN;

  Opnd oa{a.x, a.d, a.T, a.d};
  Opnd ob{a.Ap, gr, gr, a.d};
  f32x16 acc[C::MB][C::NB];
  if constexpr (GATEUP) {
    mainloop<C, false, true, true>(oa, ob, MapId{}, MapGateUp<C::WTN>{a.r}, m0, n0, 0, a.d, lds, rowss, acc);
  } else {
    mainloop<C, false, true, true>(oa, ob, MapId{}, MapId{}, m0, n0, 0, a.d, lds, rowss, acc);
  }

  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  char LR_LDS* reg = stage_region<C>(lds);
  E* h = static_cast<E*>(a.h);
  E* z = static_cast<E*>(a.z);
  // per-row sum of squares -> rstd, once per row (in place)
  for (int i = threadIdx.x; i < C::BM; i += C::THREADS) {
    const float ssv = rowss[i];
    if (a.mode == DOWN_PARTIAL) {
      if (tn == 0 && m0 + i < a.T) a.sumsq[m0 + i] = ssv;
    } else {
      const float rs = a.mode == DOWN_PLAIN ? 1.0f : __builtin_amdgcn_rsqf(ssv * a.invD + a.eps);
      rowss[i] = rs;
      if (a.rstd && tn == 0 && m0 + i < a.T) a.rstd[m0 + i] = rs;
    }
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    stage_block<C>(acc, mb, reg);
    const int rbase = m0 + wm * C::WTM + mb * 32;
    if constexpr (GATEUP) {
      sweep_block<C, C::WTN / 2>(reg, [&](int rl, int cl, const char LR_LDS* rp) {
        const int row = rbase + rl;
        const int logical = n0 + wn * (C::WTN / 2) + cl;
        if (row >= a.T || logical >= a.r) return;
        const float rs = rowss[row - m0];
        const float4 g4 = lds_f4(rp + cl * 4), u4 = lds_f4(rp + (cl + C::WTN / 2) * 4);
        const float hg[4] = {g4.x * rs, g4.y * rs, g4.z * rs, g4.w * rs};
        const float hu[4] = {u4.x * rs, u4.y * rs, u4.z * rs, u4.w * rs};
        if (h) {
          store4(h + (int64_t)row * gr + logical, hg[0], hg[1], hg[2], hg[3]);
          store4(h + (int64_t)row * gr + a.r + logical, hu[0], hu[1], hu[2], hu[3]);
        }
        store4(z + (int64_t)row * a.r + logical, hg[0] * sigmoidf_(hg[0]) * hu[0], hg[1] * sigmoidf_(hg[1]) * hu[1],
               hg[2] * sigmoidf_(hg[2]) * hu[2], hg[3] * sigmoidf_(hg[3]) * hu[3]);
      });
    } else {
      sweep_block<C, C::WTN>(reg, [&](int rl, int cl, const char LR_LDS* rp) {
        const int row = rbase + rl;
        const int col = n0 + wn * C::WTN + cl;
        if (row >= a.T || col >= gr) return;
        const float4 v = lds_f4(rp + cl * 4);
        if (a.mode == DOWN_PARTIAL) {
          store4(a.partial + (int64_t)row * gr + col, v.x, v.y, v.z, v.w);
          return;
        }
        const float rs = rowss[row - m0];
        const float hv[4] = {v.x * rs, v.y * rs, v.z * rs, v.w * rs};
        if (h) store4(h + (int64_t)row * gr + col, hv[0], hv[1], hv[2], hv[3]);
        if (a.act == ACT_SILU) {
          store4(z + (int64_t)row * gr + col, hv[0] * sigmoidf_(hv[0]), hv[1] * sigmoidf_(hv[1]),
                 hv[2] * sigmoidf_(hv[2]), hv[3] * sigmoidf_(hv[3]));
        } else if (!h) {
          store4(z + (int64_t)row * gr + col, hv[0], hv[1], hv[2], hv[3]);
        }
      });
    }
  }
}

template <class C, bool GATEUP>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_down(DownArgs a) {
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  down_tile<C, GATEUP, false>(a, lds, blockIdx.x, gridDim.x, 0);
}
// whole tiles 0 .. a.tile0-1 on the first a.tile0 work-groups, the halves of the
// rest on the others
template <class C, class H, bool GATEUP>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_down_tail(
    DownArgs a) {
  static_assert(C::THREADS == H::THREADS && C::WPE == H::WPE, "one launch shape");
  constexpr int N = KernLds<C>::TOTAL > KernLds<H>::TOTAL ? KernLds<C>::TOTAL : KernLds<H>::TOTAL;
  __shared__ uint4 lds[N];
  if ((int)blockIdx.x < a.tile0)
    down_tile<C, GATEUP, false>(a, lds, blockIdx.x, a.tile0, 0);
  else
    down_tile<H, GATEUP, true>(a, lds, blockIdx.x - a.tile0, gridDim.x - a.tile0, a.tile0);
}

// ------------------------------------------------------------------ small-rank down projection
// acc = x . A' over the split's K range; fp32 partial rows of split `split` and
// the split's partial sums of squares (column tile 0 writes them).
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_down_split(
    SplitDownArgs a) {
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  float* rowss = reinterpret_cast<float*>(lds + KernLds<C>::MAIN);
  const int tiles_m = (a.T + C::BM - 1) / C::BM, tiles_n = (a.gr + C::BN - 1) / C::BN;
  const int per_split = tiles_m * tiles_n;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int split = logical / per_split;
  int tm, tn;
  grouped_tile<kGroupM>(logical % per_split, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int kbeg = split * a.ksplit;
  const int klen = min(a.ksplit, a.d - kbeg);
  Opnd oa{a.x, a.d, a.T, a.d};     // x [T, d]
  Opnd ob{a.Apt, a.d, a.gr, a.d};  // A'^T: (n = c, k = j) at Apt[c*d + j]
  f32x16 acc[C::MB][C::NB];
  mainloop<C, false, false, true>(oa, ob, MapId{}, MapId{}, m0, n0, kbeg, klen > 0 ? klen : 0, lds, rowss, acc);

  float* part = a.partial + (int64_t)split * a.T * a.gr;
  if (tn == 0) {
    for (int i = threadIdx.x; i < C::BM; i += C::THREADS)
      if (m0 + i < a.T) a.sumsq[(int64_t)split * a.T + m0 + i] = rowss[i];
  }
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  char LR_LDS* reg = stage_region<C>(lds);
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    stage_block<C>(acc, mb, reg);
    const int rbase = m0 + wm * C::WTM + mb * 32;
    sweep_block<C, C::WTN>(reg, [&](int rl, int cl, const char LR_LDS* rp) {
      const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
      if (row >= a.T || col >= a.gr) return;
      const float4 v = lds_f4(rp + cl * 4);
      store4(part + (int64_t)row * a.gr + col, v.x, v.y, v.z, v.w);
    });
  }
}

// ------------------------------------------------------------------ up projection
// y_i = z_i . B_i (+ residual_i with RES); one launch over (branch, tile)
// the up-projection's output from the accumulator v and the epilogue input r
template <int EPI>
__device__ __forceinline__ float4 up_out(const float4& v, const float4& r) {
  if constexpr (EPI == UP_SWIGLU)
    return make_float4(r.x * sigmoidf_(r.x) * v.x, r.y * sigmoidf_(r.y) * v.y, r.z * sigmoidf_(r.z) * v.z,
                       r.w * sigmoidf_(r.w) * v.w);
  else
    return make_float4(v.x + r.x, v.y + r.y, v.z + r.z, v.w + r.w);
}

template <class C, int EPI>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_up(UpArgs a) {
  using E = typename C::E;
  constexpr bool RES = EPI != UP_PLAIN;
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  const int tiles_n = (a.d + C::BN - 1) / C::BN;
  const int tiles_m = (a.T + C::BM - 1) / C::BM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int br = logical / (tiles_m * tiles_n);
  int tm, tn;
  grouped_tile<kGroupM>(logical % (tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  Opnd oa{static_cast<const E*>(a.z) + (int64_t)br * a.r, a.ldz, a.T, a.r};
  Opnd ob{a.B[br], a.d, a.d, a.r};
  f32x16 acc[C::MB][C::NB];
  E* y = static_cast<E*>(a.y[br]);
  E* y2 = EPI == UP_SWIGLU ? static_cast<E*>(a.y2[br]) : nullptr;
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  char LR_LDS* reg = stage_region<C>(lds);
  // residual (or gate) rows of 32-row block 0 are loaded during the last k step, those of
  // block mb+1 while block mb is computed, where a block's sweep is at most 8
  // iterations (the buffers fit the registers); otherwise each block's residual
  // rows are loaded, all at once, when it is due
  constexpr bool RES_PF = RES && Sweep<C, C::WTN>::IT <= 8;
  if constexpr (RES_PF) {
    using R = Raw4<E>;
    using SW = Sweep<C, C::WTN>;
    const E* res = static_cast<const E*>(a.res[br]);
    const SW sw;
    const int col = n0 + wn * C::WTN + sw.cl;
    const bool cok = col < a.d;
    typedef typename R::T Buf[SW::IT];
    Buf r0, r1;
    auto load_block = [&](int mb, Buf& buf) {
      const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
      for (int it = 0; it < SW::IT; ++it) {
        const int row = rb + sw.rl(it);
        buf[it] = row < a.T && cok ? R::load(res + (int64_t)row * a.d + col) : R::zero();
      }
    };
    mainloop<C, false, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, a.r, lds, nullptr, acc,
                                    [&]() { load_block(0, r0); });
    auto block = [&](int mb, const Buf& cur, Buf& nxt) {
      if (mb + 1 < C::MB) load_block(mb + 1, nxt);
      stage_block<C>(acc, mb, reg);
      const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
      for (int it = 0; it < SW::IT; ++it) {
        const int rl = sw.rl(it), row = rb + rl;
        if (row >= a.T || !cok) continue;
        const float4 v = lds_f4(reg + rl * RowStage<C>::PITCH + sw.cl * 4);
        const float4 o = up_out<EPI>(v, R::f4(cur[it]));
        store4(y + (int64_t)row * a.d + col, o.x, o.y, o.z, o.w);
        if (EPI == UP_SWIGLU && y2) store4(y2 + (int64_t)row * a.d + col, v.x, v.y, v.z, v.w);
      }
    };
#pragma unroll
    for (int mb = 0; mb < C::MB; mb += 2) {
      block(mb, r0, r1);
      if (mb + 1 < C::MB) block(mb + 1, r1, r0);
    }
  } else {
    const E* res = static_cast<const E*>(a.res[br]);
    mainloop<C, false, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, a.r, lds, nullptr, acc);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      stage_block<C>(acc, mb, reg);
      const int rbase = m0 + wm * C::WTM + mb * 32;
      if constexpr (RES) {
        sweep_block_pre<C, C::WTN, 1>(
            reg,
            [&](int rl, int cl, float4* in) {
              const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
              in[0] = row < a.T && col < a.d ? load4(res + (int64_t)row * a.d + col) : make_float4(0.f, 0.f, 0.f, 0.f);
            },
            [&](int rl, int cl, const char LR_LDS* rp, const float4* in) {
              const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
              if (row >= a.T || col >= a.d) return;
              const float4 v = lds_f4(rp + cl * 4);
              const float4 o = up_out<EPI>(v, in[0]);
              store4(y + (int64_t)row * a.d + col, o.x, o.y, o.z, o.w);
              if (EPI == UP_SWIGLU && y2) store4(y2 + (int64_t)row * a.d + col, v.x, v.y, v.z, v.w);
            });
      } else {
        sweep_block<C, C::WTN>(reg, [&](int rl, int cl, const char LR_LDS* rp) {
          const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
          if (row >= a.T || col >= a.d) return;
          const float4 v = lds_f4(rp + cl * 4);
          store4(y + (int64_t)row * a.d + col, v.x, v.y, v.z, v.w);
        });
      }
    }
  }
}

// Per-row values a kernel loads at its last k step and publishes in LDS after
// the mainloop: thread tid holds rows tid, tid + THREADS, ...
template <class C>
struct RowVals {
  static constexpr int N = (C::BM + C::THREADS - 1) / C::THREADS;
  float v[N];
  template <class F>
  __device__ __forceinline__ void load(F&& f) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + j * C::THREADS;
      v[j] = i < C::BM ? f(i) : 0.f;
    }
  }
  __device__ __forceinline__ void publish(float* dst) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + j * C::THREADS;
      if (i < C::BM) dst[i] = v[j];
    }
  }
};

// ------------------------------------------------------------------ backward: dz -> dh'
// acc = dy_i . B_i^T over K = d.  Row-sweep epilogue: dh' = rstd*dz*sigma'(h),
// z = sigma(h) (SiLU/SwiGLU) and one partial of S' = sum_c dh'*h per (row, wave).
// The h rows of 32-row block mb+1 are loaded while block mb is computed; those of
// block 0 and the rows' rstd are loaded at the start of the last k step.
template <class C, int ACT, bool HALF>
__device__ __forceinline__ void dz_tile(const DzArgs& a, uint4* lds, int bid, int nblk, int tile0) {
  using E = typename C::E;
  using R = Raw4<E>;
  using SW = Sweep<C, C::WTN>;
  constexpr int NL = ACT == ACT_SWIGLU ? 2 : 1;
  // four waves: the epilogue's first loads go out in the last k step and those
  // of row block mb+1 while block mb is computed; eight (two per SIMD) have no
  // registers for that, the other wave of the SIMD covers the wait instead
  constexpr bool PF = C::NWAVES <= 4;
  float* rs_tile = reinterpret_cast<float*>(lds + KernLds<C>::MAIN);  // [BM] rstd of the tile's rows
  const int tiles_n = (a.r + C::BN - 1) / C::BN;
  // tiles of all branches in turn: branch br, then (tm, tn) within it
  int br, tm, tn, m0;
  {
    const int per = tile_rows<C, HALF>(a.T) * tiles_n;
    int t, piece;
    tail_index<HALF>(tile0, bid, nblk, t, piece);
    br = t / per;
    grouped_tile<kGroupM>(t % per, tile_rows<C, HALF>(a.T), tiles_n, tm, tn);
    m0 = (tm * (HALF ? 2 : 1) + piece) * C::BM;
  }
  const int n0 = tn * C::BN;
  const int gr = a.g * a.r;
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const SW sw;
  const int c = n0 + wn * C::WTN + sw.cl;   // rank index within the branch
  const bool cok = c < a.r;
  const E* __restrict__ h = static_cast<const E*>(a.h);
  E* __restrict__ dh = static_cast<E*>(a.dh);
  E* __restrict__ z = static_cast<E*>(a.z);
  // SwiGLU reads gate (column c) and up (column r + c); otherwise branch br's column
  const int hcol = ACT == ACT_SWIGLU ? c : br * a.r + c;

  // two buffers of h values (SwiGLU: gate in `g`, up in `u`; otherwise `u` is unused)
  typedef typename R::T Buf[SW::IT];
  Buf g0, u0, g1, u1;
  auto load_block = [&](int mb, Buf& bg, Buf& bu) {
    const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
    for (int it = 0; it < SW::IT; ++it) {
      const int row = rb + sw.rl(it);
      const bool ok = row < a.T && cok;
      const E* p = h + (int64_t)row * gr + hcol;
      bg[it] = ok ? R::load(p) : R::zero();
      if constexpr (NL == 2) bu[it] = ok ? R::load(p + a.r) : R::zero();
    }
  };
  RowVals<C> rsv;
  auto pre = [&]() {   // the row values first: they are needed first
    rsv.load([&](int i) { return m0 + i < a.T ? (a.rstd ? a.rstd[m0 + i] : 1.0f) : 0.f; });
    load_block(0, g0, u0);
  };

  Opnd oa{a.dy[br], a.d, a.T, a.d};
  Opnd ob{a.B[br], a.d, a.r, a.d};  // B_i^T: (n = c, k = j) at B_i[c*d + j]
  f32x16 acc[C::MB][C::NB];
  if constexpr (PF) {
    mainloop<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, a.d, lds, nullptr, acc, pre);
  } else {
    mainloop<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, a.d, lds, nullptr, acc);
    pre();
  }
  rsv.publish(rs_tile);
  __syncthreads();

  const int part = (br * tiles_n + tn) * C::WN + wn;
  char LR_LDS* reg = stage_region<C>(lds);
  // block mb computes from `cur` while block mb+1 loads into `nxt`
  auto block = [&](int mb, const Buf& cg, const Buf& cu, Buf& ng, Buf& nu) {
    if (PF && mb + 1 < C::MB) load_block(mb + 1, ng, nu);
    stage_block<C>(acc, mb, reg);
    const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
    for (int it = 0; it < SW::IT; ++it) {
      const int rl = sw.rl(it), row = rb + rl;
      const bool ok = row < a.T && cok;
      float srow = 0.f;
      if (ok) {
        const float4 v = lds_f4(reg + rl * RowStage<C>::PITCH + sw.cl * 4);
        const float dzv[4] = {v.x, v.y, v.z, v.w};
        const float rs = rs_tile[row - m0];
        const int64_t hidx = (int64_t)row * gr + hcol;
        if constexpr (ACT == ACT_SWIGLU) {
          const float4 g4 = R::f4(cg[it]), u4 = R::f4(cu[it]);
          const float hg[4] = {g4.x, g4.y, g4.z, g4.w}, hu[4] = {u4.x, u4.y, u4.z, u4.w};
          float dg[4], du[4], zz[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = sigmoidf_(hg[e]);
            const float sl = hg[e] * sg;
            dg[e] = rs * dzv[e] * hu[e] * sg * (1.0f + hg[e] * (1.0f - sg));
            du[e] = rs * dzv[e] * sl;
            zz[e] = sl * hu[e];
            srow += dg[e] * hg[e] + du[e] * hu[e];
          }
          store4(dh + hidx, dg[0], dg[1], dg[2], dg[3]);
          store4(dh + hidx + a.r, du[0], du[1], du[2], du[3]);
          store4(z + (int64_t)row * a.r + c, zz[0], zz[1], zz[2], zz[3]);
        } else {
          const float4 h4 = R::f4(cg[it]);
          const float hv[4] = {h4.x, h4.y, h4.z, h4.w};
          float d1[4];
          if constexpr (ACT == ACT_SILU) {
            float zz[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = sigmoidf_(hv[e]);
              d1[e] = rs * dzv[e] * sg * (1.0f + hv[e] * (1.0f - sg));
              zz[e] = hv[e] * sg;
            }
            store4(z + hidx, zz[0], zz[1], zz[2], zz[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) d1[e] = rs * dzv[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) srow += d1[e] * hv[e];
          store4(dh + hidx, d1[0], d1[1], d1[2], d1[3]);
        }
      }
      srow = row_sum<SW::LPR>(srow);
      if (a.spart && row < a.T && row_sum_lane<SW::LPR>()) a.spart[(int64_t)row * a.spstride + part] = srow;
    }
  };
  if constexpr (PF) {
#pragma unroll
    for (int mb = 0; mb < C::MB; mb += 2) {
      block(mb, g0, u0, g1, u1);
      if (mb + 1 < C::MB) block(mb + 1, g1, u1, g0, u0);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (mb > 0) load_block(mb, g0, u0);
      block(mb, g0, u0, g0, u0);
    }
  }
}

template <class C, int ACT>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_dz(DzArgs a) {
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  dz_tile<C, ACT, false>(a, lds, blockIdx.x, gridDim.x, 0);
}
// whole tiles 0 .. a.tile0-1 on the first a.tile0 work-groups, the halves of the
// rest on the others
template <class C, class H, int ACT>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_dz_tail(DzArgs a) {
  static_assert(C::THREADS == H::THREADS && C::WPE == H::WPE, "one launch shape");
  constexpr int N = KernLds<C>::TOTAL > KernLds<H>::TOTAL ? KernLds<C>::TOTAL : KernLds<H>::TOTAL;
  __shared__ uint4 lds[N];
  if ((int)blockIdx.x < a.tile0)
    dz_tile<C, ACT, false>(a, lds, blockIdx.x, a.tile0, 0);
  else
    dz_tile<H, ACT, true>(a, lds, blockIdx.x - a.tile0, gridDim.x - a.tile0, a.tile0);
}

// ------------------------------------------------------------------ backward: weight gradients
// Jobs: j < n_up: dB_j = z_j^T . dy_j ; j == n_up: M = x^T . dh'; one launch over (split, job, tile).
// Each split covers a token range; with more than one split the fp32 tile
// goes to the partial buffer [split][job-major M x N] and k_wgrad_reduce finishes.
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_wgrad(WgradArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  const int gr = a.g * a.r;
  const int tmB = (a.r + C::BM - 1) / C::BM, tnB = (a.dn + C::BN - 1) / C::BN;
  const int tmA = (a.d + C::BM - 1) / C::BM, tnA = (gr + C::BN - 1) / C::BN;
  const int per_split = a.n_up * tmB * tnB + tmA * tnA;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int split, w;
  bool slot_out = false;   // a split tile's half: writes its fp32 slot
  if (a.split_tiles > 0) {
    // per XCD (logical ranges of P ids): the first U/8 ids take whole tiles
    // S, S+1, ..., the rest the halves of tiles 0..S-1 (the long work first)
    const int S = a.split_tiles, U = per_split - S, P = (U + 2 * S) / kNumXcd;
    const int x = logical / P, i = logical % P, uw = U / kNumXcd;
    if (i < uw) {
      split = 0;
      w = S + x * uw + i;
    } else {
      const int item = x * (P - uw) + (i - uw);   // 0 .. 2S-1
      split = item / S;
      w = item % S;
      slot_out = true;
    }
  } else {
    split = logical / per_split;
    w = logical % per_split;
  }
  const int tile = w;
  const int job = w < a.n_up * tmB * tnB ? w / (tmB * tnB) : a.n_up;
  w = job < a.n_up ? w % (tmB * tnB) : w - a.n_up * tmB * tnB;
  const bool isA = job == a.n_up;
  const int M = isA ? a.d : a.r, N = isA ? gr : a.dn;
  const int tiles_m = isA ? tmA : tmB, tiles_n = isA ? tnA : tnB;
  int tm, tn;
  grouped_tile<kGroupM>(w, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const bool whole = a.split_tiles > 0 && !slot_out;
  const int kbeg = whole ? 0 : split * a.ksplit;
  const int klen = whole ? a.T : min(a.ksplit, a.T - kbeg);
  Opnd oa, ob;
  if (isA) {
    oa = Opnd{a.x, a.d, a.d, a.T};   // x^T: (m = j, k = t) at x[t*d + j]
    ob = Opnd{a.dh, gr, gr, a.T};    // dh': (n = c, k = t) at dh[t*gr + c]
  } else {
    oa = Opnd{static_cast<const E*>(a.z) + (int64_t)job * a.r, a.ldz, a.r, a.T};
    ob = Opnd{a.dy[job], a.dn, a.dn, a.T};
  }
  f32x16 acc[C::MB][C::NB];
  mainloop<C, true, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, kbeg, klen > 0 ? klen : 0, lds, nullptr, acc);

  // element (row, col) of the output goes to out[(row - r0) * ldo + col - c0]
  float* out;
  int64_t ldo = N;
  int r0 = 0, c0 = 0;
  if (slot_out) {
    out = a.wpart + ((int64_t)split * a.split_tiles + tile) * (C::BM * C::BN);
    ldo = C::BN; r0 = m0; c0 = n0;
  } else if (a.nsplit > 1 && a.split_tiles == 0) {
    out = a.wpart + (int64_t)split * a.part_stride + (isA ? a.part_offA : (int64_t)job * a.r * a.dn);
  } else {
    out = isA ? a.dA : a.dB[job];
  }
  const bool finalA = isA && (a.nsplit == 1 || a.split_tiles > 0);
  // dA = diag(gamma) M and the dgamma partials (without gamma: dA = M)
  const bool dgam = finalA && a.gamma != nullptr;
  const E* Aw = static_cast<const E*>(a.A);
  const E* gamma = static_cast<const E*>(a.gamma);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  constexpr int LPR = C::WTN / 4;
  char LR_LDS* reg = stage_region<C>(lds);
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    stage_block<C>(acc, mb, reg);
    const int rbase = m0 + wm * C::WTM + mb * 32;
    // in[0] = A row segment, in[1].x = gamma_j (final dA only)
    sweep_block_pre<C, C::WTN, 2>(
        reg,
        [&](int rl, int cl, float4* in) {
          const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
          in[0] = in[1] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (dgam && row < M && col < N) {
            in[0] = load4(Aw + (int64_t)row * gr + col);
            in[1].x = to_f32(gamma[row]);
          }
        },
        [&](int rl, int cl, const char LR_LDS* rp, const float4* in) {
          const int row = rbase + rl, col = n0 + wn * C::WTN + cl;
          float s = 0.f;
          if (row < M && col < N) {
            const float4 v = lds_f4(rp + cl * 4);
            const float gj = dgam ? in[1].x : 1.0f;
            if (dgam) s = in[0].x * v.x + in[0].y * v.y + in[0].z * v.z + in[0].w * v.w;
            store4(out + (int64_t)(row - r0) * ldo + (col - c0), gj * v.x, gj * v.y, gj * v.z, gj * v.w);
          }
          if (dgam) {
            s = row_sum<LPR>(s);
            if (row < M && row_sum_lane<LPR>()) a.gpart[(int64_t)row * a.ngpart + tn * C::WN + wn] = s;
          }
        });
  }
}

// Reductions of the weight gradients: the dB elements one thread per 4
// consecutive outputs; dA one work-group per row, which also forms
// dgamma_j = sum_c A_jc M_jc (the row's partial sums added over the work-group
// in a fixed order) and writes it, so no separate pass sums partials per row.
__device__ __forceinline__ int64_t wred_blocks_b(const WgradArgs& a) {
  return ((int64_t)a.n_up * a.r * a.dn / 4 + 255) / 256;
}
__device__ __forceinline__ float wred_block_sum(float s) {
  __shared__ float red[4];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
// dA row `row` from sum4(col) (the column's 4 summed values): dA = gamma_j * M,
// dgamma_j = sum_c A_jc M_jc
template <typename E, class F>
__device__ __forceinline__ void wred_row_a(const WgradArgs& a, int row, F&& sum4) {
  const int gr = a.g * a.r;
  const E* Aw = static_cast<const E*>(a.A);
  const bool dgam = a.gamma != nullptr;   // without gamma: dA = M, no dgamma
  const float gj = dgam ? to_f32(static_cast<const E*>(a.gamma)[row]) : 1.0f;
  float s = 0.f;
  for (int c = threadIdx.x * 4; c < gr; c += 256 * 4) {
    const float4 acc = sum4(c);
    if (dgam) {
      const float4 a4 = load4(Aw + (int64_t)row * gr + c);
      s += a4.x * acc.x + a4.y * acc.y + a4.z * acc.z + a4.w * acc.w;
    }
    *reinterpret_cast<float4*>(a.dA + (int64_t)row * gr + c) =
        make_float4(gj * acc.x, gj * acc.y, gj * acc.z, gj * acc.w);
  }
  if (dgam) {
    s = wred_block_sum(s);
    if (threadIdx.x == 0) a.dgamma[row] = s;
  }
}

// Sum the split partials in split order.  Partial element i: [0, nB) the dB
// tensors (job-major), then dA.  Work-groups [0, wred_blocks_b) take dB, one
// thread per 4 consecutive outputs; the next d take one dA row each.
template <typename E>
__global__ __launch_bounds__(256) void k_wgrad_reduce(WgradArgs a) {
  const int gr = a.g * a.r;
  const int64_t nB = (int64_t)a.n_up * a.r * a.dn;
  // the 4 outputs from element i, the split partials added in split order (up
  // to U loads in flight)
  auto sum4 = [&](int64_t i) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int U = 8;
    for (int s0 = 0; s0 < a.nsplit; s0 += U) {
      float4 p[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        p[u] = s0 + u < a.nsplit ? *reinterpret_cast<const float4*>(a.wpart + (int64_t)(s0 + u) * a.part_stride + i)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u >= a.nsplit) break;
        acc.x += p[u].x; acc.y += p[u].y; acc.z += p[u].z; acc.w += p[u].w;
      }
    }
    return acc;
  };
  const int64_t nbb = wred_blocks_b(a);
  if ((int64_t)blockIdx.x < nbb) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= nB) return;
    const int job = (int)(i / ((int64_t)a.r * a.dn));
    const int64_t k = i % ((int64_t)a.r * a.dn);
    *reinterpret_cast<float4*>(a.dB[job] + k) = sum4(i);
    return;
  }
  const int row = (int)((int64_t)blockIdx.x - nbb);
  wred_row_a<E>(a, row, [&](int c) { return sum4(nB + (int64_t)row * gr + c); });
}

// Sum of the two halves of each split tile (k_wgrad with split_tiles > 0): one
// thread per 4 consecutive slot values, the halves added in order, written to
// the tile's place in dB (split tiles are dB tiles).  With gamma, the work-groups
// past the tiles' also form dgamma_j from the row partials the whole dA tiles
// left (one thread per row, the partials added in column order), so that no
// separate launch sums them.
template <class C>
__global__ __launch_bounds__(256) void k_wgrad_reduce_tiles(WgradArgs a) {
  constexpr int TS = C::BM * C::BN;
  const int64_t ntb = ((int64_t)a.split_tiles * TS / 4 + 255) / 256;
  if ((int64_t)blockIdx.x >= ntb) {
    const int j = (int)(((int64_t)blockIdx.x - ntb) * 256 + threadIdx.x);
    if (j >= a.d) return;
    const float* p = a.gpart + (int64_t)j * a.ngpart;
    float s = 0.f;
    for (int k = 0; k < a.gparts_used; ++k) s += p[k];
    a.dgamma[j] = s;
    return;
  }
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)a.split_tiles * TS) return;
  const int tile = (int)(i / TS), loc = (int)(i % TS);
  const int tmB = (a.r + C::BM - 1) / C::BM, tnB = (a.dn + C::BN - 1) / C::BN;
  const int job = tile / (tmB * tnB);
  int tm, tn;
  grouped_tile<kGroupM>(tile % (tmB * tnB), tmB, tnB, tm, tn);
  const int row = tm * C::BM + loc / C::BN, col = tn * C::BN + loc % C::BN;
  if (row >= a.r || col >= a.dn) return;
  const float4 p0 = *reinterpret_cast<const float4*>(a.wpart + i);
  const float4 p1 = *reinterpret_cast<const float4*>(a.wpart + (int64_t)a.split_tiles * TS + i);
  *reinterpret_cast<float4*>(a.dB[job] + (int64_t)row * a.dn + col) =
      make_float4(p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w);
}

// Stream-K weight gradients.  Tiles are numbered job-major (dB_0 .. dB_{n_up-1},
// dA), row-major within a job; work-group w covers the k steps [s_w, s_w + len_w)
// of the concatenated (tile, k step) sequence and writes one fp32 slot per tile
// it touches.  k_wgrad_sk_reduce sums each tile's slots in work-group order.
__device__ __forceinline__ int sk_owner(int64_t q, int Q, int R) {
  const int64_t big = (int64_t)R * (Q + 1);
  return q < big ? (int)(q / (Q + 1)) : (int)(R + (q - big) / Q);
}

// The tile at sequence position p, and the position of tile t.  Work-groups w,
// w+8, ... share an XCD (ids are dealt to the 8 XCDs in turn); when they sit S
// tiles apart in the sequence and start at one k offset, the interleave puts the
// tiles they run concurrently into one contiguous block of the tile order, whose
// operand panels the XCD's L2 then shares for the token rows they stream.
__device__ __forceinline__ int sk_tile_at(int p, int S, int tiles) {
  const int n = tiles / S;
  return (p % S) * n + p / S;
}
__device__ __forceinline__ int sk_pos_of(int t, int S, int tiles) {
  const int n = tiles / S;
  return (t % n) * S + t / n;
}

struct SkTile {
  int job, tm, tn, M, N;
};
template <class C>
__device__ __forceinline__ SkTile sk_tile(const WgradArgs& a, int t) {
  const int gr = a.g * a.r;
  const int tmB = (a.r + C::BM - 1) / C::BM, tnB = (a.dn + C::BN - 1) / C::BN;
  const int tnA = (gr + C::BN - 1) / C::BN;
  SkTile s;
  const int nB = a.n_up * tmB * tnB;
  if (t < nB) {
    s.job = t / (tmB * tnB);
    const int w = t % (tmB * tnB);
    s.tm = w / tnB; s.tn = w % tnB; s.M = a.r; s.N = a.dn;
  } else {
    const int w = t - nB;
    s.job = a.n_up; s.tm = w / tnA; s.tn = w % tnA; s.M = a.d; s.N = gr;
  }
  return s;
}

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_wgrad_sk(
    WgradArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  const int gr = a.g * a.r;
  // No XCD renumbering: the hardware deals ids to the 8 XCDs in turn, and work-groups
  // w, w+8, ... start at the same k offset within their tiles, so an XCD's L2 holds
  // the same token rows for all of its tiles.
  const int w = blockIdx.x;
  const int64_t s0 = (int64_t)w * a.sk_Q + min(w, a.sk_R);
  const int64_t s1 = s0 + a.sk_Q + (w < a.sk_R ? 1 : 0);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  for (int64_t cur = s0; cur < s1;) {
    const int t = (int)(cur / a.sk_KS);   // sequence position
    const int64_t tend = min(s1, (int64_t)(t + 1) * a.sk_KS);
    const int kk0 = (int)(cur - (int64_t)t * a.sk_KS), kk1 = (int)(tend - (int64_t)t * a.sk_KS);
    const int ord = w - sk_owner((int64_t)t * a.sk_KS, a.sk_Q, a.sk_R);
    const SkTile st = sk_tile<C>(a, sk_tile_at(t, a.sk_S, a.sk_tiles));
    const int m0 = st.tm * C::BM, n0 = st.tn * C::BN;
    const int kbeg = kk0 * C::BK;
    const int klen = min(kk1 * C::BK, a.T) - kbeg;
    Opnd oa, ob;
    if (st.job == a.n_up) {
      oa = Opnd{a.x, a.d, a.d, a.T};   // x^T: (m = j, k = t) at x[t*d + j]
      ob = Opnd{a.dh, gr, gr, a.T};    // dh': (n = c, k = t) at dh[t*gr + c]
    } else {
      oa = Opnd{static_cast<const E*>(a.z) + (int64_t)st.job * a.r, a.ldz, a.r, a.T};
      ob = Opnd{a.dy[st.job], a.dn, a.dn, a.T};
    }
    __syncthreads();   // the previous segment's epilogue is done with LDS
    f32x16 acc[C::MB][C::NB];
    mainloop<C, true, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, kbeg, klen > 0 ? klen : 0, lds, nullptr, acc);
    float* slot = a.wpart + ((int64_t)t * a.sk_maxseg + ord) * (C::BM * C::BN);
    char LR_LDS* reg = stage_region<C>(lds);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      stage_block<C>(acc, mb, reg);
      const int rl0 = wm * C::WTM + mb * 32;
      sweep_block<C, C::WTN>(reg, [&](int rl, int cl, const char LR_LDS* rp) {
        const int lr_ = rl0 + rl, lc = wn * C::WTN + cl;
        if (m0 + lr_ >= st.M || n0 + lc >= st.N) return;
        const float4 v = lds_f4(rp + cl * 4);
        store4(slot + (int64_t)lr_ * C::BN + lc, v.x, v.y, v.z, v.w);
      });
    }
    cur = tend;
  }
}

// Sum of each tile's stream-K slots in work-group order.  Work-groups
// [0, wred_blocks_b) take the dB tensors (job-major), one thread per 4
// consecutive outputs; the next d take one dA row each.
template <class C>
__global__ __launch_bounds__(256) void k_wgrad_sk_reduce(WgradArgs a) {
  using E = typename C::E;
  const int gr = a.g * a.r;
  const int64_t nB = (int64_t)a.n_up * a.r * a.dn;
  // the 4 outputs at (job, row, col): the slots of the covering work-groups
  auto sum4 = [&](int job, int row, int col) {
    const int tmB = (a.r + C::BM - 1) / C::BM, tnB = (a.dn + C::BN - 1) / C::BN;
    const int tnA = (gr + C::BN - 1) / C::BN;
    const int tm = row / C::BM, tn = col / C::BN;
    const int t = sk_pos_of(job < a.n_up ? job * tmB * tnB + tm * tnB + tn : a.n_up * tmB * tnB + tm * tnA + tn,
                            a.sk_S, a.sk_tiles);
    const int first = sk_owner((int64_t)t * a.sk_KS, a.sk_Q, a.sk_R);
    const int last = sk_owner((int64_t)(t + 1) * a.sk_KS - 1, a.sk_Q, a.sk_R);
    const float* slot = a.wpart + (int64_t)t * a.sk_maxseg * (C::BM * C::BN) +
                        (int64_t)(row - tm * C::BM) * C::BN + (col - tn * C::BN);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j <= last - first; ++j) {
      const float4 p = *reinterpret_cast<const float4*>(slot + (int64_t)j * (C::BM * C::BN));
      acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    return acc;
  };
  const int64_t nbb = wred_blocks_b(a);
  if ((int64_t)blockIdx.x < nbb) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= nB) return;
    const int job = (int)(i / ((int64_t)a.r * a.dn));
    const int64_t k = i % ((int64_t)a.r * a.dn);
    const int row = (int)(k / a.dn), col = (int)(k % a.dn);
    *reinterpret_cast<float4*>(a.dB[job] + (int64_t)row * a.dn + col) = sum4(job, row, col);
    return;
  }
  const int row = (int)((int64_t)blockIdx.x - nbb);
  wred_row_a<E>(a, row, [&](int c) { return sum4(a.n_up, row, c); });
}

// rstd * S' / D of a tile's rows, one row per thread.  The S' partials of the
// row are issued as float4 loads at the start of the last k step and summed (in
// column order) after the mainloop, so that no load is waited for inside it;
// partials past the first 4*Q are read after the mainloop.
template <class C>
struct SprimeRows {
  static constexpr int N = (C::BM + C::THREADS - 1) / C::THREADS;
  static constexpr int Q = 8;
  float4 q[N][Q];
  float rs[N];
  __device__ __forceinline__ void load(const DxArgs& a, int m0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + j * C::THREADS, t = m0 + i;
      const bool ok = i < C::BM && t < a.T;
      rs[j] = ok ? a.rstd[t] * a.invD : 0.f;
      const float4* p = reinterpret_cast<const float4*>(a.spart + (int64_t)(ok ? t : 0) * a.spstride);
#pragma unroll
      for (int k = 0; k < Q; ++k) q[j][k] = ok && 4 * k < a.nspart ? p[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void publish(const DxArgs& a, int m0, float* dst) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = threadIdx.x + j * C::THREADS, t = m0 + i;
      if (i >= C::BM) continue;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < Q; ++k) {
        const int b = 4 * k;
        sum += b < a.nspart ? q[j][k].x : 0.f;
        sum += b + 1 < a.nspart ? q[j][k].y : 0.f;
        sum += b + 2 < a.nspart ? q[j][k].z : 0.f;
        sum += b + 3 < a.nspart ? q[j][k].w : 0.f;
      }
      if (t < a.T)
        for (int k = 4 * Q; k < a.nspart; ++k) sum += a.spart[(int64_t)t * a.spstride + k];
      dst[i] = t < a.T ? sum * rs[j] : 0.f;
    }
  }
};

// ------------------------------------------------------------------ backward: dx
// acc = dh' . A^T over K = g*r.  Row-sweep epilogue: dx = gamma*acc - x*rstd*S'/D
// (+ dres with DX_NORM_RES), with S' summed from the dz partials.  x (and dres)
// rows of block mb+1 are loaded while block mb is computed; block 0, gamma and
// the row statistic at the last k step.
// DX_SWIGLU: acc is the gradient ds of s = SiLU(gate) * up; the epilogue reads
// gate (in x's place) and up (in dres's) and writes dgate = ds * up * SiLU'(gate)
// to dx and dup = ds * SiLU(gate) to dx2.
template <class C, int MODE>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void k_dx(DxArgs a) {
  using E = typename C::E;
  constexpr bool RES = MODE != DX_NORM;   // a second row input (dres, or up)
  using R = Raw4<E>;
  using SW = Sweep<C, C::WTN>;
  constexpr bool PF = C::NWAVES <= 4;  // prefetch of the next row block's x (see dz)
  __shared__ uint4 lds[KernLds<C>::TOTAL];
  float* srow = reinterpret_cast<float*>(lds + KernLds<C>::MAIN);  // [BM] : rstd*S'/D
  const int gr = a.g * a.r;
  const int tiles_n = (a.d + C::BN - 1) / C::BN;
  const int tiles_m = (a.T + C::BM - 1) / C::BM;
  int tm, tn;
  grouped_tile<kGroupM>(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const SW sw;
  const int col = n0 + wn * C::WTN + sw.cl;
  const bool cok = col < a.d;
  const E* __restrict__ x = static_cast<const E*>(a.x);
  const E* dres = static_cast<const E*>(a.dres);
  E* dx = static_cast<E*>(a.dx);
  E* dx2 = static_cast<E*>(a.dx2);

  // x rows, then (RES) the dres rows: buf[it] and buf[SW::IT + it]
  constexpr int NBUF = RES ? 2 * SW::IT : SW::IT;
  typename R::T xin0[NBUF], xin1[NBUF];
  auto load_block = [&](int mb, typename R::T (&buf)[NBUF]) {
    const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
    for (int it = 0; it < SW::IT; ++it) {
      const int row = rb + sw.rl(it);
      buf[it] = row < a.T && cok ? R::load(x + (int64_t)row * a.d + col) : R::zero();
      if constexpr (RES) buf[SW::IT + it] = row < a.T && cok ? R::load(dres + (int64_t)row * a.d + col) : R::zero();
    }
  };
  typename R::T graw = R::zero();
  SprimeRows<C> srv;
  auto pre = [&]() {   // the row values first: they are needed first
    if constexpr (MODE != DX_SWIGLU) {
      srv.load(a, m0);
      graw = cok ? R::load(static_cast<const E*>(a.gamma) + col) : R::zero();
    }
    load_block(0, xin0);
  };

  Opnd oa{a.dh, gr, a.T, gr};   // dh' [T, gr]
  Opnd ob{a.A, gr, a.d, gr};    // A^T: (n = j, k = c) at A[j*gr + c]
  f32x16 acc[C::MB][C::NB];
  if constexpr (PF) {
    mainloop<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, gr, lds, nullptr, acc, pre);
  } else {
    mainloop<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, 0, gr, lds, nullptr, acc);
    pre();
  }
  if constexpr (MODE != DX_SWIGLU) srv.publish(a, m0, srow);
  __syncthreads();

  const float4 g4 = R::f4(graw);
  char LR_LDS* reg = stage_region<C>(lds);
  // block mb computes from `cur` while block mb+1 loads into `nxt`
  auto block = [&](int mb, const typename R::T (&cur)[NBUF], typename R::T (&nxt)[NBUF]) {
    if (PF && mb + 1 < C::MB) load_block(mb + 1, nxt);
    stage_block<C>(acc, mb, reg);
    const int rb = m0 + wm * C::WTM + mb * 32;
#pragma unroll
    for (int it = 0; it < SW::IT; ++it) {
      const int rl = sw.rl(it), row = rb + rl;
      if (row >= a.T || !cok) continue;
      const float4 v = lds_f4(reg + rl * RowStage<C>::PITCH + sw.cl * 4);
      const float4 x4 = R::f4(cur[it]);
      if constexpr (MODE == DX_SWIGLU) {
        const float4 u4 = R::f4(cur[SW::IT + it]);
        const float ds[4] = {v.x, v.y, v.z, v.w}, gv[4] = {x4.x, x4.y, x4.z, x4.w}, uv[4] = {u4.x, u4.y, u4.z, u4.w};
        float dg[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = sigmoidf_(gv[e]);
          dg[e] = ds[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
          du[e] = ds[e] * gv[e] * sg;
        }
        store4(dx + (int64_t)row * a.d + col, dg[0], dg[1], dg[2], dg[3]);
        store4(dx2 + (int64_t)row * a.d + col, du[0], du[1], du[2], du[3]);
        continue;
      }
      const float sr = srow[row - m0];
      float4 o = make_float4(g4.x * v.x - x4.x * sr, g4.y * v.y - x4.y * sr, g4.z * v.z - x4.z * sr,
                             g4.w * v.w - x4.w * sr);
      if constexpr (RES) {
        const float4 r4 = R::f4(cur[SW::IT + it]);
        o.x += r4.x; o.y += r4.y; o.z += r4.z; o.w += r4.w;
      }
      store4(dx + (int64_t)row * a.d + col, o.x, o.y, o.z, o.w);
    }
  };
  if constexpr (PF) {
#pragma unroll
    for (int mb = 0; mb < C::MB; mb += 2) {
      block(mb, xin0, xin1);
      if (mb + 1 < C::MB) block(mb + 1, xin1, xin0);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (mb > 0) load_block(mb, xin0);
      block(mb, xin0, xin0);
    }
  }
}

// ------------------------------------------------------------------ launchers

template <typename E>
struct Cfgs;
template <>
struct Cfgs<bf16> {
  using Main = PipeCfg<256, 256, 64, 2, 2, 2>;
  // 64-row tiles for a down-projection whose 256 x 256 grid would leave CUs idle
  // (small g*r): four waves side by side over 256 columns
  using Skinny = PipeCfg<64, 256, 64, 1, 4, 2>;
  // small-rank split-K down-projection: 256 rows by 64 or 128 columns, waves stacked in M
  using N64 = PipeCfg<256, 64, 64, 4, 1, 3>;
  using N128 = PipeCfg<256, 128, 32, 4, 1, 4>;
  using N256 = PipeCfg<256, 256, 32, 2, 2, 4>;
  // short-K up-projection: 128 x 256 tiles, two work-groups per CU, so that one
  // group's stores overlap the other's loads and MFMAs
  using UpShort = PipeCfg<128, 256, 32, 2, 2, 2, 2>;
  // up-projection: eight waves (two per SIMD, 128 x 64 each, accumulators in
  // VGPRs), so that one wave's load issue overlaps the other's MFMAs
  using Up = PipeCfg<256, 256, 64, 2, 4, 2, 2>;
  // 128-row halves of the main tiles, for the last round of a grid (see tail_tile)
  using Half = PipeCfg<128, 256, 64, 2, 2, 2>;
  // down-projection: eight waves (two per SIMD, 64 x 128 each, accumulators in
  // VGPRs), so that one wave's load issue overlaps the other's MFMAs
  using Down = PipeCfg<256, 256, 64, 4, 2, 2, 2>;
  using DownHalf = PipeCfg<128, 256, 64, 4, 2, 2, 2>;
  using Wgrad = Main;
  // dz and dx: eight waves as the down-projection
  using Dz = Down;
  using Dx = Down;
  static constexpr bool HAS_SKINNY = true;
};
template <>
struct Cfgs<float> {
  using Main = TileCfg<float, 128, 128, 2, 2>;
  using Skinny = Main;
  using N64 = Main;
  using N128 = Main;
  using N256 = Main;
  using UpShort = Main;
  using Up = Main;
  using Half = Main;
  using Down = Main;
  using DownHalf = Main;
  using Wgrad = Main;
  using Dz = Main;
  using Dx = Main;
  static constexpr bool HAS_SKINNY = false;
};


constexpr int kNumCu = 256;
constexpr int kUpShortK = 256;   // up-projections with K = r up to this use UpShort tiles

// The skinny down tiles are used when the 256 x 256 grid has fewer tiles than CUs.
template <typename E>
bool down_uses_skinny(int T, int r, int g, bool gateup) {
  if (!Cfgs<E>::HAS_SKINNY) return false;
  using C = typename Cfgs<E>::Main;
  const int tiles = ((T + C::BM - 1) / C::BM) * (gateup ? (2 * r + C::BN - 1) / C::BN : (g * r + C::BN - 1) / C::BN);
  return tiles < kNumCu;
}
template bool down_uses_skinny<bf16>(int, int, int, bool);
template bool down_uses_skinny<float>(int, int, int, bool);

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Tiles of a grid of `tiles` main tiles that run whole: all of them, unless the
// last round would occupy at most half of the CUs; then only the full rounds (the
// rest runs as 128-row halves, one round).
// the 128-row half configuration of a 256-row tile configuration (void: none)
template <class C>
struct HalfOf {
  using type = void;
};
template <>
struct HalfOf<Cfgs<bf16>::Main> {
  using type = Cfgs<bf16>::Half;
};
template <>
struct HalfOf<Cfgs<bf16>::Down> {
  using type = Cfgs<bf16>::DownHalf;
};
template <class C>
constexpr bool kHasHalf = !std::is_void<typename HalfOf<C>::type>::value;
template <typename E, class C>
int tail_full_tiles(int tiles) {
  if constexpr (!kHasHalf<C>) {
    return tiles;
  } else {
    const int rem = tiles % kNumCu;
    return rem > 0 && 2 * rem <= kNumCu ? tiles - rem : tiles;
  }
}

template <typename E>
hipError_t launch_rms_stats(const void* x, const void* gamma, void* y, float* sumsq, float* rstd, int T, int d,
                            float invD, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rms_stats<E>, dim3(cdiv(T, 4)), dim3(256), 0, s, static_cast<const E*>(x),
                     static_cast<const E*>(gamma), static_cast<E*>(y), sumsq, rstd, T, d, invD, eps);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_fold_gamma(const void* A, const void* gamma, void* Ap, int d, int n, hipStream_t s) {
  constexpr int VEC = 16 / (int)sizeof(E);
  const int64_t total = (int64_t)d * n / VEC;
  hipLaunchKernelGGL(k_fold_gamma<E>, dim3(cdiv(total, 256)), dim3(256), 0, s, static_cast<const E*>(A),
                     static_cast<const E*>(gamma), static_cast<E*>(Ap), d, n);
  return hipGetLastError();
}

template <class C>
hipError_t launch_down_cfg(const DownArgs& a0, hipStream_t s) {
  const bool gateup = a0.act == ACT_SWIGLU && a0.mode == DOWN_BLOCK;
  const int tiles = cdiv(a0.T, C::BM) * (gateup ? cdiv(a0.r, C::BN / 2) : cdiv(a0.g * a0.r, C::BN));
  DownArgs a = a0;
  a.tile0 = tail_full_tiles<typename C::E, C>(tiles);
  if constexpr (kHasHalf<C>) {
    if (a.tile0 < tiles) {  // full rounds of whole tiles, then the rest in halves
      using H = typename HalfOf<C>::type;
      const int grid = a.tile0 + 2 * (tiles - a.tile0);
      if (gateup)
        hipLaunchKernelGGL((k_down_tail<C, H, true>), dim3(grid), dim3(C::THREADS), 0, s, a);
      else
        hipLaunchKernelGGL((k_down_tail<C, H, false>), dim3(grid), dim3(C::THREADS), 0, s, a);
      return hipGetLastError();
    }
  }
  if (gateup) {
    hipLaunchKernelGGL((k_down<C, true>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_down<C, false>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Down;
  if (a.T == 0) return hipSuccess;
  if constexpr (Cfgs<E>::HAS_SKINNY) {
    if (down_uses_skinny<E>(a.T, a.r, a.g, a.act == ACT_SWIGLU && a.mode == DOWN_BLOCK))
      return launch_down_cfg<typename Cfgs<E>::Skinny>(a, s);
  }
  return launch_down_cfg<C>(a, s);
}

template <class C>
hipError_t launch_up_cfg(const UpArgs& a, int n_up, hipStream_t s) {
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.d, C::BN);
  if (a.res[0] && a.swiglu)
    hipLaunchKernelGGL((k_up<C, UP_SWIGLU>), dim3(tiles * n_up), dim3(C::THREADS), 0, s, a);
  else if (a.res[0])
    hipLaunchKernelGGL((k_up<C, UP_RES>), dim3(tiles * n_up), dim3(C::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_up<C, UP_PLAIN>), dim3(tiles * n_up), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_up(const UpArgs& a, int n_up, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if constexpr (Cfgs<E>::HAS_SKINNY) {
    if (a.r <= kUpShortK) return launch_up_cfg<typename Cfgs<E>::UpShort>(a, n_up, s);
  }
  return launch_up_cfg<typename Cfgs<E>::Up>(a, n_up, s);
}

template <typename E>
hipError_t launch_fold_gamma_t(const void* A, const void* gamma, void* Apt, int d, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_fold_gamma_t<E>, dim3(d / 64, n / 16), dim3(256), 0, s, static_cast<const E*>(A),
                     static_cast<const E*>(gamma), static_cast<E*>(Apt), d, n);
  return hipGetLastError();
}

// The split-K path serves g*r <= 256 when the regular down-projection would have
// fewer 256 x 256 tiles than CUs; the splits bring the work-groups to about one
// per CU, each split covering whole k steps.
template <typename E>
int small_rank_splits(int T, int d, int r, int g, int act) {
  if (!Cfgs<E>::HAS_SKINNY || g * r > 256 || T <= 0) return 0;
  if (!down_uses_skinny<E>(T, r, g, act == ACT_SWIGLU)) return 0;
  using C = typename Cfgs<E>::Main;
  const int tiles = cdiv(T, C::BM);
  const int ksteps = cdiv(d, C::BK);
  int ns = cdiv(kNumCu, tiles);
  return ns < 1 ? 1 : (ns > ksteps ? ksteps : ns);
}

template <class C>
hipError_t launch_down_split_cfg(const SplitDownArgs& a, hipStream_t s) {
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.gr, C::BN) * a.nsplit;
  hipLaunchKernelGGL((k_down_split<C>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_down_split(const SplitDownArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if constexpr (Cfgs<E>::HAS_SKINNY) {
    if (a.gr <= 64) return launch_down_split_cfg<typename Cfgs<E>::N64>(a, s);
    if (a.gr <= 128) return launch_down_split_cfg<typename Cfgs<E>::N128>(a, s);
    return launch_down_split_cfg<typename Cfgs<E>::N256>(a, s);
  } else {
    return hipErrorInvalidValue;  // the fp32 path has no split-K down-projection
  }
}

template <typename E>
hipError_t launch_finish(const float* partial, const float* sumsq, void* h, void* z, float* rstd, int T, int r,
                         int g, int act, float invD, float eps, int nsplit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int ncols = act == ACT_SWIGLU ? r : g * r;
  hipLaunchKernelGGL(k_finish<E>, dim3(cdiv((int64_t)T * (ncols / 4), 256)), dim3(256), 0, s, partial, sumsq,
                     static_cast<E*>(h), static_cast<E*>(z), rstd, T, r, g, act, invD, eps, nsplit);
  return hipGetLastError();
}

template <typename E>
int dz_nparts(int r) {
  using C = typename Cfgs<E>::Dz;
  return cdiv(r, C::BN) * C::WN;
}
template <typename E>
int gemm_bk() {
  return Cfgs<E>::Main::BK;
}
template int gemm_bk<bf16>();
template int gemm_bk<float>();

template <typename E>
int wgrad_nparts_used(int gr, bool reduced) {
  using C = typename Cfgs<E>::Wgrad;
  return reduced ? gr / 64 : cdiv(gr, C::BN) * C::WN;
}
template int wgrad_nparts_used<bf16>(int, bool);
template int wgrad_nparts_used<float>(int, bool);

template <typename E>
int wgrad_nparts(int gr) {
  // one partial per (column tile, wave column) without splits, one per 64 columns with
  using C = typename Cfgs<E>::Wgrad;
  const int a = cdiv(gr, C::BN) * C::WN, b = gr / 64;
  return a > b ? a : b;
}

template <typename E>
hipError_t launch_dz(const DzArgs& a, int n_up, hipStream_t s) {
  using C = typename Cfgs<E>::Dz;
  if (a.T == 0) return hipSuccess;
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.r, C::BN) * n_up;
  DzArgs b = a;
  b.tile0 = tail_full_tiles<E, C>(tiles);
  if constexpr (kHasHalf<C>) {
    if (b.tile0 < tiles) {  // full rounds of whole tiles, then the rest in halves
      using H = typename HalfOf<C>::type;
      const int grid = b.tile0 + 2 * (tiles - b.tile0);
      if (a.act == ACT_SWIGLU)
        hipLaunchKernelGGL((k_dz_tail<C, H, ACT_SWIGLU>), dim3(grid), dim3(C::THREADS), 0, s, b);
      else if (a.act == ACT_SILU)
        hipLaunchKernelGGL((k_dz_tail<C, H, ACT_SILU>), dim3(grid), dim3(C::THREADS), 0, s, b);
      else
        hipLaunchKernelGGL((k_dz_tail<C, H, ACT_IDENTITY>), dim3(grid), dim3(C::THREADS), 0, s, b);
      return hipGetLastError();
    }
  }
  if (a.act == ACT_SWIGLU) {
    hipLaunchKernelGGL((k_dz<C, ACT_SWIGLU>), dim3(tiles), dim3(C::THREADS), 0, s, b);
  } else if (a.act == ACT_SILU) {
    hipLaunchKernelGGL((k_dz<C, ACT_SILU>), dim3(tiles), dim3(C::THREADS), 0, s, b);
  } else {
    hipLaunchKernelGGL((k_dz<C, ACT_IDENTITY>), dim3(tiles), dim3(C::THREADS), 0, s, b);
  }
  return hipGetLastError();
}

template <typename E>
WgradPlan wgrad_plan(int T, int d, int r, int g, int n_up, int dn) {
  using C = typename Cfgs<E>::Wgrad;
  const int gr = g * r;
  WgradPlan p{};
  p.S = 1;
  p.tiles = n_up * cdiv(r, C::BM) * cdiv(dn, C::BN) + cdiv(d, C::BM) * cdiv(gr, C::BN);
  p.KS = cdiv(T, C::BK);
  const int64_t total = (int64_t)p.tiles * p.KS;
  p.nsplit = 1;
  // Nearly one round of whole tiles (7/8 of the CUs or more): one token pass.
  // Stream-K would spread the few idle CUs' share over every tile at the price
  // of fp32 slots and a reduction (236 tiles: 578 + 35 us against ~450).
  if (p.tiles <= kNumCu && 8 * p.tiles >= 7 * kNumCu) return p;
  if (Cfgs<E>::HAS_SKINNY && p.tiles < kNumCu && total >= 2 * kNumCu) {
    // stream-K: about one work-group per CU, at least 8 k steps each
    p.streamk = 1;
    p.G = (int)(total / 8 < kNumCu ? total / 8 : kNumCu);
    p.Q = (int)(total / p.G);
    p.R = (int)(total % p.G);
    // interleave S: with R == 0, work-groups w and w+8 (one XCD) start 8Q steps
    // apart, S = 8Q / KS whole tiles when that divides, and tiles == S * G / 8
    p.S = 1;
    if (p.R == 0 && p.G % 8 == 0 && (8 * (int64_t)p.Q) % p.KS == 0) p.S = (int)(8 * (int64_t)p.Q / p.KS);
    if (p.S < 1 || p.tiles % p.S != 0) p.S = 1;
    p.maxseg = 0;
    for (int t = 0; t < p.tiles; ++t) {
      const int64_t q0 = (int64_t)t * p.KS, q1 = q0 + p.KS - 1;
      auto owner = [&](int64_t q) {
        const int64_t big = (int64_t)p.R * (p.Q + 1);
        return q < big ? (int)(q / (p.Q + 1)) : (int)(p.R + (q - big) / p.Q);
      };
      const int n = owner(q1) - owner(q0) + 1;
      p.maxseg = n > p.maxseg ? n : p.maxseg;
    }
    p.part_floats = (int64_t)p.tiles * p.maxseg * C::BM * C::BN;
    return p;
  }
  // Between one and two rounds of whole tiles: split just enough (dB) tiles in
  // two that the work-groups fill exactly two rounds, the whole tiles first
  // (one tile-time) and then the halves (half a tile-time), instead of
  // splitting every tile and reducing all of dA and dB.  Only when the whole
  // tiles fit in the first round (up to 1.5 rounds of tiles): beyond that the
  // second round holds whole tiles too, and the split saves nothing.
  {
    const int S = 2 * kNumCu - p.tiles, U = p.tiles - S;
    const int tilesB = n_up * cdiv(r, C::BM) * cdiv(dn, C::BN);
    if (Cfgs<E>::HAS_SKINNY && p.tiles > kNumCu && S > 0 && S <= tilesB && U <= kNumCu && U % kNumXcd == 0 &&
        (2 * S) % kNumXcd == 0 && p.KS >= 32) {
      p.nsplit = 2;
      p.split_tiles = S;
      p.part_floats = (int64_t)2 * S * C::BM * C::BN;
      return p;
    }
  }
  // token splits: aim for at least two waves of work-groups on 256 CUs, with
  // >= 16 k steps per split, as long as doubling the splits shortens the
  // schedule (rounds of work-groups times the split's share of a tile)
  auto tile_times = [&](int sp) { return (double)cdiv((int64_t)p.tiles * sp, kNumCu) / sp; };
  int sp = 1;
  while (p.tiles * sp < 2 * kNumCu && p.KS / (2 * sp) >= 16 && sp < 16 && tile_times(2 * sp) < tile_times(sp))
    sp *= 2;
  p.nsplit = sp;
  p.part_floats = sp > 1 ? (int64_t)sp * ((int64_t)n_up * r * dn + (int64_t)d * gr) : 0;
  return p;
}

template <typename E>
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Wgrad;
  const int gr = a.g * a.r;
  const int tilesB = cdiv(a.r, C::BM) * cdiv(a.dn, C::BN);
  const int tilesA = cdiv(a.d, C::BM) * cdiv(gr, C::BN);
  const int total = a.split_tiles > 0 ? a.n_up * tilesB + tilesA + a.split_tiles
                                     : (a.n_up * tilesB + tilesA) * a.nsplit;
  if constexpr (Cfgs<E>::HAS_SKINNY) {
    if (a.streamk) {
      hipLaunchKernelGGL((k_wgrad_sk<C>), dim3(a.sk_G), dim3(C::THREADS), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_wgrad<C>), dim3(total), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_wgrad_reduce(const WgradArgs& a, hipStream_t s) {
  // dB work-groups (one thread per 4 outputs), then one work-group per dA row
  const int64_t blocks = cdiv((int64_t)a.n_up * a.r * a.dn / 4, 256) + a.d;
  if constexpr (Cfgs<E>::HAS_SKINNY) {
    if (a.streamk) {
      hipLaunchKernelGGL((k_wgrad_sk_reduce<typename Cfgs<E>::Wgrad>), dim3(blocks), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.nsplit == 1) return hipSuccess;
  if (a.split_tiles > 0) {
    using C = typename Cfgs<E>::Wgrad;
    const int64_t n4 = (int64_t)a.split_tiles * C::BM * C::BN / 4;
    const int64_t gblocks = a.gamma ? cdiv(a.d, 256) : 0;   // dgamma rows (see the kernel)
    hipLaunchKernelGGL((k_wgrad_reduce_tiles<C>), dim3(cdiv(n4, 256) + gblocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_wgrad_reduce<E>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_dx(const DxArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Dx;
  if (a.T == 0) return hipSuccess;
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.d, C::BN);
  if (a.swiglu)
    hipLaunchKernelGGL((k_dx<C, DX_SWIGLU>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  else if (a.dres)
    hipLaunchKernelGGL((k_dx<C, DX_NORM_RES>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_dx<C, DX_NORM>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, float* out, int n, int nparts, int stride, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_parts, dim3(cdiv(n, 256)), dim3(256), 0, s, parts, out, n, nparts, stride);
  return hipGetLastError();
}

template hipError_t launch_rms_stats<bf16>(const void*, const void*, void*, float*, float*, int, int, float, float, hipStream_t);
template hipError_t launch_rms_stats<float>(const void*, const void*, void*, float*, float*, int, int, float, float, hipStream_t);
template hipError_t launch_fold_gamma<bf16>(const void*, const void*, void*, int, int, hipStream_t);
template hipError_t launch_fold_gamma<float>(const void*, const void*, void*, int, int, hipStream_t);
template hipError_t launch_down<bf16>(const DownArgs&, hipStream_t);
template hipError_t launch_down<float>(const DownArgs&, hipStream_t);
template hipError_t launch_up<bf16>(const UpArgs&, int, hipStream_t);
template hipError_t launch_up<float>(const UpArgs&, int, hipStream_t);
template hipError_t launch_finish<bf16>(const float*, const float*, void*, void*, float*, int, int, int, int, float,
                                        float, int, hipStream_t);
template hipError_t launch_finish<float>(const float*, const float*, void*, void*, float*, int, int, int, int, float,
                                         float, int, hipStream_t);
template hipError_t launch_fold_gamma_t<bf16>(const void*, const void*, void*, int, int, hipStream_t);
template hipError_t launch_fold_gamma_t<float>(const void*, const void*, void*, int, int, hipStream_t);
template int small_rank_splits<bf16>(int, int, int, int, int);
template int small_rank_splits<float>(int, int, int, int, int);
template hipError_t launch_down_split<bf16>(const SplitDownArgs&, hipStream_t);
template hipError_t launch_down_split<float>(const SplitDownArgs&, hipStream_t);
template hipError_t launch_dz<bf16>(const DzArgs&, int, hipStream_t);
template hipError_t launch_dz<float>(const DzArgs&, int, hipStream_t);
template hipError_t launch_wgrad<bf16>(const WgradArgs&, hipStream_t);
template hipError_t launch_wgrad<float>(const WgradArgs&, hipStream_t);
template hipError_t launch_wgrad_reduce<bf16>(const WgradArgs&, hipStream_t);
template hipError_t launch_wgrad_reduce<float>(const WgradArgs&, hipStream_t);
template hipError_t launch_dx<bf16>(const DxArgs&, hipStream_t);
template hipError_t launch_dx<float>(const DxArgs&, hipStream_t);
template int dz_nparts<bf16>(int);
template int dz_nparts<float>(int);
template int wgrad_nparts<bf16>(int);
template int wgrad_nparts<float>(int);
template WgradPlan wgrad_plan<bf16>(int, int, int, int, int, int);
template WgradPlan wgrad_plan<float>(int, int, int, int, int, int);

}  // namespace lr

// HIP kernels of the fused low-rank bottleneck block (gfx950).
//
// Forward  (lr_block_fwd):
//   fold_gamma : A' = diag(gamma) . A                      (weights only, d x g*r)
//   down       : acc = x . A'  with the per-token sum of squares of x accumulated
//                from the same x tiles on their way to LDS (Online-RMSNorm: the
//                statistic is local, the normalisation is applied late), then
//                h = rstd * acc, sigma(h) in fp32 registers; writes h (checkpoint)
//                and z = sigma(h).  SwiGLU pairs gate/up columns in one lane.
//   up         : y_i = z_i . B_i, batched over branches (one launch).
// Backward (lr_block_bwd), with h' = rstd * dh (rstd recomputed from x):
//   stats      : rstd from x
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
#include "lr_kernels.h"

namespace lr {

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
  float s = 0.f;
  for (int j = lane * VEC; j < d; j += 64 * VEC) s += sumsq_vec(*reinterpret_cast<const uint4*>(xr + j), (E*)nullptr);
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

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// seam: h = partial * rstd, z = sigma(h)
template <typename E>
__global__ __launch_bounds__(256) void k_finish(const float* __restrict__ partial, const float* __restrict__ sumsq,
                                                E* __restrict__ h, E* __restrict__ z, int T, int r, int g,
                                                int act, float invD, float eps) {
  const int gr = g * r;
  const int ncols = (act == ACT_SWIGLU) ? r : gr;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * ncols) return;
  const int t = (int)(i / ncols), c = (int)(i % ncols);
  const float rs = 1.0f / sqrtf(sumsq[t] * invD + eps);
  const float* pr = partial + (int64_t)t * gr;
  if (act == ACT_SWIGLU) {
    const float hg = pr[c] * rs, hu = pr[r + c] * rs;
    if (h) {
      h[(int64_t)t * gr + c] = from_f32<E>(hg);
      h[(int64_t)t * gr + r + c] = from_f32<E>(hu);
    }
    z[(int64_t)t * r + c] = from_f32<E>(hg * sigmoidf_(hg) * hu);
  } else {
    const float hv = pr[c] * rs;
    if (h) h[(int64_t)t * gr + c] = from_f32<E>(hv);
    if (act == ACT_SILU) z[(int64_t)t * gr + c] = from_f32<E>(hv * sigmoidf_(hv));
    else if (!h) z[(int64_t)t * gr + c] = from_f32<E>(hv);
  }
}

template <int PARTS>
__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ parts, float* __restrict__ out,
                                                   int n, int nparts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float* p = parts + (int64_t)i * nparts;
  float s = 0.f;
  for (int k = 0; k < nparts; ++k) s += p[k];
  out[i] = s;
}

// ------------------------------------------------------------------ down projection
// acc = x . A' over K = d; mode DOWN_BLOCK: h = rstd*acc, z = sigma(h);
// mode DOWN_PARTIAL: fp32 partial = acc and sumsq (tile column 0 writes it).
template <class C, bool GATEUP>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_down(DownArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[2 * C::LDS_STAGE + C::BM / 4];
  float* rowss = reinterpret_cast<float*>(lds + 2 * C::LDS_STAGE);
  const int gr = a.g * a.r;
  const int ncols_logical = GATEUP ? a.r : gr;  // columns walked by tiles
  const int tiles_n = (ncols_logical + (GATEUP ? C::BN / 2 : C::BN) - 1) / (GATEUP ? C::BN / 2 : C::BN);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * C::BM;
  const int n0 = tn * (GATEUP ? C::BN / 2 : C::BN);

  Opnd oa{a.x, a.d, a.T, a.d};
  Opnd ob{a.Ap, gr, gr, a.d};
  f32x16 acc[C::MB][C::NB];
  if constexpr (GATEUP) {
    gemm_tile<C, false, true, true>(oa, ob, MapId{}, MapGateUp<C::WTN>{a.r}, m0, n0, a.d, lds, rowss, acc);
  } else {
    gemm_tile<C, false, true, true>(oa, ob, MapId{}, MapId{}, m0, n0, a.d, lds, rowss, acc);
  }

  FragPos<C> fp(m0, 0);
  const int wn = (threadIdx.x >> 6) % C::WN;
  if (a.mode == DOWN_PARTIAL) {
    if (tn == 0 && threadIdx.x < C::BM && m0 + (int)threadIdx.x < a.T)
      a.sumsq[m0 + threadIdx.x] = rowss[threadIdx.x];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = fp.row(mb, v);
        if (row >= a.T) continue;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          int col;
          if constexpr (GATEUP) {
            MapGateUp<C::WTN> mp{a.r};
            col = mp(n0, wn * C::WTN + nb * 32 + (fp.lane & 31));
          } else {
            col = n0 + wn * C::WTN + nb * 32 + (fp.lane & 31);
          }
          if (col < 0 || col >= gr) continue;
          a.partial[(int64_t)row * gr + col] = acc[mb][nb][v];
        }
      }
    return;
  }

  E* h = static_cast<E*>(a.h);
  E* z = static_cast<E*>(a.z);
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = fp.row(mb, v);
      if (row >= a.T) continue;
      const float rs = 1.0f / sqrtf(rowss[row - m0] * a.invD + a.eps);
      if constexpr (GATEUP) {
#pragma unroll
        for (int nb = 0; nb < C::NB / 2; ++nb) {
          const int logical = n0 + wn * (C::WTN / 2) + nb * 32 + (fp.lane & 31);
          if (logical >= a.r) continue;
          const float hg = acc[mb][nb][v] * rs, hu = acc[mb][nb + C::NB / 2][v] * rs;
          if (h) {
            h[(int64_t)row * gr + logical] = from_f32<E>(hg);
            h[(int64_t)row * gr + a.r + logical] = from_f32<E>(hu);
          }
          z[(int64_t)row * a.r + logical] = from_f32<E>(hg * sigmoidf_(hg) * hu);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const int col = n0 + wn * C::WTN + nb * 32 + (fp.lane & 31);
          if (col >= gr) continue;
          const float hv = acc[mb][nb][v] * rs;
          if (h) h[(int64_t)row * gr + col] = from_f32<E>(hv);
          if (a.act == ACT_SILU) z[(int64_t)row * gr + col] = from_f32<E>(hv * sigmoidf_(hv));
          else if (!h) z[(int64_t)row * gr + col] = from_f32<E>(hv);
        }
      }
    }
}

// ------------------------------------------------------------------ up projection
// y_i = z_i . B_i ; blockIdx.y = branch
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_up(UpArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[2 * C::LDS_STAGE];
  const int br = blockIdx.y;
  const int tiles_n = (a.d + C::BN - 1) / C::BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  Opnd oa{static_cast<const E*>(a.z) + (int64_t)br * a.r, a.ldz, a.T, a.r};
  Opnd ob{a.B[br], a.d, a.d, a.r};
  f32x16 acc[C::MB][C::NB];
  gemm_tile<C, false, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, a.r, lds, nullptr, acc);
  E* y = static_cast<E*>(a.y[br]);
  FragPos<C> fp(m0, n0);
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = fp.row(mb, v);
      if (row >= a.T) continue;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int col = fp.col(nb);
        if (col < a.d) y[(int64_t)row * a.d + col] = from_f32<E>(acc[mb][nb][v]);
      }
    }
}

// ------------------------------------------------------------------ backward: dz -> dh'
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dz(DzArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[2 * C::LDS_STAGE];
  const int br = blockIdx.y;
  const int tiles_n = (a.r + C::BN - 1) / C::BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  Opnd oa{a.dy[br], a.d, a.T, a.d};
  Opnd ob{a.B[br], a.d, a.r, a.d};  // B_i^T: (n = c, k = j) at B_i[c*d + j]
  f32x16 acc[C::MB][C::NB];
  gemm_tile<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, a.d, lds, nullptr, acc);

  const int gr = a.g * a.r;
  const E* h = static_cast<const E*>(a.h);
  E* dh = static_cast<E*>(a.dh);
  E* z = static_cast<E*>(a.z);
  FragPos<C> fp(m0, n0);
  const int wn = (threadIdx.x >> 6) % C::WN;
  const int part = (br * tiles_n + tn) * C::WN + wn;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = fp.row(mb, v);
      const bool rok = row < a.T;
      const float rs = rok ? a.rstd[row] : 0.f;
      float srow = 0.f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int c = fp.col(nb);
        if (!rok || c >= a.r) continue;
        const float dzv = acc[mb][nb][v];
        const int64_t hrow = (int64_t)row * gr;
        if (a.act == ACT_IDENTITY) {
          const float hv = to_f32(h[hrow + br * a.r + c]);
          const float d1 = rs * dzv;
          dh[hrow + br * a.r + c] = from_f32<E>(d1);
          srow += d1 * hv;
        } else if (a.act == ACT_SILU) {
          const float hv = to_f32(h[hrow + br * a.r + c]);
          const float s = sigmoidf_(hv);
          const float d1 = rs * dzv * s * (1.0f + hv * (1.0f - s));
          dh[hrow + br * a.r + c] = from_f32<E>(d1);
          z[hrow + br * a.r + c] = from_f32<E>(hv * s);
          srow += d1 * hv;
        } else {  // SwiGLU, one branch
          const float hg = to_f32(h[hrow + c]), hu = to_f32(h[hrow + a.r + c]);
          const float s = sigmoidf_(hg);
          const float sg = hg * s;
          const float dg = rs * dzv * hu * s * (1.0f + hg * (1.0f - s));
          const float du = rs * dzv * sg;
          dh[hrow + c] = from_f32<E>(dg);
          dh[hrow + a.r + c] = from_f32<E>(du);
          z[(int64_t)row * a.r + c] = from_f32<E>(sg * hu);
          srow += dg * hg + du * hu;
        }
      }
      // reduce over the 32 columns held by lanes with the same lane>>5
      srow += __shfl_xor(srow, 1);
      srow += __shfl_xor(srow, 2);
      srow += __shfl_xor(srow, 4);
      srow += __shfl_xor(srow, 8);
      srow += __shfl_xor(srow, 16);
      if ((fp.lane & 31) == 0 && rok) a.spart[(int64_t)row * a.nspart + part] = srow;
    }
}

// ------------------------------------------------------------------ backward: weight gradients
// blockIdx.y < n_up: dB_i = z_i^T . dy_i ; blockIdx.y == n_up: M = x^T . dh' -> dA, dgamma partials
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_wgrad(WgradArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[2 * C::LDS_STAGE];
  const int job = blockIdx.y;
  const int gr = a.g * a.r;
  const bool isA = job == a.n_up;
  const int M = isA ? a.d : a.r, N = isA ? gr : a.d;
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  if ((int)blockIdx.x >= tiles_m * tiles_n) return;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  Opnd oa, ob;
  if (isA) {
    oa = Opnd{a.x, a.d, a.d, a.T};   // x^T: (m = j, k = t) at x[t*d + j]
    ob = Opnd{a.dh, gr, gr, a.T};    // dh': (n = c, k = t) at dh[t*gr + c]
  } else {
    oa = Opnd{static_cast<const E*>(a.z) + (int64_t)job * a.r, a.ldz, a.r, a.T};
    ob = Opnd{a.dy[job], a.d, a.d, a.T};
  }
  f32x16 acc[C::MB][C::NB];
  gemm_tile<C, true, true, false>(oa, ob, MapId{}, MapId{}, m0, n0, a.T, lds, nullptr, acc);

  FragPos<C> fp(m0, n0);
  if (!isA) {
    float* dB = a.dB[job];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = fp.row(mb, v);
        if (row >= M) continue;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const int col = fp.col(nb);
          if (col < N) dB[(int64_t)row * N + col] = acc[mb][nb][v];
        }
      }
    return;
  }
  const E* Aw = static_cast<const E*>(a.A);
  const E* gamma = static_cast<const E*>(a.gamma);
  const int wn = (threadIdx.x >> 6) % C::WN;
  const int part = tn * C::WN + wn;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = fp.row(mb, v);  // j
      const bool rok = row < M;
      const float gj = rok ? to_f32(gamma[row]) : 0.f;
      float s = 0.f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int col = fp.col(nb);
        if (!rok || col >= N) continue;
        const float m = acc[mb][nb][v];
        a.dA[(int64_t)row * gr + col] = gj * m;
        s += to_f32(Aw[(int64_t)row * gr + col]) * m;
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 16);
      if ((fp.lane & 31) == 0 && rok) a.gpart[(int64_t)row * a.ngpart + part] = s;
    }
}

// ------------------------------------------------------------------ backward: dx
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dx(DxArgs a) {
  using E = typename C::E;
  __shared__ uint4 lds[2 * C::LDS_STAGE + C::BM / 4];
  float* srow = reinterpret_cast<float*>(lds + 2 * C::LDS_STAGE);  // [BM] : rstd*S'/D
  const int gr = a.g * a.r;
  const int tiles_n = (a.d + C::BN - 1) / C::BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  Opnd oa{a.dh, gr, a.T, gr};   // dh' [T, gr]
  Opnd ob{a.A, gr, a.d, gr};    // A^T: (n = j, k = c) at A[j*gr + c]
  f32x16 acc[C::MB][C::NB];
  gemm_tile<C, false, false, false>(oa, ob, MapId{}, MapId{}, m0, n0, gr, lds, nullptr, acc);
  for (int i = threadIdx.x; i < C::BM; i += C::THREADS) {
    const int t = m0 + i;
    float s = 0.f;
    if (t < a.T) {
      const float* p = a.spart + (int64_t)t * a.nspart;
      for (int k = 0; k < a.nspart; ++k) s += p[k];
      s *= a.rstd[t] * a.invD;
    }
    srow[i] = s;
  }
  __syncthreads();
  const E* x = static_cast<const E*>(a.x);
  const E* gamma = static_cast<const E*>(a.gamma);
  E* dx = static_cast<E*>(a.dx);
  FragPos<C> fp(m0, n0);
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int col = fp.col(nb);
    if (col >= a.d) continue;
    const float gj = to_f32(gamma[col]);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = fp.row(mb, v);
        if (row >= a.T) continue;
        const int64_t idx = (int64_t)row * a.d + col;
        dx[idx] = from_f32<E>(gj * acc[mb][nb][v] - to_f32(x[idx]) * srow[row - m0]);
      }
  }
}

// ------------------------------------------------------------------ launchers
template <typename E>
struct Cfgs;
template <>
struct Cfgs<bf16> {
  using Main = TileCfg<bf16, 256, 256, 2, 2>;
};
template <>
struct Cfgs<float> {
  using Main = TileCfg<float, 128, 128, 2, 2>;
};

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

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

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(cdiv(n, 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_down(const DownArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Main;
  if (a.T == 0) return hipSuccess;
  const int gr = a.g * a.r;
  const bool gateup = a.act == ACT_SWIGLU && a.mode == DOWN_BLOCK;
  if (gateup) {
    const int tiles = cdiv(a.T, C::BM) * cdiv(a.r, C::BN / 2);
    hipLaunchKernelGGL((k_down<C, true>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  } else {
    const int tiles = cdiv(a.T, C::BM) * cdiv(gr, C::BN);
    hipLaunchKernelGGL((k_down<C, false>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_up(const UpArgs& a, int n_up, hipStream_t s) {
  using C = typename Cfgs<E>::Main;
  if (a.T == 0) return hipSuccess;
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.d, C::BN);
  hipLaunchKernelGGL((k_up<C>), dim3(tiles, n_up), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_finish(const float* partial, const float* sumsq, void* h, void* z, int T, int r, int g, int act,
                         float invD, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int ncols = act == ACT_SWIGLU ? r : g * r;
  hipLaunchKernelGGL(k_finish<E>, dim3(cdiv((int64_t)T * ncols, 256)), dim3(256), 0, s, partial, sumsq,
                     static_cast<E*>(h), static_cast<E*>(z), T, r, g, act, invD, eps);
  return hipGetLastError();
}

template <typename E>
int dz_nparts(int r) {
  using C = typename Cfgs<E>::Main;
  return cdiv(r, C::BN) * C::WN;
}
template <typename E>
int wgrad_nparts(int gr) {
  using C = typename Cfgs<E>::Main;
  return cdiv(gr, C::BN) * C::WN;
}

template <typename E>
hipError_t launch_dz(const DzArgs& a, int n_up, hipStream_t s) {
  using C = typename Cfgs<E>::Main;
  if (a.T == 0) return hipSuccess;
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.r, C::BN);
  hipLaunchKernelGGL((k_dz<C>), dim3(tiles, n_up), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Main;
  const int gr = a.g * a.r;
  const int tilesB = cdiv(a.r, C::BM) * cdiv(a.d, C::BN);
  const int tilesA = cdiv(a.d, C::BM) * cdiv(gr, C::BN);
  const int tiles = tilesA > tilesB ? tilesA : tilesB;
  hipLaunchKernelGGL((k_wgrad<C>), dim3(tiles, a.n_up + 1), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_dx(const DxArgs& a, hipStream_t s) {
  using C = typename Cfgs<E>::Main;
  if (a.T == 0) return hipSuccess;
  const int tiles = cdiv(a.T, C::BM) * cdiv(a.d, C::BN);
  hipLaunchKernelGGL((k_dx<C>), dim3(tiles), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, float* out, int n, int nparts, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_parts<0>, dim3(cdiv(n, 256)), dim3(256), 0, s, parts, out, n, nparts);
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
template hipError_t launch_finish<bf16>(const float*, const float*, void*, void*, int, int, int, int, float, float, hipStream_t);
template hipError_t launch_finish<float>(const float*, const float*, void*, void*, int, int, int, int, float, float, hipStream_t);
template hipError_t launch_dz<bf16>(const DzArgs&, int, hipStream_t);
template hipError_t launch_dz<float>(const DzArgs&, int, hipStream_t);
template hipError_t launch_wgrad<bf16>(const WgradArgs&, hipStream_t);
template hipError_t launch_wgrad<float>(const WgradArgs&, hipStream_t);
template hipError_t launch_dx<bf16>(const DxArgs&, hipStream_t);
template hipError_t launch_dx<float>(const DxArgs&, hipStream_t);
template int dz_nparts<bf16>(int);
template int dz_nparts<float>(int);
template int wgrad_nparts<bf16>(int);
template int wgrad_nparts<float>(int);

}  // namespace lr

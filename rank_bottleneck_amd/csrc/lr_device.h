// Device-side building blocks of the low-rank block kernels (gfx950 / CDNA4).
//
// A GEMM tile C[BM x BN] += A[BM x K] . B[K x BN] is computed by NWAVES = WM x WN
// wavefronts of 64 lanes.  Operand tiles of BK columns of K are staged in LDS,
// always K-contiguous: one LDS row per M (or N) index, eight 16-byte chunks per
// row, chunk index XOR-swizzled with the row's low three bits so that the MFMA
// operand reads (eight consecutive rows, same chunk) and the staging writes
// (one row, eight chunks) are both free of bank conflicts.
//
// Operands come from HBM in one of two orientations:
//   KC  : element (mn, k) at p[mn*ld + k]  (K contiguous)  -> copied as 16-byte vectors
//   MNC : element (mn, k) at p[k*ld + mn]  (M/N contiguous) -> VEC x VEC blocks are read
//         as VEC row vectors and transposed in registers before the LDS write
// so one mainloop serves the forward projections (weights stored [K, N]), the
// input-gradient products (weights read transposed) and the weight gradients
// (both operands reduced over tokens).
//
// MFMA: bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2_f32.  In both,
// lane l supplies row (l % 32) of A and column (l % 32) of B; lanes 0-31 take the
// even 16-byte chunk of a chunk pair and lanes 32-63 the odd one.  Any assignment
// of K positions works as long as A and B agree, so an fp32 chunk pair feeds four
// 32x32x2 MFMAs (element s of each lane's chunk in the s-th one).  The 32x32
// accumulator of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l%32 in
// register v.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

typedef __bf16 bf16;  // also declared in lr_kernels.h
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename E> __device__ __forceinline__ E from_f32(float f);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return (bf16)f; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_(float v) { return fast_rcp(1.0f + __expf(-v)); }

// sum of squares of the VEC elements held in a 16-byte vector
__device__ __forceinline__ float sumsq_vec(const uint4& q, bf16*) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}
__device__ __forceinline__ float sumsq_vec(const uint4& q, float*) {
  float a = __uint_as_float(q.x), b = __uint_as_float(q.y), c = __uint_as_float(q.z),
        d = __uint_as_float(q.w);
  return fmaf(a, a, fmaf(b, b, fmaf(c, c, d * d)));
}

// VEC x VEC register transpose: in[e] holds elements (k = e, mn = 0..VEC-1); out[j]
// holds (k = 0..VEC-1, mn = j).
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, bf16*) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(in);  // a[e*4 + p]: mn = 2p, 2p+1
  uint32_t* o = reinterpret_cast<uint32_t*>(out);            // o[j*4 + q]: k = 2q, 2q+1
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = a[(2 * q) * 4 + j / 2], hi = a[(2 * q + 1) * 4 + j / 2];
      o[j * 4 + q] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                             : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
}
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, float*) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(in);  // a[e*4 + j]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) o[j * 4 + q] = a[q * 4 + j];
}

__device__ __forceinline__ void mfma_chunk(f32x16& acc, const uint4& a, const uint4& b, bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(f32x16& acc, const uint4& a, const uint4& b, float*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

template <typename E_, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  using E = E_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int VEC = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  static constexpr int CH = 8;                      // chunks per LDS row
  static constexpr int BK = CH * VEC;               // 64 (bf16) or 32 (fp32)
  static constexpr int NWAVES = WM * WN;
  static constexpr int THREADS = NWAVES * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static constexpr int LDS_A = BM * CH, LDS_B = BN * CH;  // uint4 units per stage
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static constexpr int LDS_GEMM_BYTES = 2 * LDS_STAGE * 16;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM % VEC == 0 && BN % VEC == 0, "tile must be a multiple of VEC");
};

// One operand of a GEMM: base pointer, leading dimension (elements) and the valid
// extents; loads outside [0, MN) x [0, K) read as zero.
struct Opnd {
  const void* p;
  int64_t ld;
  int MN;
  int K;
};

// tile-local row/column -> global index (identity)
struct MapId {
  __device__ __forceinline__ int operator()(int base, int local) const { return base + local; }
};

// Column map that puts matching gate and up columns of a [d, 2r] concatenated
// weight into the same lane: within a wave's WTN columns, the first half of the
// 32-column blocks are gate columns and the second half the up columns of the same
// logical positions.  `base` is the tile's first logical (gate) column.
template <int WTN>
struct MapGateUp {
  int r;
  __device__ __forceinline__ int operator()(int base, int local) const {
    constexpr int NBW = WTN / 32;
    const int wn = local / WTN, bw = (local % WTN) / 32, c = local % 32;
    const bool up = bw >= NBW / 2;
    const int logical = base + wn * (WTN / 2) + (up ? bw - NBW / 2 : bw) * 32 + c;
    if (logical >= r) return -1;
    return up ? r + logical : logical;
  }
};

template <class C, int ROWS, bool MNC>
struct Loader {
  using E = typename C::E;
  static constexpr int VEC = C::VEC, CH = C::CH, NT = C::THREADS;
  static constexpr int UNITS = MNC ? (ROWS / VEC) * CH : ROWS * CH;
  static constexpr int PER = (UNITS + NT - 1) / NT;
  static constexpr int REGS = MNC ? PER * VEC : PER;
  uint4 r[REGS];

  template <class Map>
  __device__ __forceinline__ void load(const Opnd& o, const Map& map, int mn0, int k0, int tid) {
    const E* base = static_cast<const E*>(o.p);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      const bool in_tile = (UNITS % NT == 0) || u < UNITS;
      if (!MNC) {
        const int row = u / CH, ch = u % CH;
        const int gmn = map(mn0, row);
        const int gk = k0 + ch * VEC;
        const bool ok = in_tile && gmn >= 0 && gmn < o.MN && gk < o.K;
        r[i] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)gmn * o.ld + gk)
                  : make_uint4(0, 0, 0, 0);
      } else {
        const int ch = u % CH, blk = u / CH;
        const int gmn = map(mn0, blk * VEC);
        const int gk = k0 + ch * VEC;
        const bool okmn = in_tile && gmn >= 0 && gmn < o.MN;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const bool ok = okmn && (gk + e) < o.K;
          r[i * VEC + e] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)(gk + e) * o.ld + gmn)
                              : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  // running per-row sum of squares of a K-contiguous operand (one value per unit)
  __device__ __forceinline__ void accum_sumsq(float* ss) const {
    static_assert(!MNC, "row statistics need a K-contiguous operand");
#pragma unroll
    for (int i = 0; i < PER; ++i) ss[i] += sumsq_vec(r[i], (E*)nullptr);
  }

  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if ((UNITS % NT != 0) && u >= UNITS) continue;
      if (!MNC) {
        const int row = u / CH, ch = u % CH;
        lds[row * CH + (ch ^ (row & 7))] = r[i];
      } else {
        const int ch = u % CH, blk = u / CH;
        uint4 t[VEC];
        transpose_block(&r[i * VEC], t, (E*)nullptr);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int row = blk * VEC + j;
          lds[row * CH + (ch ^ (row & 7))] = t[j];
        }
      }
    }
  }
};

template <class C>
__device__ __forceinline__ void mma_stage(const uint4* ldsA, const uint4* ldsB,
                                          f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane) {
  const int lr = lane & 31, hi = lane >> 5, sw = lane & 7;
#pragma unroll
  for (int ks = 0; ks < C::CH / 2; ++ks) {
    const int ch = (2 * ks + hi) ^ sw;
    uint4 a[C::MB], b[C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) a[mb] = ldsA[(wm * C::WTM + mb * 32 + lr) * C::CH + ch];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) b[nb] = ldsB[(wn * C::WTN + nb * 32 + lr) * C::CH + ch];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) mfma_chunk(acc[mb][nb], a[mb], b[nb], (typename C::E*)nullptr);
  }
}

// Double-buffered mainloop over K.  With ROWSTAT the K-contiguous A operand's
// per-row sum of squares is accumulated on the way through registers and left,
// reduced, in rowss[0..BM) (LDS).
template <class C, bool A_MNC, bool B_MNC, bool ROWSTAT, class MapA, class MapB>
__device__ __forceinline__ void gemm_tile(const Opnd& oa, const Opnd& ob, const MapA& ma,
                                          const MapB& mbm, int m0, int n0, int K, uint4* lds,
                                          float* rowss, f32x16 (&acc)[C::MB][C::NB]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  Loader<C, C::BM, A_MNC> la;
  Loader<C, C::BN, B_MNC> lb;
  float ss[ROWSTAT ? Loader<C, C::BM, A_MNC>::PER : 1];
#pragma unroll
  for (int i = 0; i < (ROWSTAT ? Loader<C, C::BM, A_MNC>::PER : 1); ++i) ss[i] = 0.f;

  const int nk = (K + C::BK - 1) / C::BK;
  if (nk > 0) {
    la.load(oa, ma, m0, 0, tid);
    lb.load(ob, mbm, n0, 0, tid);
    if constexpr (ROWSTAT) la.accum_sumsq(ss);
    la.store(lds, tid);
    lb.store(lds + C::LDS_A, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint4* cur = lds + (kt & 1) * C::LDS_STAGE;
      uint4* nxt = lds + ((kt + 1) & 1) * C::LDS_STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(oa, ma, m0, (kt + 1) * C::BK, tid);
        lb.load(ob, mbm, n0, (kt + 1) * C::BK, tid);
      }
      mma_stage<C>(cur, cur + C::LDS_A, acc, wm, wn, lane);
      if (more) {
        if constexpr (ROWSTAT) la.accum_sumsq(ss);
        la.store(nxt, tid);
        lb.store(nxt + C::LDS_A, tid);
      }
      __syncthreads();
    }
  }
  if constexpr (ROWSTAT) {
    static_assert(!A_MNC, "row statistics need a K-contiguous A");
    constexpr int PER = Loader<C, C::BM, A_MNC>::PER;
    constexpr int UNITS = Loader<C, C::BM, A_MNC>::UNITS;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float s = ss[i];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      const int u = tid + i * C::THREADS;
      if ((u % C::CH) == 0 && ((UNITS % C::THREADS == 0) || u < UNITS)) rowss[u / C::CH] = s;
    }
    __syncthreads();
  }
}

// Global (row, col) of accumulator register v of block (mb, nb) for this lane.
template <class C>
struct FragPos {
  int row0, col0, lane;
  __device__ __forceinline__ FragPos(int m0, int n0) {
    const int tid = threadIdx.x, wave = tid >> 6;
    lane = tid & 63;
    row0 = m0 + (wave / C::WN) * C::WTM + 4 * (lane >> 5);
    col0 = n0 + (wave % C::WN) * C::WTN + (lane & 31);
  }
  __device__ __forceinline__ int row(int mb, int v) const { return row0 + mb * 32 + 8 * (v >> 2) + (v & 3); }
  __device__ __forceinline__ int col(int nb) const { return col0 + nb * 32; }
};

}  // namespace lr

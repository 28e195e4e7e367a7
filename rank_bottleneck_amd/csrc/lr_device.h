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

// LDS slot of 16-byte chunk `ch` of tile row `row`.  Rows are 128 bytes; the chunk
// index is XORed with bits 1..3 of the row, so that 16 consecutive rows reading
// the same chunk (one ds_read_b128 quarter-wave) and 2 rows written whole both
// touch 16 distinct 16-byte slots of a 256-byte bank window.
__device__ __forceinline__ int lds_slot(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

template <typename E_, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  using E = E_;
  static constexpr bool PIPE = false;
  static constexpr int WPE = 1;
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
  static constexpr int LDS_UINT4 = 2 * LDS_STAGE;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM % VEC == 0 && BN % VEC == 0, "tile must be a multiple of VEC");
};

// One operand of a GEMM: base pointer, leading dimension (elements) and the valid
// extents.  Loads at K >= K read as zero (hardware range check of the buffer
// resource); loads at M/N >= MN only feed output rows/columns that are never
// stored, and never read past the operand's last element.
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

constexpr uint32_t kOffInvalid = 0x80000000u;  // beyond every resource's range -> reads 0
constexpr int64_t kMaxRecords = 0x7fffffff;

// Buffer resource (gfx9 raw buffer, no stride) over [p, p + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// Global -> register -> LDS staging of one operand tile (ROWS x BK).
// KC : unit = one 16-byte vector (row, chunk); MNC: unit = a VEC x VEC block.
// Byte offsets are relative to the tile origin (row mn0 / k0 for KC, k0 / mn0 for
// MNC) and fixed for the whole K loop; the resource is rebased every k step.
template <class C, int ROWS, bool MNC>
struct Loader {
  using E = typename C::E;
  static constexpr int VEC = C::VEC, CH = C::CH, NT = C::THREADS;
  static constexpr int ES = (int)sizeof(E);
  static constexpr int UNITS = MNC ? (ROWS / VEC) * CH : ROWS * CH;
  static constexpr int PER = (UNITS + NT - 1) / NT;
  static constexpr int REGS = MNC ? PER * VEC : PER;
  uint32_t off[PER];
  uint4 r[REGS];

  template <class Map>
  __device__ __forceinline__ void init(const Opnd& o, const Map& map, int mn0, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      const bool in_tile = (UNITS % NT == 0) || u < UNITS;
      if (!MNC) {
        const int row = u / CH, ch = u % CH;
        const int gmn = map(mn0, row);
        const bool ok = in_tile && gmn >= 0;
        off[i] = ok ? (uint32_t)(((int64_t)(gmn - mn0) * o.ld + ch * VEC) * ES) : kOffInvalid;
      } else {
        const int ch = u % CH, blk = u / CH;
        const int gmn = map(mn0, blk * VEC);
        const bool ok = in_tile && gmn >= 0;
        off[i] = ok ? (uint32_t)(((int64_t)(ch * VEC) * o.ld + (gmn - mn0)) * ES) : kOffInvalid;
      }
    }
  }

  // Resource for the k step starting at k0: KC rows mn0.., columns k0..; MNC rows k0.., columns mn0..
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const Opnd& o, int mn0, int k0) const {
    const char* base = static_cast<const char*>(o.p);
    if (!MNC) {
      const int64_t rows = (int64_t)o.MN - mn0;
      return make_rsrc(base + ((int64_t)mn0 * o.ld + k0) * ES, rows <= 0 ? 0 : ((rows - 1) * o.ld + (o.K - k0)) * ES);
    } else {
      const int64_t rows = (int64_t)o.K - k0;
      return make_rsrc(base + ((int64_t)k0 * o.ld + mn0) * ES, rows <= 0 ? 0 : ((rows - 1) * o.ld + (o.MN - mn0)) * ES);
    }
  }

  __device__ __forceinline__ void load(const Opnd& o, int mn0, int k0) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(o, mn0, k0);
    const uint32_t rowb = (uint32_t)(o.ld * ES);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!MNC) {
        r[i] = buf_load16(rs, off[i]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) r[i * VEC + e] = buf_load16(rs, off[i] == kOffInvalid ? kOffInvalid : off[i] + e * rowb);
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
        lds[lds_slot(row, ch)] = r[i];
      } else {
        // lanes of odd blocks store the rows of each pair in swapped order, so
        // that the 16 lanes of one LDS cycle write rows of both parities
        const int ch = u % CH, blk = u / CH, flip = blk & 1;
        uint4 t[VEC];
        transpose_block(&r[i * VEC], t, (E*)nullptr);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int jj = j ^ flip;
          const int row = blk * VEC + jj;
          lds[lds_slot(row, ch)] = flip ? t[j ^ 1] : t[j];
        }
      }
    }
  }
};

template <class C>
__device__ __forceinline__ void load_frags(const uint4* ldsA, const uint4* ldsB, uint4 (&a)[C::MB], uint4 (&b)[C::NB],
                                           int ks, int wm, int wn, int lane) {
  const int lr = lane & 31, ch = 2 * ks + (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) a[mb] = ldsA[lds_slot(wm * C::WTM + mb * 32 + lr, ch)];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) b[nb] = ldsB[lds_slot(wn * C::WTN + nb * 32 + lr, ch)];
}

// MFMAs over one LDS stage; the fragments of sub-step ks+1 are read while the
// MFMAs of sub-step ks run.
template <class C>
__device__ __forceinline__ void mma_stage(const uint4* ldsA, const uint4* ldsB,
                                          f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane) {
  uint4 a[2][C::MB], b[2][C::NB];
  load_frags<C>(ldsA, ldsB, a[0], b[0], 0, wm, wn, lane);
#pragma unroll
  for (int ks = 0; ks < C::CH / 2; ++ks) {
    if (ks + 1 < C::CH / 2) load_frags<C>(ldsA, ldsB, a[(ks + 1) & 1], b[(ks + 1) & 1], ks + 1, wm, wn, lane);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
        mfma_chunk(acc[mb][nb], b[ks & 1][nb], a[ks & 1][mb], (typename C::E*)nullptr);
  }
}

// Double-buffered mainloop over k in [kbeg, kbeg + K).  With ROWSTAT the K-contiguous A operand's
// per-row sum of squares is accumulated on the way through registers and left,
// reduced, in rowss[0..BM) (LDS).
template <class C, bool A_MNC, bool B_MNC, bool ROWSTAT, class MapA, class MapB>
__device__ __forceinline__ void gemm_tile(const Opnd& oa, const Opnd& ob, const MapA& ma,
                                          const MapB& mbm, int m0, int n0, int kbeg, int K, uint4* lds,
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
    la.init(oa, ma, m0, tid);
    lb.init(ob, mbm, n0, tid);
    la.load(oa, m0, kbeg);
    lb.load(ob, n0, kbeg);
    if constexpr (ROWSTAT) la.accum_sumsq(ss);
    la.store(lds, tid);
    lb.store(lds + C::LDS_A, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint4* cur = lds + (kt & 1) * C::LDS_STAGE;
      uint4* nxt = lds + ((kt + 1) & 1) * C::LDS_STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(oa, m0, kbeg + (kt + 1) * C::BK);
        lb.load(ob, n0, kbeg + (kt + 1) * C::BK);
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
    __syncthreads();  // rowss may alias the staging buffers
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

// Work-group scheduling.  The dispatcher hands consecutive work-group ids to the 8
// XCDs in turn, and each XCD has its own L2.  xcd_remap() renumbers ids so that
// every XCD receives one contiguous range of logical tiles, and grouped_tile()
// walks each range in groups of GROUP_M row panels, so that the work-groups
// resident on one XCD at a time share few operand panels.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int xcd = bid % kNumXcd, idx = bid / kNumXcd;
  const int per = nblk / kNumXcd, extra = nblk % kNumXcd;
  return xcd * per + (xcd < extra ? xcd : extra) + idx;
}
template <int GROUP_M>
__device__ __forceinline__ void grouped_tile(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (logical / in_group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int w = logical % in_group;
  tm = first_m + w % gsz;
  tn = w / gsz;
}

#define LR_LDS __attribute__((address_space(3)))

// Row-sweep epilogue.  A wave's WTM x WTN fp32 accumulators are staged through
// its own LDS region one 32-row block at a time (rows padded by 16 bytes, so the
// column-major writes of 16 lanes hit distinct banks); lanes then sweep the block
// row by row, each taking 4 consecutive columns, so every global access of the
// epilogue is a contiguous run of whole cache lines.
template <class C>
struct RowStage {
  static constexpr int PITCH = C::WTN * 4 + 16;  // bytes per staged row
  static constexpr int REGION = 32 * PITCH;      // bytes per wave
  static constexpr int UINT4 = C::NWAVES * REGION / 16;
};

template <class C>
__device__ __forceinline__ char LR_LDS* stage_region(uint4* lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return (char LR_LDS*)(lds) + wave * RowStage<C>::REGION;
}

template <class C>
__device__ __forceinline__ void stage_block(const f32x16 (&acc)[C::MB][C::NB], int mb, char LR_LDS* region) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  char LR_LDS* rowp = region + (lane & 31) * RowStage<C>::PITCH + 16 * (lane >> 5);
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f4 v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
      *reinterpret_cast<f4 LR_LDS*>(rowp + (nb * 32 + 8 * q) * 4) = v;
    }
}

__device__ __forceinline__ float4 lds_f4(const char LR_LDS* p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = *reinterpret_cast<const f4 LR_LDS*>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// Sweep the staged block: COLS leading columns of each of the 32 rows; f(rl, cl,
// row pointer) is called with the block-local row, the wave-local column (a
// multiple of 4) and the staged row.  LPR = COLS/4 lanes share one row.
template <class C, int COLS, class F>
__device__ __forceinline__ void sweep_block(const char LR_LDS* region, F&& f) {
  constexpr int LPR = COLS / 4, RPI = 64 / LPR;
  static_assert(LPR <= 64 && 64 % LPR == 0, "row sweep width");
  const int lane = threadIdx.x & 63;
#pragma unroll 4
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rl = it * RPI + lane / LPR, cl = (lane % LPR) * 4;
    f(rl, cl, region + rl * RowStage<C>::PITCH);
  }
}

// Same sweep in two phases: load(it, rl, cl, in[it]) for every iteration first
// (global loads of epilogue inputs, all in flight together), then
// f(it, rl, cl, row pointer, in[it]).
template <class C, int COLS, int NL, class FL, class F>
__device__ __forceinline__ void sweep_block_pre(const char LR_LDS* region, FL&& load, F&& f) {
  constexpr int LPR = COLS / 4, RPI = 64 / LPR, IT = 32 / RPI;
  const int lane = threadIdx.x & 63;
  float4 in[IT][NL];
#pragma unroll
  for (int it = 0; it < IT; ++it) load(it * RPI + lane / LPR, (lane % LPR) * 4, in[it]);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int rl = it * RPI + lane / LPR, cl = (lane % LPR) * 4;
    f(rl, cl, region + rl * RowStage<C>::PITCH, in[it]);
  }
}

// Lane geometry of a row sweep over COLS staged columns, for kernels that
// interleave their own loads with it: iteration it covers block row rl(it) and
// the 4 columns from cl.
template <class C, int COLS>
struct Sweep {
  static constexpr int LPR = COLS / 4, RPI = 64 / LPR, IT = 32 / RPI;
  static_assert(LPR <= 64 && 64 % LPR == 0, "row sweep width");
  int r0, cl;
  __device__ __forceinline__ Sweep() {
    const int lane = threadIdx.x & 63;
    r0 = lane / LPR;
    cl = (lane % LPR) * 4;
  }
  __device__ __forceinline__ int rl(int it) const { return it * RPI + r0; }
};

// DPP lane move of x (ISA data-parallel primitives); lanes of rows outside
// ROWMASK read 0.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF,
                                                               false));
}

// Sum over the LPR consecutive lanes that share a row in a sweep (LPR a power of
// two up to 32), with DPP moves instead of LDS shuffles: pair and quad swaps,
// the mirrors within 8 and 16 lanes, then for 32 lanes a broadcast of lane 15 of
// each 16-lane row into the next.  The sum is complete in the group's last lane
// (row_sum_lane), and in every lane of the group when LPR <= 16.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(LPR >= 1 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row width");
  if constexpr (LPR >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
  if constexpr (LPR >= 16) v += dpp_mov<0x140>(v);  // row_mirror
  if constexpr (LPR == 32) v += dpp_mov<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  return v;
}
template <int LPR>
__device__ __forceinline__ bool row_sum_lane() {
  return (threadIdx.x & (LPR - 1)) == LPR - 1;
}

// 4 consecutive values -> memory (8 bytes of bf16 / 16 bytes of fp32), as
// nontemporal stores: every CU writes its output tiles at about the same time,
// and streaming them out measured 1-5% faster per kernel than write-back stores
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, v), reinterpret_cast<unsigned long long*>(p));
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}
__device__ __forceinline__ float4 load4(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Raw 4-element loads, converted to fp32 later, so that an epilogue can issue all
// of its input loads before the first use.
template <typename E> struct Raw4;
template <> struct Raw4<bf16> {
  typedef uint2 T;
  static __device__ __forceinline__ T load(const bf16* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ T zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ float4 f4(const T& u) {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
  }
};
template <> struct Raw4<float> {
  typedef float4 T;
  static __device__ __forceinline__ T load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ float4 f4(const T& u) { return u; }
};

}  // namespace lr

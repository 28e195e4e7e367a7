// bf16 GEMM mainloop with direct global->LDS loads (gfx950).
//
// Operand tiles go from HBM straight into a ring of STAGES LDS buffers with
// `buffer_load_dwordx4 ... lds` (each lane's 16 bytes land at M0 + 16*lane, an
// out-of-range lane writes zeros), STAGES-1 stages ahead of the MFMAs, so no
// register staging and no VALU transposes are needed.  The LDS layout depends on
// how the operand is stored in memory:
//   KC  (K contiguous): [rows][BK] rows of BK*2 bytes, 16-byte chunks XOR-swizzled;
//                       MFMA fragments come from ds_read_b128.
//   MNC (M/N contiguous): [BK][rows] rows of rows*2 bytes, 32-byte granules
//                       XOR-swizzled; fragments come from two ds_read_b64_tr_b16.
//                       That instruction treats each 16-lane group's 16 addresses
//                       as a 4 x 16 block (lane j names row j/4, columns 4*(j%4)..+3)
//                       and hands lane i column i of it, which is exactly the
//                       K-packed operand layout of v_mfma_f32_32x32x16_bf16.
// Both swizzles make a quarter/half-wave's reads hit distinct banks of a 256-byte
// window; the DMA writes are 1 KiB contiguous per instruction.
//
// One barrier per k step, placed once the last fragments of stage kt are in
// registers: wait for this wave's loads of stage kt+1, barrier (all waves' loads
// visible, all waves done reading stage kt), refill stage kt's buffer with stage
// kt+STAGES, read the first fragments of stage kt+1, then run the last MFMAs of
// stage kt.  The loads are inline assembly, so the compiler neither tracks them
// nor inserts waits for them; the waits are explicit (vmcnt counts this wave's
// own loads, which complete in order).
#pragma once

#include <type_traits>

#include "lr_device.h"


namespace lr {

// sub-steps over which the refill of one stage is spread: loads issued later than
// the first sub-step of the next stage are not back in time for the wait before
// its last sub-step, and packing them denser stalls the MFMA issue
constexpr int kRefillSubsteps = 2;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int WPE_ = 1>
struct PipeCfg {
  using E = bf16;
  static constexpr bool PIPE = true;
  static constexpr int WPE = WPE_;  // waves per SIMD the kernels are built for
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int VEC = 8;
  static constexpr int NWAVES = WM * WN, THREADS = NWAVES * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, MB = WTM / 32, NB = WTN / 32;
  static constexpr int KS = BK / 16;                       // MFMA k sub-steps per stage
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LPS_A = A_BYTES / (1024 * NWAVES), LPS_B = B_BYTES / (1024 * NWAVES);
  static constexpr int LPS = LPS_A + LPS_B;                // DMA instructions per stage per wave
  // ring of STAGES stages, then a sink that takes the (zero) loads of stages past
  // the end of K, A and B parts on top of each other, so that they never land on
  // LDS the epilogue uses
  static constexpr int SINK_BYTE = STAGES * STAGE_BYTES;
  static constexpr int SINK_BYTES = A_BYTES > B_BYTES ? A_BYTES : B_BYTES;
  static constexpr int LDS_UINT4 = (STAGES * STAGE_BYTES + SINK_BYTES) / 16;
  static_assert(A_BYTES % (1024 * NWAVES) == 0 && B_BYTES % (1024 * NWAVES) == 0, "tile / wave mismatch");
  static_assert(BK % 16 == 0 && (BK * 2 == 64 || BK * 2 == 128), "BK must be 32 or 64");
  static_assert((STAGES - 1) * LPS <= 63, "vmcnt range");
  static_assert(KS % 2 == 0, "fragment double buffer assumes an even number of sub-steps");
};

// 16-byte chunk swizzle of a KC tile row (RB = row bytes, 64 or 128)
template <int RB>
__device__ __forceinline__ int kc_swz(int row) {
  constexpr int RPW = 256 / RB, CPR = RB / 16;
  return (row / RPW) % CPR;
}
// 32-byte granule swizzle of an MNC tile row (k index)
__device__ __forceinline__ int mnc_swz(int krow) { return 2 * (krow & 3); }

struct Rsrc4 {
  int x, y, z, w;
};
__device__ __forceinline__ Rsrc4 rsrc4(const void* p, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
  return Rsrc4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)n, 0x00020000};
}

__device__ __forceinline__ void dma16(const Rsrc4& r, uint32_t voff, uint32_t lds_byte) {
  typedef int int4v __attribute__((ext_vector_type(4)));
  // the resource is wave-uniform; readfirstlane keeps it in SGPRs where the
  // compiler cannot prove that by itself
  const int4v rs = {__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                    __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds_byte)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Per-lane DMA offsets of one operand tile (relative to the tile origin at k0).
template <class C, int ROWS, bool MNC>
struct DmaTile {
  static constexpr int BYTES = ROWS * C::BK * 2;
  static constexpr int Q = BYTES / (1024 * C::NWAVES);  // instructions per wave per stage
  uint32_t off[Q];

  template <class Map>
  __device__ __forceinline__ void init(const Opnd& o, const Map& map, int mn0, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = (q * C::NWAVES + wave) * 1024 + 16 * lane;  // LDS byte within the tile
      if (!MNC) {
        constexpr int RB = C::BK * 2;
        const int row = p / RB, ch = ((p % RB) / 16) ^ kc_swz<RB>(row);
        const int gmn = map(mn0, row);
        off[q] = gmn >= 0 ? (uint32_t)(((int64_t)(gmn - mn0) * o.ld + ch * 8) * 2) : kOffInvalid;
      } else {
        constexpr int RB = ROWS * 2;
        const int krow = p / RB, b = p % RB;
        const int g = (b / 32) ^ mnc_swz(krow);
        const int mn = g * 16 + ((b % 32) / 16) * 8;
        const int gmn = map(mn0, mn);
        off[q] = gmn >= 0 ? (uint32_t)(((int64_t)krow * o.ld + (gmn - mn0)) * 2) : kOffInvalid;
      }
    }
  }

  // Resource of the stage starting at kbeg + st*BK: base0 + st*step, with the bytes
  // left to the operand's last element (bytes0 - st*step, clamped); `live == false`
  // gives an empty range (reads zeros).  All scalar arithmetic.
  const char* base0;
  int64_t bytes0, step;
  __device__ __forceinline__ void init_range(const Opnd& o, int mn0, int kbeg) {
    if (!MNC) {
      base0 = static_cast<const char*>(o.p) + ((int64_t)mn0 * o.ld + kbeg) * 2;
      bytes0 = ((int64_t)(o.MN - mn0 - 1) * o.ld + (o.K - kbeg)) * 2;
      step = (int64_t)C::BK * 2;
      if (o.MN - mn0 <= 0) bytes0 = -((int64_t)1 << 62);
    } else {
      base0 = static_cast<const char*>(o.p) + ((int64_t)kbeg * o.ld + mn0) * 2;
      bytes0 = ((int64_t)(o.K - kbeg - 1) * o.ld + (o.MN - mn0)) * 2;
      step = (int64_t)C::BK * o.ld * 2;
    }
  }
  // bytes left from stage st, clamped to [0, kMaxRecords] with 32-bit compares of
  // the two halves (scalar instructions only)
  __device__ __forceinline__ uint32_t records(int st) const {
    const int64_t b = bytes0 - (int64_t)st * step;
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)b >> 32));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    return (hi >> 31) ? 0u : (hi != 0 || lo > (uint32_t)kMaxRecords ? (uint32_t)kMaxRecords : lo);
  }
  __device__ __forceinline__ Rsrc4 rsrc(int st, bool live) const {
    const uint64_t a = reinterpret_cast<uint64_t>(base0) + (uint64_t)((int64_t)st * step);
    return Rsrc4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), live ? (int)records(st) : 0, 0x00020000};
  }

  // the same range as a compiler buffer resource (register staging)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(int st, bool live) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base0) + (int64_t)st * step, (short)0,
                                             live ? (int)records(st) : 0, 0x00020000);
  }
  __device__ __forceinline__ void issue(const Rsrc4& r, uint32_t lds_tile, int wave) const {
#pragma unroll
    for (int q = 0; q < Q; ++q) dma16(r, off[q], lds_tile + (q * C::NWAVES + wave) * 1024);
  }
  __device__ __forceinline__ void issue_one(int q, const Rsrc4& r, uint32_t lds_tile, int wave) const {
    dma16(r, off[q], lds_tile + (q * C::NWAVES + wave) * 1024);
  }
};

// one MFMA operand fragment (32 rows x 16 k) of the tile whose LDS image starts at `t`
template <class C, int ROWS, bool MNC>
__device__ __forceinline__ uint4 frag(const char LR_LDS* t, int rbase, int s, int lane) {
  if (!MNC) {
    constexpr int RB = C::BK * 2;
    const int row = rbase + (lane & 31);
    const int ch = (2 * s + (lane >> 5)) ^ kc_swz<RB>(row);
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4 LR_LDS*>(t + row * RB + ch * 16));
  } else {
    constexpr int RB = ROWS * 2;
    const int G = lane >> 4, j = lane & 15;
    const int mn = rbase + 16 * (G & 1) + 4 * (j & 3);
    const int kr0 = 16 * s + 8 * (G >> 1) + (j >> 2);
    const int kr1 = kr0 + 4;
    const bf16x4 LR_LDS* p0 =
        reinterpret_cast<const bf16x4 LR_LDS*>(t + kr0 * RB + (((mn >> 4) ^ mnc_swz(kr0)) * 32) + (mn & 15) * 2);
    const bf16x4 LR_LDS* p1 =
        reinterpret_cast<const bf16x4 LR_LDS*>(t + kr1 * RB + (((mn >> 4) ^ mnc_swz(kr1)) * 32) + (mn & 15) * 2);
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<bf16x4 LR_LDS*>(p0));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<bf16x4 LR_LDS*>(p1));
    const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
    return make_uint4(u0.x, u0.y, u1.x, u1.y);
  }
}

// running sum of squares of the 8 bf16 values of a fragment register (packed
// bf16 dot products, fp32 accumulation)
__device__ __forceinline__ float frag_sumsq(const uint4& q, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w[i]);
    acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
  }
  return acc;
}


// pre() hook of kernels that load nothing ahead of their epilogue
struct NoPre {
  __device__ __forceinline__ void operator()() const {}
};

// Mainloop over k in [kbeg, kbeg + K); same contract as gemm_tile (accumulator
// layout, ROWSTAT result in rowss[0..BM)).
// `pre()` runs once, two k steps before the end (at the start when there are
// fewer): kernels issue the global loads of their epilogue inputs there so that
// they arrive while the last MFMAs run.
template <class C, bool A_MNC, bool B_MNC, bool ROWSTAT, class MapA, class MapB, class Pre>
__device__ __forceinline__ void gemm_pipe(const Opnd& oa, const Opnd& ob, const MapA& ma, const MapB& mbm, int m0,
                                          int n0, int kbeg, int K, uint4* lds, float* rowss,
                                          f32x16 (&acc)[C::MB][C::NB], Pre&& pre) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
  float ss[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) ss[mb] = 0.f;

  DmaTile<C, C::BM, A_MNC> da;
  DmaTile<C, C::BN, B_MNC> db;
  da.init(oa, ma, m0, wave, lane);
  db.init(ob, mbm, n0, wave, lane);
  da.init_range(oa, m0, kbeg);
  db.init_range(ob, n0, kbeg);
  const char LR_LDS* ldsp = (const char LR_LDS*)(lds);
  const uint32_t lds0 = (uint32_t)(uintptr_t)ldsp;
  const int nk = (K + C::BK - 1) / C::BK;

  auto issue_stage = [&](int st) {
    // stages past the end read nothing (empty resource) and fill a buffer no one reads with zeros
    const bool live = st < nk;
    const uint32_t ba = lds0 + (live ? (st % C::STAGES) * C::STAGE_BYTES : C::SINK_BYTE);
    da.issue(da.rsrc(st, live), ba, wave);
    db.issue(db.rsrc(st, live), live ? ba + C::A_BYTES : ba, wave);
  };
  auto read_frags = [&](int st, int s, uint4 (&fa)[C::MB], uint4 (&fb)[C::NB]) {
    const char LR_LDS* ta = ldsp + (st % C::STAGES) * C::STAGE_BYTES;
    const char LR_LDS* tb = ta + C::A_BYTES;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) fa[mb] = frag<C, C::BM, A_MNC>(ta, wm * C::WTM + mb * 32, s, lane);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) fb[nb] = frag<C, C::BN, B_MNC>(tb, wn * C::WTN + nb * 32, s, lane);
  };


  if (nk > 0) {
    // Prefetch distance: STAGES stages.  Once every wave holds its last fragments of
    // stage kt, stage kt's buffer is refilled with stage kt+STAGES: the first half
    // of those loads goes out during the last MFMA sub-step of stage kt, the second
    // half during the first sub-step of stage kt+1, one load per few MFMAs, so that
    // this in-order wave never stalls on a burst of load issues while the MFMA pipe
    // runs dry.  Fragment reads of the next sub-step are interleaved the same way.
    // Stages past the end read an empty range into the sink, which keeps the load
    // count of every k step the same.  pre() runs at the start of the last k step,
    // which has no wait and no barrier, so its loads overlap the last MFMAs.
    constexpr int QA = DmaTile<C, C::BM, A_MNC>::Q, QB = DmaTile<C, C::BN, B_MNC>::Q;
    // the refill of a stage is cut into NS chunks: chunk 0 goes out in the last
    // sub-step of stage kt, chunk u in sub-step u-1 of stage kt+1
    constexpr int NS = kRefillSubsteps < C::KS ? kRefillSubsteps : C::KS;
    constexpr int HALF = (QA + QB) / NS;         // loads of chunk 0 (issued in the prologue too)
    constexpr int NMF = C::MB * C::NB;
    constexpr int NF = C::MB + C::NB;
    static_assert(C::KS >= 2 && NS >= 2, "the refill is split over at least two sub-steps");
    // ba / bb: LDS bases of the A and B parts (both the sink for stages past the end)
    auto issue_q = [&](int q, const Rsrc4& ra, const Rsrc4& rb, uint32_t ba, uint32_t bb) {
      if (q < QA)
        da.issue_one(q, ra, ba, wave);
      else
        db.issue_one(q - QA, rb, bb, wave);
    };
#pragma unroll
    for (int st = 0; st < C::STAGES - 1; ++st) issue_stage(st);
    constexpr int ST0 = C::STAGES - 1;
    Rsrc4 pra = da.rsrc(ST0, ST0 < nk), prb = db.rsrc(ST0, ST0 < nk);
    uint32_t pba = lds0 + (ST0 < nk ? ST0 * C::STAGE_BYTES : C::SINK_BYTE);
    uint32_t pbb = ST0 < nk ? pba + C::A_BYTES : pba;
#pragma unroll
    for (int q = 0; q < HALF; ++q) issue_q(q, pra, prb, pba, pbb);
    wait_vmcnt<(C::STAGES - 2) * C::LPS + HALF>();
    block_barrier();
    uint4 a[2][C::MB], b[2][C::NB];
    read_frags(0, 0, a[0], b[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const bool final_k = kt + 1 == nk;
      if (final_k) pre();
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int cur = s & 1, nxt = cur ^ 1;
        const bool last = s + 1 == C::KS;
        Rsrc4 ra = pra, rb = prb;
        uint32_t ba = pba, bb = pbb;
        int fst = kt, fs = s + 1;       // source of the next fragments
        if (last) {
          if (!final_k) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wait_vmcnt<(C::STAGES - 2) * C::LPS>();
            block_barrier();
          }
          const int st = kt + C::STAGES;
          const bool live = st < nk;
          ra = da.rsrc(st, live);
          rb = db.rsrc(st, live);
          ba = lds0 + (live ? (st % C::STAGES) * C::STAGE_BYTES : C::SINK_BYTE);
          bb = live ? ba + C::A_BYTES : ba;
          pra = ra;
          prb = rb;
          pba = ba;
          pbb = bb;
          fst = kt + 1;                 // past the end: reads nobody uses
          fs = 0;
        }
        const bool loads_here = last || s < NS - 1;
        const int u = last ? 0 : s + 1;  // refill chunk of this sub-step
        const int qlo = u * (QA + QB) / NS, qn = (u + 1) * (QA + QB) / NS - qlo;
        const char LR_LDS* fa = ldsp + (fst % C::STAGES) * C::STAGE_BYTES;
        const char LR_LDS* fb = fa + C::A_BYTES;
        if constexpr (ROWSTAT) {   // every wave (no branch); the wn == 0 waves publish
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) ss[mb] = frag_sumsq(a[cur][mb], ss[mb]);
        }
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          mfma_chunk(acc[i / C::NB][i % C::NB], b[cur][i % C::NB], a[cur][i / C::NB], (bf16*)nullptr);
          // fragment fi is read after MFMA slot(fi): after the even MFMAs, with the
          // refill loads after the odd ones, where there are MFMAs enough for that
          // (a slot with both stalls the MFMA pipe); spread over all MFMAs otherwise
          constexpr bool DISJ = NMF >= 2 * NF;
#pragma unroll
          for (int fi = 0; fi < NF; ++fi) {
            const int slot = DISJ ? 2 * fi : (NF <= NMF ? fi : fi * NMF / NF);
            if (slot != i) continue;
            if (fi < C::MB)
              a[nxt][fi] = frag<C, C::BM, A_MNC>(fa, wm * C::WTM + fi * 32, fs, lane);
            else
              b[nxt][fi - C::MB] = frag<C, C::BN, B_MNC>(fb, wn * C::WTN + (fi - C::MB) * 32, fs, lane);
          }
          // the sub-step's n loads go out after MFMAs floor(j*NMF/n) + NMF/n - 1, spread evenly
          if (loads_here) {
            constexpr int QMAX = (QA + QB + NS - 1) / NS;
#pragma unroll
            for (int j = 0; j < QMAX; ++j)
              if (j < qn && (j * NMF) / qn + (NMF / qn > 0 ? NMF / qn : 1) - 1 == (i < NMF ? i : NMF - 1))
                issue_q(qlo + j, ra, rb, ba, bb);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // Every load of a real stage has landed.  Sink loads may still be in flight:
    // without epilogue loads nothing else waits for them before the work-group ends.
    if constexpr (std::is_same<std::decay_t<Pre>, NoPre>::value) wait_vmcnt<0>();
  } else {
    pre();
  }
  if constexpr (ROWSTAT) {
    static_assert(!A_MNC, "row statistics need a K-contiguous A");
    __syncthreads();  // rowss may alias the ring: every wave is past its last fragment read
    if (wn == 0) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const float s = ss[mb] + __shfl_xor(ss[mb], 32);
        if (lane < 32) rowss[wm * C::WTM + mb * 32 + lane] = s;
      }
    }
  }
  __syncthreads();
}

template <class C, bool A_MNC, bool B_MNC, bool ROWSTAT, class MapA, class MapB, class Pre = NoPre>
__device__ __forceinline__ void mainloop(const Opnd& oa, const Opnd& ob, const MapA& ma, const MapB& mbm, int m0,
                                         int n0, int kbeg, int K, uint4* lds, float* rowss,
                                         f32x16 (&acc)[C::MB][C::NB], Pre&& pre = Pre{}) {
  if constexpr (C::PIPE) {
    gemm_pipe<C, A_MNC, B_MNC, ROWSTAT>(oa, ob, ma, mbm, m0, n0, kbeg, K, lds, rowss, acc, pre);
  } else {
    gemm_tile<C, A_MNC, B_MNC, ROWSTAT>(oa, ob, ma, mbm, m0, n0, kbeg, K, lds, rowss, acc);
    pre();
  }
}

}  // namespace lr

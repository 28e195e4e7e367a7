// Small-rank forward of the block in one kernel (bf16, g*r <= 256: r = 64 with
// g <= 4, r = 128 with g <= 2, r = 256 with g = 1; SwiGLU's gate/up pair at
// r = 64, 128):
//   h = diag(rstd) . ((x (.) gamma) . A),  z_i = sigma(h_i) (SwiGLU: SiLU(h_gate) * h_up),
//   y_i = z_i . B_i
// BOOST's low-rank layer pairs a d x r and an r x d projection with the
// operations between them (summary, section 2.1) and normalizes with statistics
// accumulated alongside the projection (section 2.2, Online RMSNorm).  At small r
// both GEMMs are thin and the block is bound by HBM: it must read x once and
// write y (and the checkpoint h) once.  Here the rank-r activation z never
// leaves the chip: each work-group owns BM token rows, forms z for them in LDS
// and streams the up-projection out of it.
//
// Work-group of 8 waves in two roles, because on this chip the vector memory
// counter counts stores as well as loads: a wave that waits for a DMA stage
// after issuing output stores also waits for those stores.
//   MMA waves (0-3): the x tiles' DMA into LDS (phase 1), the B fragments'
//     loads into registers (phase 3) and the MFMAs.
//   store waves (4-7): the A'^T tiles' DMA (phase 1), h and z (phase 2) and the
//     y stores (phase 3, from bf16 tiles the MMA waves stage in LDS,
//     double-buffered).  After phase 1 they issue no global loads.
// The row sum of squares comes from the x fragments of the MMA waves.
// Both roles run the same sequence of barriers (one per k step of phase 1, one
// per column tile of phase 3, and the phase boundaries), with every branch on
// the role inside a barrier interval.
//
// Phase 3 reads B in MFMA fragment order (written with A'^T by the fold kernel):
// the operand fragment of 32 columns x 16 k values is 1 KB of consecutive memory,
// lane l's 16 bytes holding column l%32 and k values 8(l/32) .. +7, so every
// fragment is one fully coalesced load into registers.  The MMA waves hold the
// next column tile's fragments while they multiply the current one, so the
// up-projection needs no LDS ring and no wait on other waves' loads.
//
// LDS (bytes from 0):
//   phase 1: a ring of SX x tiles, then a ring of SA A'^T tiles;
//   phases 2-3 (after the ring is drained): z as [BM][64] tiles (K contiguous,
//     swizzled as an MFMA A tile), the partial row sums of squares, then the
//     fp32 staging of h (phase 2) or two bf16 y tiles (phase 3).
#include "lr_kernels.h"
#include "lr_pipe.h"

namespace lr {

// GR = g*r columns of h (phase 1), K3 = rows of each B_i, the up-projection's
// depth (r), NBR = up-projection branches (1 for SwiGLU, else g)
template <int GR, int K3, int NBR>
struct FusedGeo {
  static constexpr int BM = 64;
  static constexpr int BK1 = 64;
  // phase-1 rings: x tiles (from HBM, the MMA waves' DMA) SX stages deep, A'^T
  // tiles (L2-resident, the store waves' DMA) SA deep; each role waits only for
  // its own loads, so the x stream keeps 7-11 stages in flight however large
  // the A'^T tiles are.  Every width takes 64-deep stages: the fixed cost of a
  // stage (wait, barrier, DMA issue) is paid once per 64 k values, which for
  // g*r = 256 measured 10% faster than 32-deep stages in a deeper ring.
  static constexpr int SX = GR == 64 ? 12 : 8;
  static constexpr int SA = GR > 128 ? 3 : 4;
  // phase 1 tile [BM, GR], k split inside the work-group, so that each wave has
  // 4-8 independent accumulators and every LDS fragment is read by one wave (or
  // one wave pair):
  // Each stage holds four 16-deep k sub-steps.
  //   g*r <= 128: MMA wave w the whole tile over sub-step w; NSP = 4 partials,
  //     added in phase 2;
  //   wider: MMA wave w sub-steps w/2 and w/2 + 2 and column half w%2, all BM
  //     rows; the waves of sub-steps 1 and 3 add their partial into the others'
  //     staging in place (four partials would not fit in LDS).
  // NSS = partial row sums of squares (one per wave's set of sub-steps).
  using C1 = PipeCfg<BM, GR, BK1, 2, 2, 2>;  // tile and fragment geometry
  static constexpr bool KSPLIT = GR <= 128;
  static constexpr int NSP = KSPLIT ? 4 : 1, NSS = KSPLIT ? 4 : 2;
  static constexpr int MB1 = 2, NB1 = KSPLIT ? GR / 32 : GR / 64;
  static_assert(C1::KS == 4, "four k sub-steps per stage");
  // phase 3 tile [BM, BN3] per column tile: each MMA wave all BM rows of NB3
  // 32-column blocks; the B fragments of PF column tiles ahead in flight
  // (register buffers NBUF = PF + 1), 48-64 KB per CU.  NB3 = 2 for g*r = 64
  // (256-column tiles, half the tiles and barriers; measured 2-4% faster), else
  // 1 (the wider phase-1 shapes need the registers: 2 measured slower for
  // SwiGLU at r = 64)
  static constexpr int NB3 = GR == 64 ? 2 : 1;
  static constexpr int BN3 = 128 * NB3;
  static constexpr int PF = GR == 64 ? 2 : (K3 == 64 ? 3 : (K3 == 128 ? 2 : 1));
  static constexpr int NBUF = PF + 1;
  using C3 = PipeCfg<BM, 128, 64, 2, 2, 2>;  // z fragment geometry (BK = 64)
  static constexpr int KT = K3 / 64;  // 64-deep k blocks of one branch's z

  static constexpr int XB = C1::A_BYTES, AB = C1::B_BYTES;  // one x / A'^T stage
  static constexpr int A_RING = SX * XB;
  static constexpr int P1 = A_RING + SA * AB;
  static constexpr int ZT = BM * 128;                  // one [BM][64] bf16 z tile
  static constexpr int ZB = NBR * KT * ZT;
  static constexpr int ROWSS = ZB;                     // NSS x BM partial sums of squares
  static constexpr int STG = ZB + 4 * BM * 4;
  static constexpr int STG2_PITCH = GR * 4 + 16;       // fp32 h row + pad
  static constexpr int STG2_BYTES = BM * STG2_PITCH;
  static constexpr int STG3_PITCH = BN3 * 2 + 16;      // bf16 y row + pad
  static constexpr int STG3_BUF = BM * STG3_PITCH;
  static constexpr int P3 = STG + 2 * STG3_BUF;
  static constexpr int P2 = STG + NSP * STG2_BYTES;
  static constexpr int LDS = P1 > P3 ? (P1 > P2 ? P1 : P2) : (P3 > P2 ? P3 : P2);
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(GR % 64 == 0 && GR <= 256 && K3 % 64 == 0 && NBR * K3 <= GR && NBR <= MAX_G, "rank");
  static constexpr int Q1X = DmaTile<C1, BM, false>::Q, Q1A = DmaTile<C1, GR, false>::Q;
  static_assert((SX - 2) * Q1X <= 63 && (SA - 2) * Q1A <= 63, "vmcnt range");
};

__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int GR, int K3, int ACT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fused_fwd(FusedArgs a) {
  constexpr bool SW = ACT == ACT_SWIGLU;
  constexpr int NBR = SW ? 1 : GR / K3;  // up-projection branches
  constexpr int ZC = NBR * K3;           // z columns (SwiGLU: gate and up pair up)
  using G = FusedGeo<GR, K3, NBR>;
  using C1 = typename G::C1;
  using C3 = typename G::C3;
  __shared__ uint4 lds[G::LDS / 16];
  char LR_LDS* ldsp = (char LR_LDS*)(lds);
  const uint32_t lds0 = (uint32_t)(uintptr_t)ldsp;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mma = wave < 4;
  const int w = wave & 3;                 // index within the role
  const int wm = w >> 1, wn = w & 1;      // wide phase 1: k sub-steps wm, wm + 2, column half wn
  const int u = w * 64 + lane;            // store-role thread index 0..255
  const int m0 = blockIdx.x * G::BM;
  const int d = a.d;

  // ---------------------------------------------------------------- phase 1: acc1 = x . A'
  const int nk1 = d / C1::BK;
  constexpr int MB1 = G::MB1, NB1 = G::NB1;
  f32x16 acc1[MB1][NB1];
#pragma unroll
  for (int mb = 0; mb < MB1; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB1; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc1[mb][nb][v] = 0.f;
  // row sums of squares from the x fragments (lane l: row l%32, half l/32 of
  // the fragment's k values)
  float ss[MB1];
#pragma unroll
  for (int mb = 0; mb < MB1; ++mb) ss[mb] = 0.f;

  DmaTile<C1, G::BM, false> dxt;
  DmaTile<C1, GR, false> dat;
  const Opnd ox{a.x, d, a.T, d};
  const Opnd oa{a.Apt, d, GR, d};
  if (mma) {
    dxt.init(ox, MapId{}, m0, w, lane);
    dxt.init_range(ox, m0, 0);
  } else {
    dat.init(oa, MapId{}, 0, w, lane);
    dat.init_range(oa, 0, 0);
  }
  // stages past the end read an empty range, which keeps each role's load count
  // per k step the same; they land in the slot of stage st - S, consumed before
  // the barrier that precedes the issue, and no later stage maps there
  auto issue_x = [&](int st) {
    const bool live = st < nk1;
    dxt.issue(dxt.rsrc(st, live), lds0 + (st % G::SX) * G::XB, w);
  };
  auto issue_a = [&](int st) {
    const bool live = st < nk1;
    dat.issue(dat.rsrc(st, live), lds0 + G::A_RING + (st % G::SA) * G::AB, w);
  };
  if (mma) {
#pragma unroll
    for (int st = 0; st < G::SX - 1; ++st) issue_x(st);
  } else {
#pragma unroll
    for (int st = 0; st < G::SA - 1; ++st) issue_a(st);
  }
  for (int kt = 0; kt < nk1; ++kt) {
    if (mma)
      wait_vmcnt<(G::SX - 2) * G::Q1X>();
    else
      wait_vmcnt<(G::SA - 2) * G::Q1A>();
    lgkm_wait0();
    block_barrier();  // stage kt landed for every wave; stage kt-1's buffers are free
    if (!mma) issue_a(kt + G::SA - 1);
    if (mma) {
      issue_x(kt + G::SX - 1);
      const char LR_LDS* ta = ldsp + (kt % G::SX) * G::XB;
      const char LR_LDS* tb = ldsp + G::A_RING + (kt % G::SA) * G::AB;
      // sub-step(s) s1 of the stage, all BM rows, columns col0 .. col0 + 32*NB1
      const int col0 = G::KSPLIT ? 0 : wn * (GR / 2);
#pragma unroll
      for (int sp = 0; sp < (G::KSPLIT ? 1 : 2); ++sp) {
        const int s1 = G::KSPLIT ? w : wm + 2 * sp;
        uint4 fa[MB1], fb[NB1];
#pragma unroll
        for (int mb = 0; mb < MB1; ++mb) fa[mb] = frag<C1, G::BM, false>(ta, mb * 32, s1, lane);
#pragma unroll
        for (int nb = 0; nb < NB1; ++nb) fb[nb] = frag<C1, GR, false>(tb, col0 + nb * 32, s1, lane);
#pragma unroll
        for (int mb = 0; mb < MB1; ++mb) {
          ss[mb] = frag_sumsq(fa[mb], ss[mb]);
#pragma unroll
          for (int nb = 0; nb < NB1; ++nb) mfma_chunk(acc1[mb][nb], fb[nb], fa[mb], (bf16*)nullptr);
        }
      }
    }
  }
  wait_vmcnt<0>();  // the empty loads of dead stages (both roles)
  lgkm_wait0();
  block_barrier();  // the rings are dead from here on

  // ---------------------------------------------------------------- phase 2: h, z
  // NSP fp32 partials of x . A' ([BM][GR] each, padded rows) and NSS x BM
  // partial sums of squares; the store role adds them in partial order
  float LR_LDS* ssp = reinterpret_cast<float LR_LDS*>(ldsp + G::ROWSS);
  char LR_LDS* stg = ldsp + G::STG;
  typedef float f4 __attribute__((ext_vector_type(4)));
  // lane l holds row l%32 of each 32-row block, columns 8q + 4(l/32) + 0..3 of
  // each 32-column block nb (the swapped operand order of mfma_chunk); ADD:
  // add into what the staging already holds
  auto stage_acc1 = [&](int part, int c0, bool add) {
#pragma unroll
    for (int mb = 0; mb < MB1; ++mb) {
      char LR_LDS* rowp = stg + part * G::STG2_BYTES + (mb * 32 + (lane & 31)) * G::STG2_PITCH + 16 * (lane >> 5);
#pragma unroll
      for (int nb = 0; nb < NB1; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f4 v = {acc1[mb][nb][4 * q], acc1[mb][nb][4 * q + 1], acc1[mb][nb][4 * q + 2], acc1[mb][nb][4 * q + 3]};
          f4 LR_LDS* dst = reinterpret_cast<f4 LR_LDS*>(rowp + (c0 + nb * 32 + 8 * q) * 4);
          if (add) v = *dst + v;
          *dst = v;
        }
    }
  };
  if (mma) {
    if (G::KSPLIT || wm == 0) stage_acc1(G::KSPLIT ? w : 0, G::KSPLIT ? 0 : wn * (GR / 2), false);
#pragma unroll
    for (int mb = 0; mb < MB1; ++mb) {
      ss[mb] += __shfl_xor(ss[mb], 32);
      // the partial of this wave's sub-step(s) (KSPLIT: every wave; else the column-half-0 waves)
      if ((G::KSPLIT || wn == 0) && lane < 32) ssp[(G::KSPLIT ? w : wm) * G::BM + mb * 32 + lane] = ss[mb];
    }
  }
  if constexpr (!G::KSPLIT) {
    lgkm_wait0();
    block_barrier();  // the wm = 0 waves' partial is staged
    if (mma && wm == 1) stage_acc1(0, wn * (GR / 2), true);
  }
  lgkm_wait0();
  block_barrier();
  if (!mma) {
    // each item 4 consecutive z columns of a row (SwiGLU: gate columns c.. and
    // the up columns K3 + c..)
    constexpr int LPR = ZC / 4;
    bf16* h = static_cast<bf16*>(a.h);
#pragma unroll 4
    for (int it = u; it < G::BM * LPR; it += 256) {
      const int rl = it / LPR, c = (it % LPR) * 4;
      // z tile of column c: [BM][64] K-contiguous, 16-byte chunks swizzled as
      // the MFMA A-operand reads expect
      const int zt = c / 64, kk = c % 64;
      // x . A' at (rl, col): the NSP partials added in order
      auto acc_at = [&](int col) {
        float4 v = lds_f4(stg + rl * G::STG2_PITCH + col * 4);
#pragma unroll
        for (int pp = 1; pp < G::NSP; ++pp) {
          const float4 v2 = lds_f4(stg + pp * G::STG2_BYTES + rl * G::STG2_PITCH + col * 4);
          v.x += v2.x; v.y += v2.y; v.z += v2.z; v.w += v2.w;
        }
        return v;
      };
      float ssr = ssp[rl];
#pragma unroll
      for (int pp = 1; pp < G::NSS; ++pp) ssr += ssp[pp * G::BM + rl];
      const float rs = __builtin_amdgcn_rsqf(ssr * a.invD + a.eps);
      if (a.rstd && c == 0 && m0 + rl < a.T) a.rstd[m0 + rl] = rs;
      const float4 v = acc_at(c);
      float hv[4] = {v.x * rs, v.y * rs, v.z * rs, v.w * rs};
      const bool keep = h && m0 + rl < a.T;
      if (keep) store4(h + (int64_t)(m0 + rl) * GR + c, hv[0], hv[1], hv[2], hv[3]);
      if constexpr (ACT == ACT_SILU || SW) {
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = hv[e] * sigmoidf_(hv[e]);
      }
      if constexpr (SW) {
        const float4 w4 = acc_at(K3 + c);
        const float hu[4] = {w4.x * rs, w4.y * rs, w4.z * rs, w4.w * rs};
        if (keep) store4(h + (int64_t)(m0 + rl) * GR + K3 + c, hu[0], hu[1], hu[2], hu[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] *= hu[e];
      }
      const bf16x4 zv = {(bf16)hv[0], (bf16)hv[1], (bf16)hv[2], (bf16)hv[3]};
      const int slot = (kk / 8) ^ kc_swz<128>(rl);
      *reinterpret_cast<bf16x4 LR_LDS*>(ldsp + zt * G::ZT + rl * 128 + slot * 16 + (kk % 8) * 2) = zv;
    }
  }
  lgkm_wait0();
  block_barrier();  // z complete; the h staging and the sums of squares are dead

  // ---------------------------------------------------------------- phase 3: y = z . B
  // column tiles walk branch by branch: tile nt is tile nt % ntpb of branch
  // nt / ntpb; tiles past the end count as tiles past d of the last branch
  const int ntpb = (d + G::BN3 - 1) / G::BN3;
  const int nt_count = NBR * ntpb;
  auto branch_of = [&](int nt) { return min(nt / ntpb, NBR - 1); };
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  // z fragments (both 32-row blocks) in registers for one branch up to r = 128;
  // otherwise (r = 256, or several branches, whose z the tiles walk in turn)
  // they are read from LDS, where z stays through phase 3
  constexpr bool ZREG = K3 <= 128 && NBR == 1;
  uint4 zf[ZREG ? 2 : 1][ZREG ? G::KT : 1][4];
  constexpr int NB3 = G::NB3;
  f32x16 acc3[2][NB3];
  uint4 bb[G::NBUF][G::KT][4][NB3];
  const bf16* Bf = static_cast<const bf16*>(a.Bf);
  // B fragments of this wave's 32 columns of column tile nt: branch br's
  // fragment (column block cb, k16 block kb) starts at element
  // br*d*K3 + ((cb * K3/16 + kb) * 64) * 8; a column block past d (the last
  // tile's upper half when d is an odd multiple of 64, or a tile past the end)
  // reads the last one and feeds y columns that are never stored
  auto load_b = [&](int nt, uint4 (&bf)[G::KT][4][NB3]) {
    const int br = branch_of(nt);
#pragma unroll
    for (int nb = 0; nb < NB3; ++nb) {
      const int cb = min((nt - br * ntpb) * (G::BN3 / 32) + w * NB3 + nb, d / 32 - 1);
      const bf16* fp = Bf + (int64_t)br * d * K3 + ((int64_t)cb * (K3 / 16) * 64 + lane) * 8;
#pragma unroll
      for (int kt = 0; kt < G::KT; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bf[kt][s][nb] = __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4*>(fp + (kt * 4 + s) * 64 * 8));
    }
  };
  if (mma) {
    if constexpr (ZREG) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kt = 0; kt < G::KT; ++kt)
#pragma unroll
          for (int s = 0; s < 4; ++s) zf[mb][kt][s] = frag<C3, G::BM, false>(ldsp + kt * G::ZT, mb * 32, s, lane);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB3; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc3[mb][nb][v] = 0.f;
#pragma unroll
    for (int j = 0; j < G::PF; ++j) load_b(j, bb[j]);
  }
  // store role: one staged [BM][BN3] bf16 tile -> y (BN3/8 lanes per row, 16
  // bytes each); write-back stores, which stream faster than nontemporal ones here
  auto store_tile = [&](int nt) {
    constexpr int LPR = G::BN3 / 8, RPI = 256 / LPR;
    const char LR_LDS* buf = stg + (nt & 1) * G::STG3_BUF;
    const int br = branch_of(nt);
    bf16* y = static_cast<bf16*>(a.y[br]);
    const int ch = u % LPR, col = (nt - br * ntpb) * G::BN3 + ch * 8;
#pragma unroll
    for (int p = 0; p < G::BM / RPI; ++p) {
      const int rl = p * RPI + u / LPR;
      const u32x4 v = *reinterpret_cast<const u32x4 LR_LDS*>(buf + rl * G::STG3_PITCH + ch * 16);
      if (m0 + rl < a.T && col < d) *reinterpret_cast<u32x4*>(y + (int64_t)(m0 + rl) * d + col) = v;
    }
  };
  // MMA role: column tile nt from buffer bc while tile nt+PF loads into bn (the
  // buffer tile nt-1 used); the tile is staged as bf16 in LDS buffer nt & 1.
  // Loads and tiles past the end are not skipped but clamped or masked (see
  // below): a skipped load would make the compiler merge register values with
  // copies, and each copy of a load target waits for every load in flight.
  auto mma_tile = [&](int nt, const uint4 (&bc)[G::KT][4][NB3], uint4 (&bn)[G::KT][4][NB3]) {
    load_b(nt + G::PF, bn);
    const char LR_LDS* zb = ldsp + branch_of(nt) * G::KT * G::ZT;  // this branch's z
#pragma unroll
    for (int kt = 0; kt < G::KT; ++kt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          uint4 za;
          if constexpr (ZREG)
            za = zf[mb][kt][s];
          else
            za = frag<C3, G::BM, false>(zb + kt * G::ZT, mb * 32, s, lane);
#pragma unroll
          for (int nb = 0; nb < NB3; ++nb) mfma_chunk(acc3[mb][nb], bc[kt][s][nb], za, (bf16*)nullptr);
        }
    // lane l holds row l%32 of row block mb, columns 8q + 4(l/32) + 0..3 of each
    // of the wave's 32-column blocks
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      char LR_LDS* rowp = stg + (nt & 1) * G::STG3_BUF + (mb * 32 + (lane & 31)) * G::STG3_PITCH + 8 * (lane >> 5);
#pragma unroll
      for (int nb = 0; nb < NB3; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4 v = {(bf16)acc3[mb][nb][4 * q], (bf16)acc3[mb][nb][4 * q + 1], (bf16)acc3[mb][nb][4 * q + 2],
                            (bf16)acc3[mb][nb][4 * q + 3]};
          *reinterpret_cast<bf16x4 LR_LDS*>(rowp + ((w * NB3 + nb) * 32 + 8 * q) * 2) = v;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc3[mb][nb][v] = 0.f;
      }
    }
  };
  // NBUF tiles per outer step so that every buffer index is a constant.  The
  // tile count is rounded up to a multiple of NBUF: the extra tiles multiply the
  // clamped fragments and stage a tile whose columns all lie past d, which the
  // store role masks.  Each role runs its own loop with one barrier per tile
  // (the same count in both): in a shared loop body the compiler's wait analysis
  // would merge the store role's pending stores with the MMA role's pending
  // loads and wait for all of them before every fragment load.
  const int nt_pad = (nt_count + G::NBUF - 1) / G::NBUF * G::NBUF;
  if (mma) {
    for (int base = 0; base < nt_pad; base += G::NBUF) {
#pragma unroll
      for (int j = 0; j < G::NBUF; ++j) {
        mma_tile(base + j, bb[j], bb[(j + G::PF) % G::NBUF]);
        lgkm_wait0();
        block_barrier();  // tile staged; the previous tile's reads are done, so its buffer is free
      }
    }
  } else {
    for (int nt = 0; nt < nt_pad; ++nt) {
      if (nt > 0) store_tile(nt - 1);  // staged in the previous interval
      lgkm_wait0();
      block_barrier();
    }
    store_tile(nt_pad - 1);
  }
}

// A'^T = (diag(gamma) A)^T [na, d] for A [d, na], and the nbr matrices B_i
// [nb, d] in MFMA fragment order one after another, in one launch.
//   Blocks [0, d/64 * na/64): one 64 x 64 tile of A each, read as rows of
//     16-byte chunks, scaled by gamma, rounded to bf16 once, transposed
//     through LDS and written as rows of A'^T (whole 128-byte runs both ways).
//   The other blocks: one thread per 16-byte chunk of the reordered B: branch
//     i = t / (nb*d/8); within it fragment f = t' / 64 = cb * (nb/16) + kb,
//     lane l = t' % 64: column 32 cb + l%32, k values 16 kb + 8(l/32) .. +7.
struct FoldArgs {
  const bf16* A;
  const bf16* gamma;
  const bf16* B[MAX_G];
  bf16* Apt;
  bf16* Bf;
  int d, na, nb, nbr;
};

__global__ __launch_bounds__(256) void k_fold_fused(FoldArgs a) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  __shared__ bf16 tile[64][64 + 8];  // [j][c]; rows padded by 16 bytes
  const int tiles_c = a.na / 64, tiles_a = (a.d / 64) * tiles_c;
  if ((int)blockIdx.x < tiles_a) {
    const int j0 = ((int)blockIdx.x / tiles_c) * 64, c0 = ((int)blockIdx.x % tiles_c) * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = threadIdx.x + 256 * i, jj = q / 8, cc = (q % 8) * 8;
      const bf16x8 in = *reinterpret_cast<const bf16x8*>(a.A + (int64_t)(j0 + jj) * a.na + c0 + cc);
      const float gj = (float)a.gamma[j0 + jj];
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)in[e] * gj);
      *reinterpret_cast<bf16x8*>(&tile[jj][cc]) = o;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = threadIdx.x + 256 * i, cr = q / 8, jc = (q % 8) * 8;
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = tile[jc + e][cr];
      *reinterpret_cast<bf16x8*>(a.Apt + (int64_t)(c0 + cr) * a.d + j0 + jc) = o;
    }
    return;
  }
  const int64_t t = (int64_t)((int)blockIdx.x - tiles_a) * 256 + threadIdx.x;
  const int64_t per = (int64_t)a.nb * a.d / 8;
  bf16x8 v;
  if (t < a.nbr * per) {
    const int64_t tb = t;
    const int br = (int)(tb / per);
    const int64_t tl = tb % per;
    const int l = (int)(tl % 64);
    const int64_t f = tl / 64;
    const int kb = (int)(f % (a.nb / 16)), cb = (int)(f / (a.nb / 16));
    const int col = cb * 32 + (l & 31), k0 = kb * 16 + 8 * (l >> 5);
    const bf16* B = a.B[br];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = B[(int64_t)(k0 + i) * a.d + col];
    *reinterpret_cast<bf16x8*>(a.Bf + tb * 8) = v;
  }
}

hipError_t launch_fold_fused(const void* A, const void* gamma, const void* const* B, int nbr, void* Apt, void* Bf,
                             int d, int na, int nb, hipStream_t s) {
  if (nbr < 1 || nbr > MAX_G) return hipErrorInvalidValue;
  FoldArgs f{};
  f.A = static_cast<const bf16*>(A);
  f.gamma = static_cast<const bf16*>(gamma);
  for (int i = 0; i < nbr; ++i) f.B[i] = static_cast<const bf16*>(B[i]);
  f.Apt = static_cast<bf16*>(Apt);
  f.Bf = static_cast<bf16*>(Bf);
  f.d = d; f.na = na; f.nb = nb; f.nbr = nbr;
  const int64_t tiles_a = (int64_t)(d / 64) * (na / 64), chunks_b = (int64_t)nbr * nb * d / 8;
  hipLaunchKernelGGL(k_fold_fused, dim3((unsigned)(tiles_a + (chunks_b + 255) / 256)), dim3(256), 0, s, f);
  return hipGetLastError();
}

template <int GR, int K3, int ACT>
static hipError_t launch_fused_g(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_fused_fwd<GR, K3, ACT>), dim3((a.T + 63) / 64), dim3(512), 0, s, a);
  return hipGetLastError();
}

bool fused_fwd_supported(int r, int g, int act) {
  if (act == ACT_SWIGLU) return g == 2 && (r == 64 || r == 128);
  if (act != ACT_IDENTITY && act != ACT_SILU) return false;
  return (r == 64 && g >= 1 && g <= 4) || (r == 128 && (g == 1 || g == 2)) || (r == 256 && g == 1);
}

template <int ACT>
static hipError_t launch_fused_act(const FusedArgs& a, hipStream_t s) {
  switch (a.g * a.r) {
    case 64: return launch_fused_g<64, 64, ACT>(a, s);
    case 128: return a.r == 64 ? launch_fused_g<128, 64, ACT>(a, s) : launch_fused_g<128, 128, ACT>(a, s);
    case 192: return launch_fused_g<192, 64, ACT>(a, s);
    default:
      return a.r == 64 ? launch_fused_g<256, 64, ACT>(a, s)
                       : (a.r == 128 ? launch_fused_g<256, 128, ACT>(a, s) : launch_fused_g<256, 256, ACT>(a, s));
  }
}

hipError_t launch_fused_fwd(const FusedArgs& a, int act, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!fused_fwd_supported(a.r, a.g, act)) return hipErrorInvalidValue;
  if (act == ACT_SWIGLU)
    return a.r == 64 ? launch_fused_g<128, 64, ACT_SWIGLU>(a, s) : launch_fused_g<256, 128, ACT_SWIGLU>(a, s);
  return act == ACT_SILU ? launch_fused_act<ACT_SILU>(a, s) : launch_fused_act<ACT_IDENTITY>(a, s);
}

}  // namespace lr

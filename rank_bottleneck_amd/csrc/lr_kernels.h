// Argument blocks and launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

typedef __bf16 bf16;

enum { ACT_IDENTITY = 0, ACT_SILU = 1, ACT_SWIGLU = 2 };
// DOWN_PLAIN: h = x . A with no normalisation (a low-rank layer's down factor
// on an input that is not normalised)
enum { DOWN_BLOCK = 0, DOWN_PARTIAL = 1, DOWN_PLAIN = 2 };
// up-projection epilogues: y = acc; y = res + acc; y = SiLU(res) * acc
enum { UP_PLAIN = 0, UP_RES = 1, UP_SWIGLU = 2 };
// dx epilogues: the RMSNorm backward; the same plus dres; the SwiGLU backward
// (x = gate, dres = up, dx = dgate, dx2 = dup) with no normalisation
enum { DX_NORM = 0, DX_NORM_RES = 1, DX_SWIGLU = 2 };
constexpr int MAX_G = 8;

struct DownArgs {
  const void* x;      // [T, d]
  const void* Ap;     // [d, g*r], gamma folded in
  int T, d, r, g, act, mode;
  float invD, eps;
  void* h;            // [T, g*r] or null
  void* z;            // [T, g*r] (SwiGLU: [T, r]); identity: used only when h is null
  float* partial;     // DOWN_PARTIAL: [T, g*r]
  float* sumsq;       // DOWN_PARTIAL: [T]
  float* rstd;        // DOWN_BLOCK: [T], the rows' rstd (tile column 0 writes it), or null
  int tile0;          // first tile of this launch (launch_down sets it)
};

// Small-rank forward: split-K down-projection into fp32 partials.
struct SplitDownArgs {
  const void* x;      // [T, d]
  const void* Apt;    // [g*r, d]: (diag(gamma) A)^T, K-contiguous
  int T, d, gr;
  int nsplit, ksplit; // token-independent split of K = d (ksplit a multiple of the k step)
  float* partial;     // [nsplit][T][g*r]
  float* sumsq;       // [nsplit][T]
};

// Small-rank forward in one kernel (g*r <= 256, see fused_fwd_supported): x,
// A'^T [g*r, d] (gamma folded in), the B_i [r, d] in MFMA fragment order
struct FusedArgs {
  const void* x;      // [T, d]
  const void* Apt;    // [g*r, d]: (diag(gamma) A)^T, K-contiguous
  const void* Bf;     // the n_up matrices B_i [r, d] in MFMA fragment order, one after another
  void* y[MAX_G];     // n_up x [T, d]
  void* h;            // [T, g*r] or null
  float* rstd;        // [T] or null: the rows' rstd
  int T, d, r, g;
  float invD, eps;
};

struct UpArgs {
  const void* z;      // A operand source; branch i starts at column i*r
  int64_t ldz;
  const void* B[MAX_G];
  void* y[MAX_G];
  const void* res[MAX_G];  // residual_i [T, d] added to y_i (all null: none); may equal y[i]
  // swiglu != 0: res[i] holds the gate and y_i = SiLU(res_i) * acc; y2[i], when
  // non-null, receives acc as well
  int swiglu;
  void* y2[MAX_G];
  int T, d, r;        // d: the output width (columns of B_i and y_i)
};

struct DzArgs {
  const void* dy[MAX_G];
  const void* B[MAX_G];
  const void* h;      // saved pre-activation [T, g*r]
  const float* rstd;  // [T], or null: no normalisation (the factor is 1)
  void* dh;           // [T, g*r]   rstd * dh
  void* z;            // sigma(h): [T, g*r] (SiLU) or [T, r] (SwiGLU); unused for identity
  float* spart;       // [T, spstride]: partials of S' (columns past the partial count unused), or null
  int spstride;
  int T, d, r, g, act;
  int tile0;          // first tile of this launch (launch_dz sets it)
};

struct WgradArgs {
  const void* z;      // sigma(h) source, branch i at column i*r, leading dim ldz
  int64_t ldz;
  const void* dy[MAX_G];
  float* dB[MAX_G];
  const void* x;
  const void* dh;
  const void* A;
  const void* gamma;  // null: no normalisation, dA = M and no dgamma (A unused)
  float* dA;
  float* dgamma;      // [d]: written by the reductions (launch_wgrad_reduce)
  float* gpart;       // [d, ngpart]: dgamma partials of an unsplit launch_wgrad
  int ngpart;
  int gparts_used;    // split-tile plan with gamma: partials per row that k_wgrad_reduce_tiles sums into dgamma
  int T, d, r, g, n_up;     // d: width of x (rows of dA)
  int dn;                   // width of dy_i (columns of dB_i)
  int nsplit, ksplit;       // token splits and tokens per split (a multiple of the k step)
  float* wpart;             // nsplit x part_stride fp32 partial tiles (nsplit > 1), or the stream-K slots
  int64_t part_stride;      // n_up*r*dn + d*g*r
  int64_t part_offA;        // n_up*r*dn
  // stream-K (streamk != 0): G work-groups split tiles*KS k steps evenly, the first R
  // taking Q+1 and the rest Q; each (sequence position, covering work-group) writes a
  // BM x BN fp32 slot at wpart[(position*maxseg + ordinal) * BM*BN].  Position p
  // holds tile (p % S) * (tiles / S) + p / S (S = 1: tile p).
  int streamk, sk_G, sk_Q, sk_R, sk_KS, sk_maxseg, sk_S, sk_tiles;
  // split_tiles S > 0 (nsplit == 2): only the first S tiles (all dB tiles) run
  // as two token halves, writing BM x BN fp32 slots wpart[(half * S + tile) *
  // BM*BN] that k_wgrad_reduce_tiles adds; the other tiles run whole and write
  // dB / dA directly.  Work-group ids: per XCD, its share of the whole tiles
  // first, then its share of the halves.
  int split_tiles;
};

// How the token-reduced weight gradients are split.
struct WgradPlan {
  int streamk;        // 1: stream-K over (tile, k step); 0: nsplit equal token splits
  int nsplit;         // token splits when !streamk (1 = one pass, no reduction)
  int split_tiles;    // > 0: only this many (dB) tiles split in two (see WgradArgs)
  int G, Q, R, KS, maxseg, tiles;
  int S;              // stream-K tile interleave (see WgradArgs)
  int64_t part_floats;  // fp32 partial floats the plan needs in the workspace
};

struct DxArgs {
  const void* dh;
  const void* A;
  const void* x;
  const void* gamma;
  const float* rstd;
  const float* spart;  // [T, spstride], the first nspart columns of each row used
  int nspart, spstride;
  void* dx;
  const void* dres;    // [T, d] added to dx (the residual path's gradient), or null; may equal dx
  // swiglu != 0: the SwiGLU backward instead of the RMSNorm one: x holds the
  // gate and dres the up values, dx receives dgate and dx2 dup (both may equal
  // their input); gamma, rstd and the S' partials are unused
  int swiglu;
  void* dx2;
  int T, d, r, g;
  float invD;
};

template <typename E> hipError_t launch_rms_stats(const void* x, const void* gamma, void* y, float* sumsq,
                                                  float* rstd, int T, int d, float invD, float eps, hipStream_t s);
template <typename E> hipError_t launch_fold_gamma(const void* A, const void* gamma, void* Ap, int d, int n,
                                                   hipStream_t s);
template <typename E> hipError_t launch_down(const DownArgs& a, hipStream_t s);
// whether launch_down picks its 64-row tiles for this shape (fewer 256 x 256 tiles than CUs)
template <typename E> bool down_uses_skinny(int T, int r, int g, bool gateup);
template <typename E> hipError_t launch_up(const UpArgs& a, int n_up, hipStream_t s);
// h = rstd * sum of the nsplit partials, z = sigma(h); partial [nsplit][T][g*r], sumsq [nsplit][T];
// rstd [T] written when non-null
template <typename E> hipError_t launch_finish(const float* partial, const float* sumsq, void* h, void* z,
                                               float* rstd, int T, int r, int g, int act, float invD, float eps,
                                               int nsplit, hipStream_t s);
// A'^T [n, d] = (diag(gamma) A)^T for A [d, n]
template <typename E> hipError_t launch_fold_gamma_t(const void* A, const void* gamma, void* Apt, int d, int n,
                                                     hipStream_t s);
// Number of K splits of the small-rank forward path for this shape, 0 when the
// regular down-projection is used.
template <typename E> int small_rank_splits(int T, int d, int r, int g, int act);
template <typename E> hipError_t launch_down_split(const SplitDownArgs& a, hipStream_t s);
// whether the one-kernel small-rank forward serves these dims (bf16 only):
// identity / SiLU with g*r <= 256 (r = 64: g <= 4; r = 128: g <= 2; r = 256:
// g = 1), SwiGLU with r = 64 or 128
bool fused_fwd_supported(int r, int g, int act);
hipError_t launch_fused_fwd(const FusedArgs& a, int act, hipStream_t s);
// A'^T = (diag(gamma) A)^T [na, d] for A [d, na], and the nbr matrices B[i]
// [nb, d] in MFMA fragment order (fragment of 32 columns x 16 k values = 64
// lanes x 8 consecutive k), one after another (bf16)
hipError_t launch_fold_fused(const void* A, const void* gamma, const void* const* B, int nbr, void* Apt, void* Bf,
                             int d, int na, int nb, hipStream_t s);
template <typename E> hipError_t launch_dz(const DzArgs& a, int n_up, hipStream_t s);
template <typename E> hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s);
// sums the split partials (or stream-K slots) of launch_wgrad into dB and dA and
// forms dgamma (nothing to do when nsplit == 1 without stream-K); with split
// tiles it forms dgamma from gpart's first gparts_used partials of each row
template <typename E> hipError_t launch_wgrad_reduce(const WgradArgs& a, hipStream_t s);
template <typename E> hipError_t launch_dx(const DxArgs& a, hipStream_t s);
hipError_t launch_sum_parts(const float* parts, float* out, int n, int nparts, int stride, hipStream_t s);
template <typename E> int dz_nparts(int r);
// row stride of the S' partials: the count rounded up to whole float4s
inline int spart_stride(int nparts) { return (nparts + 3) & ~3; }
template <typename E> int wgrad_nparts(int gr);
template <typename E> int gemm_bk();
template <typename E> int wgrad_nparts_used(int gr, bool reduced);
// dn: width of dy_i and dB_i (d for the block)
template <typename E> WgradPlan wgrad_plan(int T, int d, int r, int g, int n_up, int dn);

}  // namespace lr

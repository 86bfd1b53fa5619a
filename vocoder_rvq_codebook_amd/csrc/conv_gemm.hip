// Implicit-GEMM causal convolution on the MFMA units (gfx950): fp32 MFMA, or
// fp16 MFMA with fp16 operands or with fp32 operands split into fp16 pairs.
//
// One kernel family serves every dense contraction of the decoder:
//  - causal dilated Conv1d (pre-conv, conv_pre, the AMP convs of every BigVGAN
//    stage): A = weights [Cout][tap][Cin], B = input rows shifted by
//    (k-1-tap)*dil, rows before the chunk read from the stream's history slot;
//  - causal ConvTranspose1d with kernel 2 x stride: each output phase p is a
//    2-tap conv of the input (tap 0 -> row t-1, tap 1 -> row t), and the s
//    phases are stacked along M, so [T][s*Cout] written channels-last is
//    exactly the upsampled [T*s][Cout] (blixt/phonon, Weights: a transposed
//    conv becomes one GEMM per output phase that gathers its inputs);
//  - transformer linears (k = 1).
// The epilogue fuses bias, GELU, residual add, the multi-receptive-field mean,
// one to four Snake outputs (x + sin^2(alpha x)/alpha), and the write of each
// output's last rows into the stream's next state.
//
// Each output element's reduction order depends only on (tap, channel): the K
// loop order is fixed, and split-K splits only between accumulation groups and
// folds them in order, so results are bitwise independent of batch, chunking,
// tile shape and split.

#include <algorithm>
#include <type_traits>

#include "common.h"


namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// IGLP_: the compiler's MFMA/LDS interleaving strategy for the K-step body
// (__builtin_amdgcn_iglp_opt), or -1 for none; chosen per tile by measurement.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int IGLP_ = -1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, BK = BK_, IGLP = IGLP_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int LDK = BK + 4;  // padded LDS row (floats): 16-byte rows shift 4 banks
  static constexpr int KV = BK / 4;   // float4 per row per k-step
  static constexpr int A_F4 = BM * KV;
  static constexpr int B_F4 = BN * KV;
  static constexpr int A_LD = (A_F4 + NT - 1) / NT;
  static constexpr int B_LD = (B_F4 + NT - 1) / NT;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
};

// 4 int8 weights (one 32-bit word) times their group's scale, in fp32 (exact:
// an 8-bit integer times an fp16 value).
__device__ __forceinline__ f32x4 dequant4(int w, float sc) {
  return (f32x4){(float)((w << 24) >> 24) * sc, (float)((w << 16) >> 24) * sc, (float)((w << 8) >> 24) * sc,
                 (float)(w >> 24) * sc};
}

// Snake x + sin^2(a x)/a.  The sine is the hardware instruction (argument in
// revolutions) applied to the angle reduced to [-1/2, 1/2] revolution: the
// subtraction of the nearest integer is exact, so the only angle error is the
// rounding of a*x/(2 pi), the same size as the rounding of a*x itself.
__device__ __forceinline__ float snake1(float v, float a) {
  const float t = (a * v) * 0.159154943091895336f;
  const float s = __builtin_amdgcn_sinf(t - rintf(t));
  return v + (s * s) * __builtin_amdgcn_rcpf(a);
}

__device__ __forceinline__ float gelu1(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Values of the epilogue of output rows m..m+3 (GEMM columns) of GEMM row g
// read from tensors other than the GEMM's own: the residual and the
// multi-receptive-field partial sums.  Loaded apart from the arithmetic so
// that a thread can issue the loads of several elements before its first
// store (a store may alias any of them, so the compiler keeps them in order).
struct EpiLoads {
  f32x4 resid, mrf, mrf2;
};

__device__ __forceinline__ size_t epi_oidx(const ConvParams& p, int m, int g) {
  const int ph = m / p.cout;
  return ((size_t)g * p.phases + ph) * p.cout + (m - ph * p.cout);
}

__device__ __forceinline__ EpiLoads epilogue_loads(const ConvParams& p, int m, int g) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const size_t oidx = epi_oidx(p, m, g);
  const int mrf_mode = p.mrf_mode;
  EpiLoads e;
  e.resid = p.resid ? ld4(p.resid + oidx) : z;
  e.mrf = (mrf_mode == MRF_ACCUM || mrf_mode == MRF_LAST) ? ld4(p.mrf + oidx) : z;
  e.mrf2 = (mrf_mode == MRF_LAST && p.mrf2) ? ld4(p.mrf2 + oidx) : z;
  return e;
}

// Per-column parameters (bias; each output's Snake alpha) read from the
// weights in global memory.
struct EpiColsGlobal {
  const ConvParams& p;
  int m;
  __device__ __forceinline__ f32x4 bias() const { return ld4(p.bias + m); }
  __device__ __forceinline__ f32x4 alpha(int o) const { return ld4(p.out[o].alpha + m); }
};

// Epilogue of output rows m..m+3 of GEMM row g, given the reduced sum `acc`
// and the loaded values `e`: bias, activation, residual, multi-receptive-
// field mean, then up to four stores, each optionally through Snake and each
// optionally also written to the stream's state tail.  Shared by the GEMM
// and the split-K reduction, so both give the same bits.  Returns the first
// output's value (as stored when it is fp32).
template <class Cols>
__device__ __forceinline__ f32x4 epilogue_apply(const ConvParams& p, int m, int g, f32x4 acc, const EpiLoads& e,
                                                const Cols& cols) {
  const int nout_rows = p.nin * p.phases;
  const int ph = m / p.cout;
  const int c = m - ph * p.cout;
  f32x4 v = acc * p.acc_scale + cols.bias();
  if (p.act == ACT_GELU) {
    v.x = gelu1(v.x); v.y = gelu1(v.y); v.z = gelu1(v.z); v.w = gelu1(v.w);
  }
  const size_t orow = (size_t)g * p.phases + ph;
  const size_t oidx = orow * p.cout + c;
  if (p.resid) v = v + e.resid;
  f32x4 sm = v;
  // (fields read into scalars first: reading them in place let the optimizer
  // copy part of the argument block to private memory in some kernels)
  const int mrf_mode = p.mrf_mode;
  const float* mrf2 = p.mrf2;
  const float mrf_div = p.mrf_div;
  if (mrf_mode == MRF_FIRST) {
    sm = v;
  } else if (mrf_mode == MRF_ACCUM) {
    sm = e.mrf + v;
  } else if (mrf_mode == MRF_LAST) {
    // ((block 0 + block 1) + this block): the order of the running sum
    f32x4 acc = e.mrf;
    if (mrf2) acc = acc + e.mrf2;
    sm = (acc + v) / mrf_div;
  } else if (mrf_mode == MRF_ONLY) {
    sm = v / mrf_div;
  }
  const int b = g / p.nin;
  const int no = (g - b * p.nin) * p.phases + ph;
  f32x4 first = v;
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    if (o >= p.nout) break;
    const EpiOut& eo = p.out[o];
    f32x4 val = eo.src ? sm : v;
    if (eo.alpha) {
      const f32x4 a = cols.alpha(o);
      val.x = snake1(val.x, a.x); val.y = snake1(val.y, a.y);
      val.z = snake1(val.z, a.z); val.w = snake1(val.w, a.w);
    }
    if (eo.dst) {
      if (eo.half)
        *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(eo.dst) + oidx) =
            (f16x4){(_Float16)val.x, (_Float16)val.y, (_Float16)val.z, (_Float16)val.w};
      else
        st4(eo.dst + oidx, val);
    }
    if (eo.hist && no >= nout_rows - eo.H) {
      st4(eo.hist + (size_t)b * p.sstride + (size_t)(eo.H - nout_rows + no) * p.cout + c, val);
    }
    if (o == 0) first = val;
  }
  return first;
}

__device__ __forceinline__ f32x4 epilogue4(const ConvParams& p, int m, int g, f32x4 acc) {
  return epilogue_apply(p, m, g, acc, epilogue_loads(p, m, g), EpiColsGlobal{p, m});
}

// Reduction values per accumulation group (see the two-level accumulation
// below); split-K splits only at group boundaries.
constexpr int GROUP_K = VOC_GROUP_K;

// Sum of the group partials of output elements m..m+3 of row g, in group
// order from zero; loads issued 8 at a time.
__device__ __forceinline__ f32x4 fold_groups(const ConvParams& p, int m, int g, int ngroups) {
  const size_t stride = (size_t)p.rows * p.M;
  const float* src = p.partial + (size_t)g * p.M + m;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int j = 0;
  for (; j + 8 <= ngroups; j += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld4(src + (size_t)(j + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; j < ngroups; ++j) acc += ld4(src + (size_t)j * stride);
  return acc;
}

// Per-column parameters staged in LDS by epilogue_tile: row 0 the bias, row
// 1 + o output o's Snake alpha, BM floats each, for the tile's columns.
struct EpiColsLds {
  const float* P;
  int c;   // column within the tile
  int bm;  // floats per row
  __device__ __forceinline__ f32x4 bias() const { return ld4(P + c); }
  __device__ __forceinline__ f32x4 alpha(int o) const { return ld4(P + (1 + o) * bm + c); }
};

// LDS floats epilogue_tile needs: the [BN][BM] tile and 5 rows of BM column
// parameters.
template <class C>
constexpr int epi_lds_floats() { return C::BM * C::BN + 5 * C::BM; }

// Epilogue of a whole tile through LDS.  The accumulators go to an fp32
// [BN][BM] tile in LDS (16-byte chunks of 4 GEMM columns, chunk c of row r
// stored at c ^ (r & 7): conflict-free both for the fragment writes, 8 rows
// of one chunk, and for the row reads, 8 chunks of one row), and the tile's
// bias and Snake alphas to 5 rows after it; then thread t runs the epilogue
// of chunks t, t + NT, ... in row-major order, so a wave's loads and stores
// cover whole rows instead of 16-row columns.  The chunks are taken in
// batches of up to MAXB: every residual and multi-receptive-field load of a
// batch is issued before its first store, so a batch waits on memory once.
// Each element gets the same epilogue on the same values: the same bits as
// epilogue4 called from the fragments.  Rows from g_end on are not written.
// The caller has synchronised the block: LDS may be overwritten once every
// wave has finished reading it.
template <class C, int MAXB = 4>
__device__ __forceinline__ void epilogue_tile(const ConvParams& p, float* T, const f32x4 (&acc)[C::FM][C::FN],
                                              int m0, int g0, int g_end, int wm, int wn, int lane, int tid) {
  constexpr int CH = C::BM / 4;
  static_assert(CH % 8 == 0, "row chunks: a multiple of 8");
  const int lr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = wn * C::WTN + j * 16 + lr;
      const int c = (wm * C::WTM + i * 16) / 4 + q;
      st4(T + (r * CH + (c ^ (r & 7))) * 4, acc[i][j]);
    }
  if constexpr (MAXB == 1) {
    // one chunk at a time, column parameters read from the weights
    __syncthreads();
    for (int idx = tid; idx < C::BN * CH; idx += C::NT) {
      const int r = idx / CH, c = idx - r * CH;
      const int g = g0 + r, m = m0 + 4 * c;
      if (g < g_end && m < p.M) epilogue4(p, m, g, ld4(T + (r * CH + (c ^ (r & 7))) * 4));
    }
    return;
  }
  float* P = T + C::BM * C::BN;
#pragma unroll
  for (int o = 0; o < 5; ++o) {
    const float* src = o == 0 ? p.bias : (o - 1 < p.nout ? p.out[o - 1].alpha : nullptr);
    if (!src) continue;
    for (int c = tid; c < CH; c += C::NT)
      if (m0 + 4 * c < p.M) st4(P + o * C::BM + 4 * c, ld4(src + m0 + 4 * c));
  }
  __syncthreads();
  constexpr int ITERS = (C::BN * CH + C::NT - 1) / C::NT;
  constexpr int NB = (ITERS + MAXB - 1) / MAXB;  // batches
  constexpr int EB = (ITERS + NB - 1) / NB;  // chunks per batch
#pragma unroll
  for (int u0 = 0; u0 < ITERS; u0 += EB) {
    EpiLoads e[EB];
    bool on[EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int idx = tid + (u0 + u) * C::NT;
      const int r = idx / CH, c = idx - r * CH;
      const int g = g0 + r, m = m0 + 4 * c;
      on[u] = u0 + u < ITERS && idx < C::BN * CH && g < g_end && m < p.M;
      if (on[u]) e[u] = epilogue_loads(p, m, g);
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      if (!on[u]) continue;
      const int idx = tid + (u0 + u) * C::NT;
      const int r = idx / CH, c = idx - r * CH;
      epilogue_apply(p, m0 + 4 * c, g0 + r, ld4(T + (r * CH + (c ^ (r & 7))) * 4), e[u],
                     EpiColsLds{P, 4 * c, C::BM});
    }
  }
}

// SPLIT = false: one block computes a whole output tile and runs the epilogue.
// SPLIT = true: blocks are (tile, split) pairs; a split owns a contiguous,
// non-empty range of accumulation groups and stores each group's partial sum,
// unreduced, to p.partial[group][row][M]; splitk_reduce_kernel then folds the
// groups in order and runs the same epilogue.  Every group's partial is the
// same MFMA chain in both modes, so both modes give the same bits.
template <class C, bool SPLIT, bool Q8>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(4))) void conv_gemm_kernel(const ConvParams p) {
  // double-buffered A and B tiles; after the K loop the same LDS holds the
  // epilogue's [BN][BM] tile
  constexpr int AB_FLOATS = 2 * (C::BM + C::BN) * C::LDK;
  constexpr int T_FLOATS = SPLIT ? 0 : epi_lds_floats<C>();
  __shared__ __attribute__((aligned(16))) float smem[AB_FLOATS > T_FLOATS ? AB_FLOATS : T_FLOATS];
  constexpr int A_OFF = 0, B_OFF = 2 * C::BM * C::LDK;  // buffer b of A at A_OFF + b * BM * LDK

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::WAVES_M;
  const int wn = wave / C::WAVES_M;

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of tiles, M-tiles fastest, so the blocks
  // that share an input tile share an L2.
  const int mtiles = (p.M + C::BM - 1) / C::BM;
  int tile_id;
  {
    const int L = blockIdx.x, nb = gridDim.x;
    const int xcd = L & 7, i = L >> 3;
    const int per = nb >> 3, extra = nb & 7;
    tile_id = xcd * per + (xcd < extra ? xcd : extra) + i;
  }
  int split = 0;
  if (SPLIT) {
    split = tile_id % p.splits;
    tile_id /= p.splits;
  }
  const int mt = tile_id % mtiles;
  const int nt = tile_id / mtiles;
  const int m0 = mt * C::BM;
  const int g0 = nt * C::BN;

  const int cin = p.cin;
  const int ktaps = p.k, dil = p.dil;  // (lambdas below read locals, not the by-value argument)
  const int ksteps_per_tap = cin / C::BK;
  const int nsteps_all = p.k * ksteps_per_tap;
  constexpr int GROUP_STEPS = GROUP_K / C::BK;
  // K-steps [s_begin, nsteps) of this block: all of them, or one split's groups
  int s_begin = 0, nsteps = nsteps_all;
  if (SPLIT) {
    const int ngroups = (nsteps_all + GROUP_STEPS - 1) / GROUP_STEPS;
    const int gps = (ngroups + p.splits - 1) / p.splits;
    s_begin = min(split * gps, ngroups) * GROUP_STEPS;
    nsteps = min(min((split + 1) * gps, ngroups) * GROUP_STEPS, nsteps_all);
    if (s_begin >= nsteps) return;
  }

  // Per-thread load slots.  Each thread loads the same rows at every K-step;
  // only a uniform offset (tap shift and channel block) changes, so the row
  // base pointers are computed once.  A row whose shifted position falls
  // before the chunk reads the stream's history slot instead: both bases are
  // kept and selected per step, without branches.  Rows past the end clamp to
  // the last row (their outputs are never stored).
  // int8 weights use the same slots: 4 values (one word) and their scale
  const float* a_base[C::A_LD];
  const int8_t* q_base[C::A_LD];
  const _Float16* s_base[C::A_LD];
  int a_lds[C::A_LD], q_col[C::A_LD];
  const size_t ktot = (size_t)p.k * cin;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    int idx = tid + i * C::NT;
    if (C::A_F4 % C::NT != 0 && idx >= C::A_F4) idx = C::A_F4 - 1;  // duplicate load, same value
    const int row = idx / C::KV, col = (idx % C::KV) * 4;
    a_base[i] = p.w + (size_t)(m0 + row) * ktot + col;
    if constexpr (Q8) {
      q_base[i] = reinterpret_cast<const int8_t*>(p.w) + (size_t)(m0 + row) * ktot + col;
      s_base[i] = reinterpret_cast<const _Float16*>(p.wscale) + (size_t)(m0 + row) * (ktot / 32);
    }
    q_col[i] = col;
    a_lds[i] = row * C::LDK + col;
  }
  const float* bx[C::B_LD];
  const float* bh[C::B_LD];
  int bn[C::B_LD], b_lds[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    int idx = tid + i * C::NT;
    if (C::B_F4 % C::NT != 0 && idx >= C::B_F4) idx = C::B_F4 - 1;
    const int row = idx / C::KV, col = (idx % C::KV) * 4;
    const int g = min(g0 + row, p.rows - 1);
    const int b = g / p.nin;
    const int n = g - b * p.nin;
    bn[i] = n;
    bx[i] = p.x + (size_t)g * cin + col;
    bh[i] = p.hin ? p.hin + (size_t)b * p.sstride + (ptrdiff_t)(p.hin_rows + n) * cin + col : bx[i];
    b_lds[i] = row * C::LDK + col;
  }

  f32x4 ra[C::A_LD], rb[C::B_LD];
  int rq[C::A_LD];
  float rs[C::A_LD];

  auto gload = [&](int s) {
    const int tap = s / ksteps_per_tap;
    const int c0 = (s - tap * ksteps_per_tap) * C::BK;
    const int shift = (ktaps - 1 - tap) * dil;
    const ptrdiff_t aoff = (ptrdiff_t)tap * cin + c0;
    const ptrdiff_t boff = c0 - (ptrdiff_t)shift * cin;
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) {
        rq[i] = *reinterpret_cast<const int*>(q_base[i] + aoff);
        rs[i] = (float)s_base[i][(aoff + q_col[i]) >> 5];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) ra[i] = ld4(a_base[i] + aoff);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) rb[i] = ld4((bn[i] >= shift ? bx[i] : bh[i]) + boff);
  };
  auto lstore = [&](int buf) {
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) st4(&smem[A_OFF + buf * (C::BM * C::LDK) + a_lds[i]], dequant4(rq[i], rs[i]));
    } else {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) st4(&smem[A_OFF + buf * (C::BM * C::LDK) + a_lds[i]], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) st4(&smem[B_OFF + buf * (C::BN * C::LDK) + b_lds[i]], rb[i]);
  };

  // MFMA 16x16x4 f32: lane l supplies A[l%16][k] and B[k][l%16] with
  // k = l/16.  Lane group l/16 owns 4 consecutive k of a 16-wide slab, read
  // as one float4, and the 4 MFMAs of the slab take its components in turn.
  const int lr = lane & 15;
  const int lk = (lane >> 4) * 4;

  // Two-level accumulation: the MFMA chain of one group of GROUP_K reduction
  // values (64 MFMAs deep at most) starts from zero, and each group's partial
  // sum is added to `acc`.  A single chain over all k*cin values loses about
  // 4x more precision; the grouping depends only on the K index, so every
  // tile shape reduces each output in the same order.
  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto mma_step = [&](int cur, f32x4 (&part)[C::FM][C::FN], auto first) {
    if constexpr (C::IGLP >= 0) __builtin_amdgcn_iglp_opt(C::IGLP);
    const float* Ab = &smem[A_OFF + cur * (C::BM * C::LDK)];
    const float* Bb = &smem[B_OFF + cur * (C::BN * C::LDK)];
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 16) {
      f32x4 af[C::FM], bf[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) af[i] = ld4(&Ab[(wm * C::WTM + i * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bf[j] = ld4(&Bb[(wn * C::WTN + j * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if (decltype(first)::value && kk == 0 && q == 0)
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][q], bf[j][q], (f32x4){0.f, 0.f, 0.f, 0.f},
                                                                0, 0, 0);
            else
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][q], bf[j][q], part[i][j], 0, 0, 0);
          }
    }
  };

  gload(s_begin);
  lstore(s_begin & 1);
  __syncthreads();
  for (int gs = s_begin; gs < nsteps; gs += GROUP_STEPS) {
    const int ge = min(gs + GROUP_STEPS, nsteps);
    f32x4 part[C::FM][C::FN];
    for (int s = gs; s < ge; ++s) {
      const int cur = s & 1;
      if (s + 1 < nsteps) gload(s + 1);
      if (s == gs)
        mma_step(cur, part, std::true_type{});
      else
        mma_step(cur, part, std::false_type{});
      if (s + 1 < nsteps) lstore(cur ^ 1);
      __syncthreads();
    }
    if (SPLIT) {
      // store this group's partial sums: partial[group][g][m]
      const size_t gbase = (size_t)(gs / GROUP_STEPS) * p.rows;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = m0 + wm * C::WTM + i * 16 + (lane >> 4) * 4;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int g = g0 + wn * C::WTN + j * 16 + lr;
          if (g < p.rows) st4(p.partial + (gbase + g) * p.M + m, part[i][j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] += part[i][j];
    }
  }
  if (SPLIT) return;

  // (the K loop ended on a block barrier: every wave is done with As and Bs)
  epilogue_tile<C>(p, smem, acc, m0, g0, p.rows, wm, wn, lane, tid);
}

// Fold the split-K group partials of one output element (4 consecutive M)
// in group order, starting from zero as the unsplit loop does, then run the
// epilogue.  A separate launch: the kernel boundary makes every partial
// visible, which on a multi-XCD GPU is far cheaper than device-scope fences
// in the GEMM blocks.
__global__ void splitk_reduce_kernel(const ConvParams p, int ngroups) {
  const int M4 = p.M / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)p.rows * M4) return;
  const int g = (int)(idx / M4);
  const int m = (int)(idx - (long long)g * M4) * 4;
  epilogue4(p, m, g, fold_groups(p, m, g, ngroups));
}

// The same fold and epilogue for a GEMM whose first output feeds a LayerNorm
// (one phase, M = ln.d): one block per row, one float4 per thread as above;
// the row's epilogue values stay in registers for the LayerNorm, so the row
// is not read back.  The same values and order as splitk_reduce_kernel then
// layernorm_kernel.
template <int NV>
__global__ __launch_bounds__(64 * NV) void splitk_reduce_ln_kernel(const ConvParams p, int ngroups, const LnArgs ln) {
  __shared__ float red[64 * NV + 1];
  const int g = blockIdx.x;
  const int m = 4 * threadIdx.x;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (m < p.M) v = epilogue4(p, m, g, fold_groups(p, m, g, ngroups));
  layernorm_block<NV>(ln, v, g, red);
}

// ---------------------------------------------------------------------------
// Few-row GEMM (at most 16 GEMM rows: the transformer, upsampling and conv_pre
// linears of short chunks), fp32.  These launches stream their weights once
// and do almost no arithmetic.  A block owns 16 output columns (M) and every
// accumulation group of them; wave w computes groups w, w + waves, ...,
// reading its weight rows straight from global memory into MFMA operand
// registers (no LDS staging; 8 16-wide slabs of loads in flight, 4 for int8
// weights), and stores each group's partial sum to LDS.  After one barrier
// the first wave sums the partials in group order from zero and runs the
// epilogue: no split-K partials in HBM and no fold launch.  Operands, MFMAs
// and their order are those of conv_gemm_kernel (lane l holds A[l%16][k] and
// B[k][l%16] for the 4 consecutive k of lane group l/16 in a 16-wide slab,
// the slab's 4 MFMAs take them in turn, each group's chain starts from
// zero), and the fold is fold_groups': the same bits as every other tile.
// ---------------------------------------------------------------------------
template <bool Q8>
__global__ __launch_bounds__(1024) void conv_gemm_rows_kernel(const ConvParams p, int ngroups) {
  constexpr int SLABS = Q8 ? 4 : 8;  // 16-wide slabs of loads in flight per wave
  extern __shared__ f32x4 red[];     // [ngroups][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int m0 = blockIdx.x * 16;
  const int lr = lane & 15, lk = (lane >> 4) * 4;
  const int cin = p.cin, ktaps = p.k, dil = p.dil;
  const int K = ktaps * cin;
  // B: this lane's GEMM row (rows past the end clamp to the last row; their
  // outputs are never stored), and its history row for taps that reach
  // before the chunk
  const int g = min(lr, p.rows - 1);
  const int b = g / p.nin;
  const int n = g - b * p.nin;
  const float* bx = p.x + (size_t)g * cin + lk;
  const float* bh = p.hin ? p.hin + (size_t)b * p.sstride + (ptrdiff_t)(p.hin_rows + n) * cin + lk : bx;
  // A: weight row m0 + lr (packed rows are padded to a multiple of 128)
  const size_t arow = (size_t)(m0 + lr) * K + lk;
  const float* wa = p.w + arow;
  const int8_t* wq = reinterpret_cast<const int8_t*>(p.w) + arow;
  const _Float16* wsc = reinterpret_cast<const _Float16*>(p.wscale) + (size_t)(m0 + lr) * (K / 32);

  for (int grp = wave; grp < ngroups; grp += nw) {
    const int k0 = grp * GROUP_K;
    const int nslab = (min(k0 + GROUP_K, K) - k0) / 16;
    f32x4 part;
    for (int s0 = 0; s0 < nslab; s0 += SLABS) {
      f32x4 a[SLABS], bv[SLABS];
#pragma unroll
      for (int u = 0; u < SLABS; ++u) {
        if (s0 + u >= nslab) break;
        const int kb = k0 + (s0 + u) * 16;  // a slab lies inside one tap (cin % 16 == 0)
        const int tap = kb / cin;
        const int shift = (ktaps - 1 - tap) * dil;
        if constexpr (Q8)
          a[u] = dequant4(*reinterpret_cast<const int*>(wq + kb), (float)wsc[(kb + lk) >> 5]);
        else
          a[u] = ld4(wa + kb);
        bv[u] = ld4((n >= shift ? bx : bh) + (kb - tap * cin) - (ptrdiff_t)shift * cin);
      }
#pragma unroll
      for (int u = 0; u < SLABS; ++u) {
        if (s0 + u >= nslab) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (s0 + u == 0 && q == 0)
            part = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][q], bv[u][q], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          else
            part = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][q], bv[u][q], part, 0, 0, 0);
        }
      }
    }
    red[grp * 64 + lane] = part;
  }
  __syncthreads();
  if (wave != 0) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < ngroups; ++j) acc += red[j * 64 + lane];
  const int m = m0 + lk;
  if (m < p.M && lr < p.rows) epilogue4(p, m, lr, acc);
}

// ---------------------------------------------------------------------------
// fp16-operand variant: the same implicit GEMM with both operands rounded to
// IEEE binary16 (ties to even) and products summed in fp32 by the fp16 MFMA.
// Weights are packed as fp16; activation rows stay fp32 in memory and are
// rounded as they are staged into LDS.  SLAB is the MFMA's K: 32 halves
// (v_mfma_f32_16x16x32_f16, 8 per lane) or 16 (v_mfma_f32_16x16x16f16, 4 per
// lane) for channel counts that are multiples of 16 only.  A K-step covers BK
// halves; the accumulation groups (GROUP_K values) and split-K are as above.
// ---------------------------------------------------------------------------

// WPE_: minimum waves per SIMD the register allocation must allow (1 = no
// constraint), chosen per tile by measurement.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int SLAB_, int IGLP_ = -1, int WPE_ = 1>
struct TileCfgH {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, BK = BK_, SLAB = SLAB_,
                       IGLP = IGLP_, WPE = WPE_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int LDK = BK + 8;      // halves; 16-byte pad per row
  static constexpr int KC = BK / 8;       // 16-byte chunks (8 halves) per row per K-step
  static constexpr int A_CH = BM * KC;
  static constexpr int B_CH = BN * KC;
  static constexpr int A_LD = (A_CH + NT - 1) / NT;
  static constexpr int B_LD = (B_CH + NT - 1) / NT;
  static constexpr int PER_LANE = SLAB / 4;  // halves per lane per MFMA
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert((SLAB == 32 || SLAB == 16) && BK % SLAB == 0 && BK % 8 == 0, "bad K-step");
};

__device__ __forceinline__ f16x8 to_half8(f32x4 lo, f32x4 hi) {
  f16x8 r;
  r[0] = (_Float16)lo.x; r[1] = (_Float16)lo.y; r[2] = (_Float16)lo.z; r[3] = (_Float16)lo.w;
  r[4] = (_Float16)hi.x; r[5] = (_Float16)hi.y; r[6] = (_Float16)hi.z; r[7] = (_Float16)hi.w;
  return r;
}

template <class C, bool SPLIT, bool Q8>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE))) void conv_gemm_f16_kernel(
    const ConvParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][C::BM * C::LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][C::BN * C::LDK];
  const _Float16* W = reinterpret_cast<const _Float16*>(p.w);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::WAVES_M;
  const int wn = wave / C::WAVES_M;

  const int mtiles = (p.M + C::BM - 1) / C::BM;
  int tile_id;
  {
    const int L = blockIdx.x, nb = gridDim.x;
    const int xcd = L & 7, i = L >> 3;
    const int per = nb >> 3, extra = nb & 7;
    tile_id = xcd * per + (xcd < extra ? xcd : extra) + i;
  }
  int split = 0;
  if (SPLIT) {
    split = tile_id % p.splits;
    tile_id /= p.splits;
  }
  const int mt = tile_id % mtiles;
  const int nt = tile_id / mtiles;
  const int m0 = mt * C::BM;
  const int g0 = nt * C::BN;

  const int cin = p.cin;
  const int ktaps = p.k, dil = p.dil;  // (lambdas below read locals, not the by-value argument)
  const int ksteps_per_tap = cin / C::BK;
  const int nsteps_all = p.k * ksteps_per_tap;
  constexpr int GROUP_STEPS = GROUP_K / C::BK;
  int s_begin = 0, nsteps = nsteps_all;
  if (SPLIT) {
    const int ngroups = (nsteps_all + GROUP_STEPS - 1) / GROUP_STEPS;
    const int gps = (ngroups + p.splits - 1) / p.splits;
    s_begin = min(split * gps, ngroups) * GROUP_STEPS;
    nsteps = min(min((split + 1) * gps, ngroups) * GROUP_STEPS, nsteps_all);
    if (s_begin >= nsteps) return;
  }

  // K order.  SLAB 32 (channel counts that are multiples of 32): slab j of
  // 32 reduction values is channels 32 (j / k) .. + 32 of tap j % k
  // (channel-major), so that the taps of one channel slab are consecutive.
  // The weights are packed in that order ([Mpad][cin / 32][k][32]), so a
  // K-step's weights are contiguous; its input rows are NSUB = BK / 32 slabs,
  // each load slot belonging to one of them (its own tap shift and
  // channels).  SLAB 16: tap-major ([Mpad][k][cin]), one contiguous run of BK
  // channels of one tap per K-step.  Every fp16 kernel orders the reduction
  // this way.
  constexpr bool CM = C::SLAB == 32;
  constexpr int NSUB = CM ? C::BK / 32 : 1;
  // int8 weights use the same slots: 8 values (two words) and their scale
  const _Float16* a_base[C::A_LD];
  const int8_t* q_base[C::A_LD];
  const _Float16* s_base[C::A_LD];
  int a_lds[C::A_LD], q_col[C::A_LD];
  const size_t ktot = (size_t)p.k * cin;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    int idx = tid + i * C::NT;
    if (C::A_CH % C::NT != 0 && idx >= C::A_CH) idx = C::A_CH - 1;
    const int row = idx / C::KC, col = (idx % C::KC) * 8;
    a_base[i] = W + (size_t)(m0 + row) * ktot + col;
    if constexpr (Q8) {
      q_base[i] = reinterpret_cast<const int8_t*>(p.w) + (size_t)(m0 + row) * ktot + col;
      s_base[i] = reinterpret_cast<const _Float16*>(p.wscale) + (size_t)(m0 + row) * (ktot / 32);
    }
    q_col[i] = col;
    a_lds[i] = row * C::LDK + col;
  }
  const char* bxb[C::B_LD];  // row of x (fp32 or fp16 elements), as bytes
  const float* bh[C::B_LD];
  const bool x_half = p.x_half != 0;
  const int x_esz = x_half ? 2 : 4;
  int bn[C::B_LD], b_lds[C::B_LD], b_sub[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    int idx = tid + i * C::NT;
    if (C::B_CH % C::NT != 0 && idx >= C::B_CH) idx = C::B_CH - 1;
    const int row = idx / C::KC, col = (idx % C::KC) * 8;
    b_sub[i] = CM ? col / 32 : 0;
    const int gcol = CM ? col % 32 : col;
    const int g = min(g0 + row, p.rows - 1);
    const int b = g / p.nin;
    const int n = g - b * p.nin;
    bn[i] = n;
    bxb[i] = reinterpret_cast<const char*>(p.x) + ((size_t)g * cin + gcol) * x_esz;
    bh[i] = p.hin ? p.hin + (size_t)b * p.sstride + (ptrdiff_t)(p.hin_rows + n) * cin + gcol
                  : reinterpret_cast<const float*>(bxb[i]);
    b_lds[i] = row * C::LDK + col;
  }

  f32x4 ra[C::A_LD];
  // B: 8 fp32 values (rb_lo, rb_hi) or, for an fp16 input row, the 8 halves'
  // bits in rb_lo (bhalf set); rounded / stored as fp16 at the LDS store
  f32x4 rb_lo[C::B_LD], rb_hi[C::B_LD];
  int b_shift[C::B_LD];  // tap shift of each slot's slab in the staged step
  int2 rq[C::A_LD];
  float rs[C::A_LD];

  // (channel slab, tap) of the next slab to load: K-steps are loaded in
  // order, so it advances without divisions
  int run_cb = 0, run_tap = 0;
  if constexpr (CM) {
    const int j0 = s_begin * NSUB;
    run_cb = j0 / ktaps;
    run_tap = j0 - run_cb * ktaps;
  }
  auto gload = [&](int s) {
    // each B slot's tap shift and input offset for this step (its own slab)
    int shift_of[C::B_LD];
    ptrdiff_t boff_of[C::B_LD];
    ptrdiff_t aoff;
    if constexpr (CM) {
      aoff = (ptrdiff_t)s * C::BK;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int sh = (ktaps - 1 - run_tap) * dil;
        const ptrdiff_t bo = run_cb * 32 - (ptrdiff_t)sh * cin;
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i)
          if (u == 0 || b_sub[i] == u) {
            shift_of[i] = sh;
            boff_of[i] = bo;
          }
        if (++run_tap == ktaps) {
          run_tap = 0;
          ++run_cb;
        }
      }
    } else {
      const int tap = s / ksteps_per_tap;
      const int c0 = (s - tap * ksteps_per_tap) * C::BK;
      const int sh = (ktaps - 1 - tap) * dil;
      aoff = (ptrdiff_t)tap * cin + c0;
#pragma unroll
      for (int i = 0; i < C::B_LD; ++i) {
        shift_of[i] = sh;
        boff_of[i] = c0 - (ptrdiff_t)sh * cin;
      }
    }
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) {
        rq[i] = *reinterpret_cast<const int2*>(q_base[i] + aoff);
        rs[i] = (float)s_base[i][(aoff + q_col[i]) >> 5];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) ra[i] = *reinterpret_cast<const f32x4*>(a_base[i] + aoff);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int shift = shift_of[i];
      const ptrdiff_t boff = boff_of[i];
      b_shift[i] = shift;
      // branch-free: an fp16 row needs one 16-byte load (its second load
      // repeats the first address), an fp32 row two
      const bool fromx = bn[i] >= shift;
      const bool hx = x_half && fromx;
      const char* src = hx      ? bxb[i] + boff * 2
                        : fromx ? bxb[i] + boff * 4
                                : reinterpret_cast<const char*>(bh[i] + boff);
      rb_lo[i] = *reinterpret_cast<const f32x4*>(src);
      rb_hi[i] = *reinterpret_cast<const f32x4*>(hx ? src : src + 16);
    }
  };
  auto lstore = [&](int buf) {
    if constexpr (Q8) {
      // q * scale is exact in fp32; one rounding to fp16 as for float weights
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i)
        *reinterpret_cast<f16x8*>(&As[buf][a_lds[i]]) =
            to_half8(dequant4(rq[i].x, rs[i]), dequant4(rq[i].y, rs[i]));
    } else {
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i) *reinterpret_cast<f32x4*>(&As[buf][a_lds[i]]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i)
      *reinterpret_cast<f16x8*>(&Bs[buf][b_lds[i]]) = (x_half && bn[i] >= b_shift[i])
                                                          ? __builtin_bit_cast(f16x8, rb_lo[i])
                                                          : to_half8(rb_lo[i], rb_hi[i]);
  };

  // Lane l supplies A[l%16][k] and B[k][l%16] for the PER_LANE values of k
  // owned by lane group l/16; the group's values are consecutive in K, read
  // as one 16- or 8-byte vector from a padded LDS row.
  const int lr = lane & 15;
  const int lk = (lane >> 4) * C::PER_LANE;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto mma_step = [&](int cur, f32x4 (&part)[C::FM][C::FN], auto first) {
    if constexpr (C::IGLP >= 0) __builtin_amdgcn_iglp_opt(C::IGLP);
    const _Float16* Ab = As[cur];
    const _Float16* Bb = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += C::SLAB) {
      if constexpr (C::SLAB == 32) {
        f16x8 af[C::FM], bf[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          af[i] = *reinterpret_cast<const f16x8*>(&Ab[(wm * C::WTM + i * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          bf[j] = *reinterpret_cast<const f16x8*>(&Bb[(wn * C::WTN + j * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if (decltype(first)::value && kk == 0)
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], part[i][j], 0, 0, 0);
          }
      } else {
        f16x4 af[C::FM], bf[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          af[i] = *reinterpret_cast<const f16x4*>(&Ab[(wm * C::WTM + i * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          bf[j] = *reinterpret_cast<const f16x4*>(&Bb[(wn * C::WTN + j * 16 + lr) * C::LDK + kk + lk]);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if (decltype(first)::value && kk == 0)
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(af[i], bf[j], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              part[i][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(af[i], bf[j], part[i][j], 0, 0, 0);
          }
      }
    }
  };

  gload(s_begin);
  lstore(s_begin & 1);
  __syncthreads();
  for (int gs = s_begin; gs < nsteps; gs += GROUP_STEPS) {
    const int ge = min(gs + GROUP_STEPS, nsteps);
    f32x4 part[C::FM][C::FN];
    for (int s = gs; s < ge; ++s) {
      const int cur = s & 1;
      if (s + 1 < nsteps) gload(s + 1);
      if (s == gs)
        mma_step(cur, part, std::true_type{});
      else
        mma_step(cur, part, std::false_type{});
      if (s + 1 < nsteps) lstore(cur ^ 1);
      __syncthreads();
    }
    if (SPLIT) {
      const size_t gbase = (size_t)(gs / GROUP_STEPS) * p.rows;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = m0 + wm * C::WTM + i * 16 + (lane >> 4) * 4;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int g = g0 + wn * C::WTN + j * 16 + lr;
          if (g < p.rows) st4(p.partial + (gbase + g) * p.M + m, part[i][j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] += part[i][j];
    }
  }
  if (SPLIT) return;

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = m0 + wm * C::WTM + i * 16 + (lane >> 4) * 4;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int g = g0 + wn * C::WTN + j * 16 + lr;
      if (g < p.rows) epilogue4(p, m, g, acc[i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// fp16-operand variant fed by direct global->LDS loads (global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave's LDS base + 16 * lane), so no register
// staging: an NS-deep ring of LDS stages keeps the loads of NS - 1 K-steps in
// flight, which the register-staged kernel cannot afford in registers.  One
// K-step is one 32-half MFMA slab of one tap; the K-steps, their order, the
// accumulation groups and split-K are those of conv_gemm_f16_kernel, so both
// give the same bits.
//
// LDS stage = A tile (BM rows x 32 halves, 4 chunks of 16 bytes per row; with
// the split, the hi plane's tile then the lo plane's), then the B tile: 32
// halves per row when the input rows are fp16 (XH), else 32 floats (8 chunks
// per row), rounded to fp16 (or split) as the MFMA operands are read.
// Chunks are XOR-swizzled within a row so that the 8 lanes an LDS read
// serves together (8 rows, one 16-byte chunk each, 128 bytes of banks) hit
// distinct banks: chunk c of row r sits at position c ^ ((r >> 1) & 3)
// (4-chunk rows) or c ^ (r & 7) (8-chunk rows).
// Every wave issues the same number of loads per K-step (lanes past a tile's
// slots are masked), so a wave's vmcnt tells when its own share of a stage has
// landed; a barrier then makes every wave's share visible.  History rows of
// an fp16 input come from the fp32 state and are converted through registers.
//
// WIN (fp16 rows, no split, k >= 3): the K-steps of one 32-channel slab are
// its k taps, and tap t of output row r reads input row r + t*dil of the
// window that starts (k-1)*dil rows before the tile.  So each slab's window,
// BN + (k-1)*dil rows of 32 halves, is staged once (in buffer slab % WNB) and
// each tap reads its rows at offset t*dil; only the weights go through the
// per-step ring.  A window is loaded NS - 1 steps ahead, over the buffer of
// slab - WNB, whose last tap every wave has passed once (WNB - 1) * k >= NS - 1.  That holds while every row of the tile belongs
// to one stream, so these tiles never cross a stream: each stream's rows are
// covered by their own ceil(nin / BN) tiles.  The MFMA operands and their
// order are unchanged, hence the bits.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NS_>
struct TileCfgD {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NS = NS_;
  static constexpr int BK = 32, SLAB = 32;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int NT = WAVES * 64;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int A_SLOTS = BM * 4;            // 16-byte chunks per stage
  static constexpr int A_PER_WAVE = A_SLOTS / WAVES;
  static_assert(A_SLOTS % WAVES == 0 && A_PER_WAVE <= 64, "A chunks per wave");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0 && NS >= 2, "tile");
  template <bool XH>
  static constexpr int b_slots() { return BN * (XH ? 4 : 8); }
  template <bool XH>
  static constexpr int b_per_wave() { return b_slots<XH>() / WAVES; }  // multiple of 64 or <= 64
  template <bool XH>
  static constexpr int stage_bytes() { return (A_SLOTS + b_slots<XH>()) * 16; }
};

__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds_wave_base) {
  // m0 holds the wave's LDS destination; the address is wave-uniform.  m0 is
  // a reserved register the compiler does not preserve across asm, so these
  // kernels must not otherwise use it (checked on the generated code by the
  // test suite: every m0 write in them is this one, right before its load).
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(gaddr)
               : "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding,
// and for all of its LDS operations
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// the same for a wave-uniform count n, 0 <= n <= N
template <int N>
__device__ __forceinline__ void wait_vm_lgkm_upto(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vm_lgkm<N>();
      return;
    }
    wait_vm_lgkm_upto<N - 1>(n);
  } else {
    wait_vm_lgkm<0>();
  }
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// rows of halo a window may carry: (k-1)*dil at most
constexpr int WIN_HALO = 64;

// X3: split-fp16 operands (fp32 rows only).  The weights come as hi and lo
// fp16 planes w1 + w2 (of the weights times a power of two), both staged.
// Each fp32 input value is split as it is read from LDS into x1 = fp16(x) and
// x2 = fp16(x - x1).  Every fragment pair takes three MFMAs into the same
// accumulator, always in this order: w2 x1, w1 x2, w1 x1 (w2 x2, below 2^-22
// of the product, is dropped); the epilogue scales the sum back.
template <class C, bool SPLIT, bool XH, bool X3 = false, bool WIN = false>
__global__ __launch_bounds__(C::NT) void conv_gemm_f16_dma_kernel(const ConvParams p) {
  static_assert(!(X3 && XH), "the split takes fp32 rows");
  // (k >= 3 taps: WNB = 2 buffers serve NS <= 4, 3 serve NS <= 7)
  static_assert(!WIN || (XH && !SPLIT && !X3 && C::NS <= 7), "windows: fp16 rows, whole K");
  constexpr int WNB = C::NS <= 4 ? 2 : 3;
  constexpr int A_BYTES = C::A_SLOTS * 16;
  constexpr int A_PLANES = X3 ? 2 : 1;
  constexpr int STAGE = WIN ? A_BYTES : C::template stage_bytes<XH>() + (A_PLANES - 1) * A_BYTES;
  constexpr int WROWS = C::BN + WIN_HALO;               // window rows at most
  constexpr int WIN_BYTES = WROWS * 64;                 // 32 halves a row
  constexpr int WD = (WROWS * 4 + C::NT - 1) / C::NT;  // window loads per wave per slab, at most
  constexpr int WOFF = C::NS * STAGE;                   // window buffers after the ring
  constexpr int RING = WOFF + (WIN ? WNB * WIN_BYTES : 0);
  constexpr int B_SLOTS = C::template b_slots<XH>();
  constexpr int B_PER_WAVE = C::template b_per_wave<XH>();
  constexpr int B_DMAS = B_PER_WAVE >= 64 ? B_PER_WAVE / 64 : 1;  // loads per wave per K-step
  constexpr int B_LANES = B_PER_WAVE >= 64 ? 64 : B_PER_WAVE;
  static_assert(B_SLOTS % C::WAVES == 0 && (B_PER_WAVE <= 64 || B_PER_WAVE % 64 == 0), "B chunks per wave");
  constexpr int OPS = A_PLANES + B_DMAS;  // vector-memory operations per wave per K-step (at least)
  constexpr int LDS_BYTES = RING > epi_lds_floats<C>() * 4 ? RING : epi_lds_floats<C>() * 4;
  __shared__ __attribute__((aligned(16))) char lds[SPLIT ? RING : LDS_BYTES];
  const _Float16* W = reinterpret_cast<const _Float16*>(p.w);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::WAVES_M;
  const int wn = wave / C::WAVES_M;

  const int mtiles = (p.M + C::BM - 1) / C::BM;
  int tile_id;
  {
    const int L = blockIdx.x, nb = gridDim.x;
    const int xcd = L & 7, i = L >> 3;
    const int per = nb >> 3, extra = nb & 7;
    tile_id = xcd * per + (xcd < extra ? xcd : extra) + i;
  }
  int split = 0;
  if (SPLIT) {
    split = tile_id % p.splits;
    tile_id /= p.splits;
  }
  const int mt = tile_id % mtiles;
  const int nt = tile_id / mtiles;
  const int m0 = mt * C::BM;
  int g0 = nt * C::BN, g_end = p.rows;
  int wstream = 0, wn0 = 0;  // WIN: the tile's stream and its first row in it
  if (WIN) {
    const int tpb = (p.nin + C::BN - 1) / C::BN;
    wstream = nt / tpb;
    wn0 = (nt - wstream * tpb) * C::BN;
    g0 = wstream * p.nin + wn0;
    g_end = (wstream + 1) * p.nin;
  }

  const int cin = p.cin;
  const int ktaps = p.k, dil = p.dil;
  const int ksteps_per_tap = cin / C::BK;
  const int nsteps_all = p.k * ksteps_per_tap;
  constexpr int GROUP_STEPS = GROUP_K / C::BK;
  int s_begin = 0, nsteps = nsteps_all;
  if (SPLIT) {
    const int ngroups = (nsteps_all + GROUP_STEPS - 1) / GROUP_STEPS;
    const int gps = (ngroups + p.splits - 1) / p.splits;
    s_begin = min(split * gps, ngroups) * GROUP_STEPS;
    nsteps = min(min((split + 1) * gps, ngroups) * GROUP_STEPS, nsteps_all);
    if (s_begin >= nsteps) return;
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  // A: this lane's chunk of the wave's A_PER_WAVE slots
  const bool a_on = lane < C::A_PER_WAVE;
  const _Float16* a_src;
  {
    const int j = wave * C::A_PER_WAVE + (a_on ? lane : 0);
    const int r = j >> 2, c = (j & 3) ^ ((r >> 1) & 3);
    a_src = W + (size_t)(m0 + r) * ((size_t)p.k * cin) + c * 8;
  }
  const uint32_t a_dst = lds0 + (uint32_t)(wave * C::A_PER_WAVE) * 16;
  // the lo plane holds the same layout
  const _Float16* a_lo_src = X3 ? reinterpret_cast<const _Float16*>(p.w_lo) + (a_src - W) : nullptr;
  // B: B_DMAS loads of 64 (or B_LANES) chunks per wave
  const char* bx[B_DMAS];
  const float* bh[B_DMAS];
  int bn[B_DMAS];
  bool b_on[B_DMAS];
  const size_t esz = XH ? 2 : 4;
#pragma unroll
  for (int h = 0; h < B_DMAS; ++h) {
    b_on[h] = lane < B_LANES;
    const int j = wave * B_PER_WAVE + h * 64 + (b_on[h] ? lane : 0);
    const int r = XH ? (j >> 2) : (j >> 3);
    const int c = XH ? ((j & 3) ^ ((r >> 1) & 3)) : ((j & 7) ^ (r & 7));
    const int col = XH ? c * 8 : c * 4;
    const int g = min(g0 + r, p.rows - 1);
    const int b = g / p.nin;
    const int n = g - b * p.nin;
    bn[h] = n;
    bx[h] = reinterpret_cast<const char*>(p.x) + ((size_t)g * cin + col) * esz;
    bh[h] = p.hin ? p.hin + (size_t)b * p.sstride + (ptrdiff_t)(p.hin_rows + n) * cin + col
                  : reinterpret_cast<const float*>(bx[h]);
  }
  // WIN: a wave's loads of a slab window are the 64-chunk pieces wave,
  // wave + WAVES, ... of its (BN + halo) * 4 chunks; chunk i holds (swizzled
  // as the B tiles) a piece of window row i / 4, frame wn0 + i / 4 - halo of
  // the tile's stream
  const int halo = (ktaps - 1) * dil;
  const int wchunks = (C::BN + halo) * 4;
  const bool whist = wn0 < halo;  // some window rows come from the state
  const _Float16* wx[WD];
  const float* wh[WD];
  bool wx_on[WD], w_on[WD];
  int wcount = 0;
  if (WIN) {
#pragma unroll
    for (int h = 0; h < WD; ++h) {
      const int piece = wave + h * C::WAVES;
      const int idx = piece * 64 + lane;
      if (piece * 64 < wchunks) wcount = h + 1;
      w_on[h] = idx < wchunks;
      const int j = min(idx, wchunks - 1) >> 2;
      const int c = (idx & 3) ^ ((j >> 1) & 3);
      const int n = wn0 + j - halo;
      wx_on[h] = n >= 0;
      // rows past the stream's end feed only rows the epilogue drops
      wx[h] = reinterpret_cast<const _Float16*>(p.x) + ((size_t)wstream * p.nin + min(max(n, 0), p.nin - 1)) * cin + c * 8;
      wh[h] = p.hin ? p.hin + (size_t)wstream * p.sstride + (ptrdiff_t)(p.hin_rows + min(n, -1)) * cin + c * 8
                    : nullptr;
    }
    wcount = __builtin_amdgcn_readfirstlane(wcount);
  }

  // issue the loads of K-step s into ring stage st.  Channel-major K order
  // (one 32-channel slab of one tap per step), as conv_gemm_f16_kernel; steps
  // are issued in order, so the (slab, tap) pair advances without divisions.
  int run_cb = s_begin / ktaps, run_tap = s_begin - (s_begin / ktaps) * ktaps;
  auto issue = [&](int s, int st) __attribute__((always_inline)) {
    const int tap = run_tap;
    const int c0 = run_cb * C::BK;
    if (++run_tap == ktaps) {
      run_tap = 0;
      ++run_cb;
    }
    const int shift = (ktaps - 1 - tap) * dil;
    const uint32_t sbase = (uint32_t)(st * STAGE);
    if constexpr (WIN) {
      // a slab's window goes with its first tap, before that step's weights
      if (tap == 0) {
        const uint32_t wbase = lds0 + WOFF + (uint32_t)((c0 / C::BK) % WNB) * WIN_BYTES;
#pragma unroll
        for (int h = 0; h < WD; ++h) {
          if (h >= wcount) break;
          const uint32_t dst = wbase + (uint32_t)(wave + h * C::WAVES) * 1024;
          if (!w_on[h]) continue;
          if (wx_on[h]) {
            lds_dma16(wx[h] + c0, dst);
          } else {
            const float* src = wh[h] + c0;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
            *reinterpret_cast<f16x8*>(lds + (dst - lds0) + lane * 16) = to_half8(lo, hi);
          }
        }
        // a tile with state rows drains its loads here, so the counts the
        // K loop waits for still bound what is in flight
        if (whist) wait_vm_lgkm<0>();
      }
    }
    // weights packed in the same slab order: step s is slab s
    if (a_on) lds_dma16(a_src + (ptrdiff_t)s * C::BK, a_dst + sbase);
    if constexpr (WIN) return;
    if (X3 && a_on) lds_dma16(a_lo_src + (ptrdiff_t)s * C::BK, a_dst + sbase + A_BYTES);
#pragma unroll
    for (int h = 0; h < B_DMAS; ++h) {
      const uint32_t dst = lds0 + sbase + A_PLANES * A_BYTES + (uint32_t)(wave * B_PER_WAVE + h * 64) * 16;
      const ptrdiff_t boff = c0 - (ptrdiff_t)shift * cin;
      if (!b_on[h]) continue;
      if (bn[h] >= shift) {
        lds_dma16(bx[h] + boff * (ptrdiff_t)esz, dst);
      } else if constexpr (XH) {
        // an fp32 history row of an fp16 input: round through registers
        const float* src = bh[h] + boff;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
        *reinterpret_cast<f16x8*>(lds + (dst - lds0) + lane * 16) = to_half8(lo, hi);
      } else {
        lds_dma16(bh[h] + boff, dst);
      }
    }
  };

  // operand reads: lane l reads chunk l/16 of rows (fragment base + l%16)
  const int lr = lane & 15, q = lane >> 4;
  // (fragment rows start at multiples of 16, so the swizzle depends on l%16 only)
  const int a_rd = ((wm * C::WTM + lr) * 4 + (q ^ ((lr >> 1) & 3))) * 16;
  const int b_rd = XH ? A_BYTES + ((wn * C::WTN + lr) * 4 + (q ^ ((lr >> 1) & 3))) * 16 : 0;
  const int b_rd0 = A_PLANES * A_BYTES + ((wn * C::WTN + lr) * 8 + ((2 * q) ^ (lr & 7))) * 16;
  const int b_rd1 = A_PLANES * A_BYTES + ((wn * C::WTN + lr) * 8 + ((2 * q + 1) ^ (lr & 7))) * 16;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // (wrd: WIN, byte offset of this lane's first B fragment in the window)
  auto mma_step = [&](int st, f32x4 (&part)[C::FM][C::FN], auto first, int wrd) __attribute__((always_inline)) {
    const char* S = lds + st * STAGE;
    f16x8 af[C::FM], bf[C::FN];
    f16x8 al[X3 ? C::FM : 1];  // weight lo halves (split)
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      af[i] = *reinterpret_cast<const f16x8*>(S + a_rd + i * 16 * 64);
      if constexpr (X3) al[i] = *reinterpret_cast<const f16x8*>(S + A_BYTES + a_rd + i * 16 * 64);
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      if constexpr (WIN) {
        bf[j] = *reinterpret_cast<const f16x8*>(lds + wrd + j * 16 * 64);
      } else if constexpr (XH) {
        bf[j] = *reinterpret_cast<const f16x8*>(S + b_rd + j * 16 * 64);
      } else if constexpr (!X3) {  // (the split reads its B fragments below)
        const f32x4 lo = *reinterpret_cast<const f32x4*>(S + b_rd0 + j * 16 * 128);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(S + b_rd1 + j * 16 * 128);
        bf[j] = to_half8(lo, hi);
      }
    }
    if constexpr (X3) {
      // one B fragment's terms at a time (fewer live registers); the three
      // (FM) accumulators of a fragment interleave the dependent MFMAs
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(S + b_rd0 + j * 16 * 128);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(S + b_rd1 + j * 16 * 128);
        const f16x8 x1 = to_half8(lo, hi);
        const float r[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        f16x8 x2;
#pragma unroll
        for (int e = 0; e < 8; ++e) x2[e] = split_lo(r[e], x1[e]);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        bool fresh = decltype(first)::value;
        auto mm = [&](const f16x8(&a)[C::FM], f16x8 b) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b, fresh ? z : part[i][j], 0, 0, 0);
          fresh = false;
        };
        mm(al, x1);
        mm(af, x2);
        mm(af, x1);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          if (decltype(first)::value)
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          else
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], part[i][j], 0, 0, 0);
        }
    }
  };

  // prologue: K-steps s_begin .. s_begin + NS - 2 in flight
#pragma unroll
  for (int t = 0; t < C::NS - 1; ++t)
    if (s_begin + t < nsteps) issue(s_begin + t, t);

  int st = 0;  // ring stage of step s
  int m_tap = 0, m_cb = 0;  // WIN: tap and slab of step s (no split: s_begin = 0)
  for (int gs = s_begin; gs < nsteps; gs += GROUP_STEPS) {
    const int ge = min(gs + GROUP_STEPS, nsteps);
    f32x4 part[C::FM][C::FN];
    for (int s = gs; s < ge; ++s) {
      // this wave's loads of step s have landed once at most (steps issued
      // after it) x OPS operations remain; then every wave's have
      const int later = min(C::NS - 2, nsteps - 1 - s);
      int wrd = 0;
      if constexpr (WIN) {
        // issued after step s's weights: the weights of `later` steps, and
        // the windows of the slabs whose first tap is among them (later <= 5
        // and k >= 3: two at most)
        const int starts = (m_tap + later >= ktaps) + (m_tap + later >= 2 * ktaps);
        const int nafter = later + starts * wcount;
        wait_vm_lgkm_upto<C::NS - 2 + 2 * WD>(__builtin_amdgcn_readfirstlane(nafter));
        const int row0 = wn * C::WTN + lr + m_tap * dil;
        wrd = WOFF + (m_cb % WNB) * WIN_BYTES + (row0 * 4 + (q ^ ((row0 >> 1) & 3))) * 16;
        if (++m_tap == ktaps) {
          m_tap = 0;
          ++m_cb;
        }
      } else if constexpr (C::NS >= 4) {
        if (later >= 2) wait_vm_lgkm<2 * OPS>();
        else if (later == 1) wait_vm_lgkm<OPS>();
        else wait_vm_lgkm<0>();
      } else {
        if (later >= 1) wait_vm_lgkm<OPS>();
        else wait_vm_lgkm<0>();
      }
      block_barrier();
      // refill the stage every wave finished reading at step s - 1
      if (s + C::NS - 1 < nsteps) issue(s + C::NS - 1, st == 0 ? C::NS - 1 : st - 1);
      if (s == gs)
        mma_step(st, part, std::true_type{}, wrd);
      else
        mma_step(st, part, std::false_type{}, wrd);
      st = st == C::NS - 1 ? 0 : st + 1;
    }
    if (SPLIT) {
      const size_t gbase = (size_t)(gs / GROUP_STEPS) * p.rows;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int m = m0 + wm * C::WTM + i * 16 + (lane >> 4) * 4;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int g = g0 + wn * C::WTN + j * 16 + lr;
          if (g < p.rows) st4(p.partial + (gbase + g) * p.M + m, part[i][j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] += part[i][j];
    }
  }
  if (SPLIT) return;

  // every wave has left the K loop (no LDS reads or loads outstanding): the
  // ring becomes the epilogue's tile
  __syncthreads();
  // (the split's registers leave no room for a batch: one chunk at a time)
  epilogue_tile<C, X3 ? 1 : 4>(p, reinterpret_cast<float*>(lds), acc, m0, g0, g_end, wm, wn, lane, tid);
}

template <class C, bool HALF, bool Q8>
hipError_t launch_cfg_q(const ConvParams& p, hipStream_t s) {
  const int mtiles = (p.M + C::BM - 1) / C::BM;
  const int ntiles = (p.rows + C::BN - 1) / C::BN;
  const long long tiles = (long long)mtiles * ntiles;
  if (tiles <= 0) return hipSuccess;
  if (p.splits <= 1) {
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    if constexpr (HALF)
      hipLaunchKernelGGL((conv_gemm_f16_kernel<C, false, Q8>), dim3((unsigned)tiles), dim3(C::NT), 0, s, p);
    else
      hipLaunchKernelGGL((conv_gemm_kernel<C, false, Q8>), dim3((unsigned)tiles), dim3(C::NT), 0, s, p);
    return hipGetLastError();
  }
  // split: the blocks store group partials; the fold is launched by the caller
  const long long nb = tiles * p.splits;
  if (nb > 0x7fffffffLL || !p.partial) return hipErrorInvalidValue;
  if constexpr (HALF)
    hipLaunchKernelGGL((conv_gemm_f16_kernel<C, true, Q8>), dim3((unsigned)nb), dim3(C::NT), 0, s, p);
  else
    hipLaunchKernelGGL((conv_gemm_kernel<C, true, Q8>), dim3((unsigned)nb), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// After a split launch: fold the group partials and run the epilogue, fused
// with the LayerNorm when ln is given and fits.
hipError_t launch_fold(const ConvParams& p, hipStream_t s, const LnArgs* ln) {
  const int ngroups = (p.k * p.cin + GROUP_K - 1) / GROUP_K;
  const int nv = ln ? layernorm_nv(ln->d) : 0;
  if (ln && (nv == 0 || p.M != ln->d || p.phases != 1 || p.nout < 1 || p.out[0].half)) return hipErrorInvalidValue;
  if (ln) {
    const dim3 grid((unsigned)p.rows), block(64 * nv);
    switch (nv) {
      case 1: hipLaunchKernelGGL(splitk_reduce_ln_kernel<1>, grid, block, 0, s, p, ngroups, *ln); break;
      case 2: hipLaunchKernelGGL(splitk_reduce_ln_kernel<2>, grid, block, 0, s, p, ngroups, *ln); break;
      case 4: hipLaunchKernelGGL(splitk_reduce_ln_kernel<4>, grid, block, 0, s, p, ngroups, *ln); break;
      case 8: hipLaunchKernelGGL(splitk_reduce_ln_kernel<8>, grid, block, 0, s, p, ngroups, *ln); break;
      default: hipLaunchKernelGGL(splitk_reduce_ln_kernel<16>, grid, block, 0, s, p, ngroups, *ln); break;
    }
    return hipGetLastError();
  }
  const long long n = (long long)p.rows * (p.M / 4);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, ngroups);
  return hipGetLastError();
}

// Slab windows (WIN) for fp16 rows: whole K, k >= 3 taps with at most
// WIN_HALO rows of history that the state holds, whole streams, and per-stream
// tiles that waste at most 1/7 of their rows (the first BigVGAN stage of
// 25-frame chunks, 800 rows per stream in seven tiles, runs 0.6 % faster per
// batched step in windows despite its 12 % of idle rows; two window segments
// for tiles across a stream end, without idle rows, measured no faster).
bool dma_win_ok(const ConvParams& p, int bn) {
  if (!p.x_half || p.w_lo || p.splits > 1 || p.k < 3 || p.dil < 1 || p.nin < 1 || p.rows % p.nin != 0) return false;
  const int halo = (p.k - 1) * p.dil;
  if (halo > WIN_HALO || !p.hin || p.hin_rows < halo) return false;
  const long long tpb = (p.nin + bn - 1) / bn;
  return tpb * bn * 7 <= (long long)p.nin * 8;
}

template <class C, bool XH, bool X3 = false, class CW = C>
hipError_t launch_dma_x(const ConvParams& p, hipStream_t s) {
  const int mtiles = (p.M + C::BM - 1) / C::BM;
  const int ntiles = (p.rows + C::BN - 1) / C::BN;
  const long long tiles = (long long)mtiles * ntiles;
  if (tiles <= 0) return hipSuccess;
  if constexpr (XH && !X3) {
    static_assert(CW::BM == C::BM && CW::BN == C::BN, "window tile");
    if (dma_win_ok(p, CW::BN)) {
      const long long wt = (long long)mtiles * (p.rows / p.nin) * ((p.nin + CW::BN - 1) / CW::BN);
      if (wt > 0x7fffffffLL) return hipErrorInvalidValue;
      hipLaunchKernelGGL((conv_gemm_f16_dma_kernel<CW, false, true, false, true>), dim3((unsigned)wt), dim3(CW::NT), 0,
                         s, p);
      return hipGetLastError();
    }
  }
  if (p.splits <= 1) {
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv_gemm_f16_dma_kernel<C, false, XH, X3>), dim3((unsigned)tiles), dim3(C::NT), 0, s, p);
    return hipGetLastError();
  }
  const long long nb = tiles * p.splits;
  if (nb > 0x7fffffffLL || !p.partial) return hipErrorInvalidValue;
  hipLaunchKernelGGL((conv_gemm_f16_dma_kernel<C, true, XH, X3>), dim3((unsigned)nb), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// fp16 rows (CH; CW with slab windows) or fp32 rows (CF) as the B operand
template <class CH, class CF, class CW>
hipError_t launch_dma(const ConvParams& p, hipStream_t s) {
  return p.x_half ? launch_dma_x<CH, true, false, CW>(p, s) : launch_dma_x<CF, false>(p, s);
}

// int8 weights (p.wscale set) or float weights
template <class C, bool HALF = false>
hipError_t launch_cfg(const ConvParams& p, hipStream_t s) {
  if (p.wscale) return launch_cfg_q<C, HALF, true>(p, s);
  return launch_cfg_q<C, HALF, false>(p, s);
}

}  // namespace

int gemm_tile_bm(int tile) {
  switch (tile) {
    case TILE_128x128: return 128;
    case TILE_64x64: return 64;
    case TILE_96x128: return 96;
    case TILE_S64x16: return 64;
    case TILE_S64x32: return 64;
  }
  return 0;
}

int gemm_tile_bn(int tile) {
  switch (tile) {
    case TILE_128x128: return 128;
    case TILE_64x64: return 64;
    case TILE_96x128: return 128;
    case TILE_S64x16: return 16;
    case TILE_S64x32: return 32;
  }
  return 0;
}

namespace {
int skinny_bk(int cin) { return cin % 128 == 0 ? 128 : cin % 64 == 0 ? 64 : cin % 32 == 0 ? 32 : 16; }
int half_bk(int cin) { return cin % 64 == 0 ? 64 : cin % 32 == 0 ? 32 : 16; }
}  // namespace

bool gemm_f16_direct(bool int8, int cin, int tile) {
  return !int8 && cin % 32 == 0 && (tile == TILE_128x128 || tile == TILE_96x128);
}

bool gemm_f16_window(const ConvParams& p, int tile) {
  return gemm_f16_direct(p.wscale != nullptr, p.cin, tile) && dma_win_ok(p, gemm_tile_bn(tile));
}

int gemm_tile_bk(int tile, int cin, bool half) {
  if (tile == TILE_S64x16 || tile == TILE_S64x32) return skinny_bk(cin);
  if (half) return tile == TILE_128x128 ? std::min(half_bk(cin), 32) : half_bk(cin);
  return tile == TILE_128x128 || cin % 32 != 0 ? 16 : 32;
}

namespace {

hipError_t launch_blocks_f32(const ConvParams& p, int tile, hipStream_t s) {
  const bool bk32 = (p.cin % 32) == 0;
  if (p.cin % 16 != 0) return hipErrorInvalidValue;
  switch (tile) {
    case TILE_128x128:
      // 8 waves of 64x32 with BK = 16: four waves per SIMD (measured 119
      // TFLOP/s; 4 waves of 64x64 at BK = 32 fit one wave per SIMD and reach
      // 101).  The reduction order does not depend on BK or the wave layout.
      return launch_cfg<TileCfg<128, 128, 2, 4, 16, 1>>(p, s);
    case TILE_64x64:
      return bk32 ? launch_cfg<TileCfg<64, 64, 2, 2, 32>>(p, s) : launch_cfg<TileCfg<64, 64, 2, 2, 16>>(p, s);
    case TILE_96x128:
      // 8 waves of 48x32: four waves per SIMD
      return bk32 ? launch_cfg<TileCfg<96, 128, 2, 4, 32, 0>>(p, s) : launch_cfg<TileCfg<96, 128, 2, 4, 16, 0>>(p, s);
    case TILE_S64x16:
    case TILE_S64x32: {
      // skinny: 4 waves stacked along M, one 16- or 32-row column block; a
      // K-step moves 32 KB of weights, so a 256-deep group takes two round trips
      const int bk = skinny_bk(p.cin);
#define VOC_SKINNY(BN, WM, WN)                                                               \
  return bk == 128 ? launch_cfg<TileCfg<64, BN, WM, WN, 128>>(p, s)                        \
       : bk == 64  ? launch_cfg<TileCfg<64, BN, WM, WN, 64>>(p, s)                         \
       : bk == 32  ? launch_cfg<TileCfg<64, BN, WM, WN, 32>>(p, s)                         \
                   : launch_cfg<TileCfg<64, BN, WM, WN, 16>>(p, s)
      if (tile == TILE_S64x16) VOC_SKINNY(16, 4, 1);
      VOC_SKINNY(32, 4, 1);
#undef VOC_SKINNY
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_blocks_f16(const ConvParams& p, int tile, hipStream_t s) {
  if (p.cin % 16 != 0) return hipErrorInvalidValue;
  const int bk = half_bk(p.cin);
  // (no interleaving hint with 16-wide slabs: iglp_opt(1) sends the compiler
  // into unbounded memory use on that instance)
#define VOC_F16_CASES(BM, BN, WM, WN, IG)                                                           \
  return bk == 64 ? launch_cfg<TileCfgH<BM, BN, WM, WN, 64, 32, IG>, true>(p, s)                    \
       : bk == 32 ? launch_cfg<TileCfgH<BM, BN, WM, WN, 32, 32, IG>, true>(p, s)                    \
                  : launch_cfg<TileCfgH<BM, BN, WM, WN, 16, 16, -1>, true>(p, s)
  if (gemm_f16_direct(p.wscale != nullptr, p.cin, tile)) {
    // direct-to-LDS loads, 4 (128x128 with fp16 rows) or 3 K-steps in flight
    // (the 96x128 tile with fp16 rows measured 0.8 % faster with 3 than 4);
    // with slab windows 4 in either (5 measured slower: 128 x 128 by 0.3 %,
    // 96 x 128 by 2.5 %; 4 against 3 for 96 x 128: 1.2 % faster)
    if (tile == TILE_128x128)
      return launch_dma<TileCfgD<128, 128, 2, 4, 4>, TileCfgD<128, 128, 2, 4, 3>, TileCfgD<128, 128, 2, 4, 4>>(p, s);
    return launch_dma<TileCfgD<96, 128, 2, 4, 3>, TileCfgD<96, 128, 2, 4, 3>, TileCfgD<96, 128, 2, 4, 4>>(p, s);
  }
  switch (tile) {
    case TILE_128x128:
      // at most 32-deep K-steps: fewer staging registers, two blocks per CU
      return bk >= 32 ? launch_cfg<TileCfgH<128, 128, 2, 4, 32, 32, 1>, true>(p, s)
                      : launch_cfg<TileCfgH<128, 128, 2, 4, 16, 16, -1>, true>(p, s);
    case TILE_96x128:
      // 64-deep K-steps with registers allocated for four waves per SIMD
      return bk == 64 ? launch_cfg<TileCfgH<96, 128, 2, 4, 64, 32, 0, 4>, true>(p, s)
           : bk == 32 ? launch_cfg<TileCfgH<96, 128, 2, 4, 32, 32, 0>, true>(p, s)
                      : launch_cfg<TileCfgH<96, 128, 2, 4, 16, 16, -1>, true>(p, s);
    case TILE_64x64: VOC_F16_CASES(64, 64, 2, 2, -1);
    case TILE_S64x16:
    case TILE_S64x32: {
      // the MFMA K (SLAB) follows the channel count exactly as above
      const int sk = skinny_bk(p.cin);
#define VOC_F16_SKINNY(BN, WM, WN)                                                           \
  return sk == 128 ? launch_cfg<TileCfgH<64, BN, WM, WN, 128, 32>, true>(p, s)            \
       : sk == 64  ? launch_cfg<TileCfgH<64, BN, WM, WN, 64, 32>, true>(p, s)             \
       : sk == 32  ? launch_cfg<TileCfgH<64, BN, WM, WN, 32, 32>, true>(p, s)             \
                   : launch_cfg<TileCfgH<64, BN, WM, WN, 16, 16, -1>, true>(p, s)
      if (tile == TILE_S64x16) VOC_F16_SKINNY(16, 4, 1);
      VOC_F16_SKINNY(32, 4, 1);
#undef VOC_F16_SKINNY
    }
  }
#undef VOC_F16_CASES
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const ConvParams& p, int tile, bool half, hipStream_t s, const LnArgs* ln) {
  if (p.rows <= 0 || p.M <= 0) return hipSuccess;
  const hipError_t e = half ? launch_blocks_f16(p, tile, s) : launch_blocks_f32(p, tile, s);
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_fold(p, s, ln);
}

}  // namespace

hipError_t launch_conv_gemm(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln) {
  return launch_gemm(p, tile, false, s, ln);
}

bool conv_gemm_rows_ok(const ConvParams& p) {
  if (p.rows < 1 || p.rows > 16 || p.cin % 16 != 0 || p.M % 4 != 0 || p.x_half || p.w_lo) return false;
  const long long ngroups = ((long long)p.k * p.cin + GROUP_K - 1) / GROUP_K;
  return ngroups * 64 * 16 <= 64 * 1024;
}

hipError_t launch_conv_gemm_rows(const ConvParams& p, hipStream_t s) {
  if (!conv_gemm_rows_ok(p)) return hipErrorInvalidValue;
  const int ngroups = (p.k * p.cin + GROUP_K - 1) / GROUP_K;
  const dim3 grid((unsigned)((p.M + 15) / 16)), block(64 * std::min(ngroups, 16));
  const size_t smem = (size_t)ngroups * 64 * sizeof(f32x4);
  if (p.wscale)
    hipLaunchKernelGGL((conv_gemm_rows_kernel<true>), grid, block, smem, s, p, ngroups);
  else
    hipLaunchKernelGGL((conv_gemm_rows_kernel<false>), grid, block, smem, s, p, ngroups);
  return hipGetLastError();
}

hipError_t launch_conv_gemm_f16(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln) {
  return launch_gemm(p, tile, true, s, ln);
}

hipError_t launch_conv_gemm_split(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln) {
  if (p.rows <= 0 || p.M <= 0) return hipSuccess;
  if (!p.w_lo || p.x_half || p.wscale || p.cin % 32 != 0) return hipErrorInvalidValue;
  // two K-steps in flight: the stage holds both weight planes and fp32 rows
  // (28-32 KB), so two rings fit each CU's LDS.  96x128 keeps four waves per
  // SIMD (127 VGPRs); 128x128 needs 149 and runs one block per CU (capped at
  // 128 it spills), so the caller prefers 96-row tiles where M allows.
  // Few-row launches (small chunks) take 4-wave tiles with 3 K-steps in
  // flight: 64x64, or 64 x 32 / 64 x 16 with the waves stacked along M.  Every
  // tile runs the same K-steps and MFMA order: the same bits.
  hipError_t e;
  switch (tile) {
    case TILE_128x128: e = launch_dma_x<TileCfgD<128, 128, 2, 4, 2>, false, true>(p, s); break;
    case TILE_96x128: e = launch_dma_x<TileCfgD<96, 128, 2, 4, 2>, false, true>(p, s); break;
    case TILE_64x64: e = launch_dma_x<TileCfgD<64, 64, 2, 2, 3>, false, true>(p, s); break;
    case TILE_S64x32: e = launch_dma_x<TileCfgD<64, 32, 4, 1, 3>, false, true>(p, s); break;
    case TILE_S64x16: e = launch_dma_x<TileCfgD<64, 16, 4, 1, 3>, false, true>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_fold(p, s, ln);
}

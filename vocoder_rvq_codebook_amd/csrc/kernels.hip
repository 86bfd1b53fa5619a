// Bandwidth-bound and small kernels of the code2wav decoder (gfx950):
// state header / RoPE table, state shift, RVQ gather-sum, LayerNorm, RoPE +
// key/value state write, sliding-window attention, the final C -> 1 conv with
// tanh, weight repacking and fills.

#include <type_traits>

#include "common.h"

namespace {

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

inline unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// begin: validate each stream's state header, publish its position, write the
// next state's header, and build the RoPE cos/sin table [batch][T][half] for
// absolute positions pos + t (angles in float64).
// ---------------------------------------------------------------------------
__global__ void begin_kernel(const float* __restrict__ sin_, float* __restrict__ sout, long long sstride,
                             int batch, int T, uint64_t hash, const double* __restrict__ inv, int half,
                             float* __restrict__ tab, int* __restrict__ pos, int* __restrict__ status) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_stream = (long long)T * (half > 0 ? half : 1);
  if (idx >= (long long)batch * per_stream) return;
  const int b = (int)(idx / per_stream);
  const int r = (int)(idx - (long long)b * per_stream);
  const StateHeader* h = reinterpret_cast<const StateHeader*>(sin_ + (size_t)b * sstride);
  const bool ok = h->magic == VOC_STATE_MAGIC && h->version == VOC_STATE_VERSION && h->cfg_hash == hash &&
                  h->pos >= 0 && h->pos < (1LL << 40);
  const long long p0 = ok ? h->pos : 0;
  if (r == 0) {
    if (!ok) atomicOr(status, VOC_STATUS_STATE);
    pos[b] = (int)(p0 & 0x7fffffff);
    StateHeader* ho = reinterpret_cast<StateHeader*>(sout + (size_t)b * sstride);
    ho->magic = VOC_STATE_MAGIC;
    ho->version = VOC_STATE_VERSION;
    ho->cfg_hash = hash;
    ho->pos = p0 + T;
    for (int i = 0; i < 5; ++i) ho->reserved[i] = 0;
    float* rest = sout + (size_t)b * sstride;
    for (int i = (int)(sizeof(StateHeader) / 4); i < VOC_STATE_HEADER_FLOATS; ++i) rest[i] = 0.f;
  }
  if (half > 0) {
    const int t = r / half, i = r - t * half;
    const double ang = (double)(p0 + t) * inv[i];
    float* o = tab + (((size_t)b * T + t) * half + i) * 2;
    o[0] = (float)cos(ang);
    o[1] = (float)sin(ang);
  }
}

// ---------------------------------------------------------------------------
// state shift: for a slot of H rows that gains N = T*rate rows this call,
// rows [N, H) of the old state become rows [0, H-N) of the new one (the rest
// is written by the kernel that produces the new rows).  The slot's alignment
// padding is zeroed, so every byte of the new state is defined.
// ---------------------------------------------------------------------------
// grid: (slot, stream, part); the parts split each slot's copy evenly.
__global__ void state_shift_kernel(const Slot* __restrict__ slots, const float* __restrict__ sin_,
                                   float* __restrict__ sout, long long sstride, int T) {
  const Slot sl = slots[blockIdx.x];
  const int b = blockIdx.y;
  float* dst = sout + (size_t)b * sstride + sl.off;
  const long long used = (long long)sl.H * sl.C;
  if (blockIdx.z == 0)
    for (long long i = used + threadIdx.x; i < sl.cap; i += blockDim.x) dst[i] = 0.f;
  const long long N = (long long)T * sl.rate;
  if (N >= sl.H) return;
  const long long keep = (long long)(sl.H - N) * sl.C;  // a multiple of 4 (C is)
  const float* src = sin_ + (size_t)b * sstride + sl.off + N * sl.C;
  const long long per = (keep / 4 + gridDim.z - 1) / gridDim.z;
  const long long i0 = per * blockIdx.z, i1 = min(keep / 4, i0 + per);
  for (long long i = i0 + threadIdx.x; i < i1; i += blockDim.x) st4(dst + 4 * i, ld4(src + 4 * i));
}

// ---------------------------------------------------------------------------
// RVQ gather-sum: e[row] = sum over q (ascending) of codebooks[q][codes[row][q]],
// one fp32 add per codebook.  A code outside [0, V) flags the status word and
// contributes nothing.  With Q a multiple of 8 the codebooks are taken 8 at a
// time, branch-free: their 8 codes in two 16-byte loads, then the 8 codeword
// pieces (an out-of-range code reads row 0 of its codebook, in bounds, and
// its value is dropped), then the adds in order; a row waits on memory twice
// per 8 codebooks instead of twice per codebook.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gather_add(f32x4& e, f32x4 w, int q) {
  if (q == 0) {
    e = w;
  } else {
    e.x = __fadd_rn(e.x, w.x);
    e.y = __fadd_rn(e.y, w.y);
    e.z = __fadd_rn(e.z, w.z);
    e.w = __fadd_rn(e.w, w.w);
  }
}

__global__ void gather_kernel(const int32_t* __restrict__ codes, const float* __restrict__ cb, int Q, int V,
                              int D, int rows, int T, float* __restrict__ out, float* __restrict__ hist, int H,
                              long long sstride, int* __restrict__ status) {
  const int D4 = D / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)rows * D4) return;
  const int row = (int)(idx / D4);
  const int c = (int)(idx - (long long)row * D4) * 4;
  const int32_t* cr = codes + (size_t)row * Q;
  f32x4 e = {0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  if (Q % 8 == 0) {
    for (int q0 = 0; q0 < Q; q0 += 8) {
      const int4 c0 = *reinterpret_cast<const int4*>(cr + q0);
      const int4 c1 = *reinterpret_cast<const int4*>(cr + q0 + 4);
      const int code[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      bool ok[8];
      f32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ok[u] = code[u] >= 0 && code[u] < V;
        w[u] = ld4(cb + ((size_t)(q0 + u) * V + (ok[u] ? code[u] : 0)) * D + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (ok[u])
          gather_add(e, w[u], q0 + u);
        else
          bad = true;
      }
    }
  } else {
    for (int q = 0; q < Q; ++q) {
      const int code = cr[q];
      if (code < 0 || code >= V) {
        bad = true;
        continue;
      }
      gather_add(e, ld4(cb + ((size_t)q * V + code) * D + c), q);
    }
  }
  if (bad && c == 0) atomicOr(status, VOC_STATUS_CODE);
  st4(out + (size_t)row * D + c, e);
  const int b = row / T, t = row - b * T;
  if (hist && t >= T - H) st4(hist + (size_t)b * sstride + (size_t)(H - T + t) * D + c, e);
}

// ---------------------------------------------------------------------------
// LayerNorm over d channels (layernorm_block): one block of 64 * NV threads
// per row, biased variance, two passes.  Optionally writes the last H rows of
// each stream into a state slot.
// ---------------------------------------------------------------------------
template <int NV>
__global__ __launch_bounds__(64 * NV) void layernorm_kernel(const float* __restrict__ x, const LnArgs a) {
  __shared__ float red[64 * NV + 1];
  const int row = blockIdx.x;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if ((int)threadIdx.x < a.d / 4) v = ld4(x + (size_t)row * a.d + 4 * threadIdx.x);
  layernorm_block<NV>(a, v, row, red);
}

// ---------------------------------------------------------------------------
// Sliding-window attention.  Block = (query tile of QT frames, head, stream);
// the keys and values the tile needs (state window + new frames) are staged
// in LDS.  Query at absolute position P attends positions [P - W, P]; lane
// o <-> key position P - W + o, so every reduction order depends only on
// absolute positions.
// ---------------------------------------------------------------------------
constexpr int ATT_QT = 16;
constexpr int ATT_THREADS = 256;

// RoPE of one rotate-half pair of 4-wide pieces (channels c..c+3 and
// c+hd/2..c+hd/2+3) of frame row `row` (table entries (cos, sin) per row and i)
__device__ __forceinline__ void rope4(f32x4& x1, f32x4& x2, const float* __restrict__ tab, size_t row, int half,
                                      int c) {
  const float* cs = tab + (row * half + c) * 2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float co = cs[2 * e], sn = cs[2 * e + 1];
    const float a = x1[e], bb = x2[e];
    x1[e] = a * co - bb * sn;
    x2[e] = a * sn + bb * co;
  }
}

__global__ __launch_bounds__(ATT_THREADS) void attention_kernel(
    const float* __restrict__ qkv, const float* __restrict__ ks, const float* __restrict__ vs, long long sstride,
    const int* __restrict__ pos, int T, int n_heads, int hd, int W, const float* __restrict__ tab,
    float* __restrict__ ks_out, float* __restrict__ vs_out, float* __restrict__ out) {
  extern __shared__ float smem[];
  const int d = n_heads * hd;
  const int t0 = blockIdx.x * ATT_QT, h = blockIdx.y, b = blockIdx.z;
  const int p0 = pos[b];
  const int nq = min(ATT_QT, T - t0);
  const int nk = nq + W;  // concat rows j in [t0, t0 + nq - 1 + W]
  const int ldk = hd + 1;
  float* Ks = smem;                       // [(QT + W)][ldk]
  float* Vs = Ks + (ATT_QT + W) * ldk;    // [(QT + W)][hd]
  float* Qs = Vs + (ATT_QT + W) * hd;     // [QT][hd]
  const int tid = threadIdx.x;
  // Staged with 16-byte loads, a rotate-half pair of pieces per thread (hd is
  // a multiple of 8).  State rows hold rotated keys already; new frames' q
  // and k are rotated here, and the block whose query tile holds a new frame
  // writes that frame's rotated key and its value to the state tail.
  const int half = hd / 2, half4 = half / 4;
  for (int idx = tid; idx < nk * half4; idx += ATT_THREADS) {
    const int r = idx / half4, c = (idx - r * half4) * 4;
    const int j = t0 + r;  // concat index: j < W state row, else new frame j - W
    f32x4 k1 = {0.f, 0.f, 0.f, 0.f}, k2 = k1, v1 = k1, v2 = k1;
    if (j < W) {
      if (p0 - W + j >= 0) {
        const size_t o = (size_t)b * sstride + (size_t)j * d + h * hd + c;
        k1 = *reinterpret_cast<const f32x4*>(ks + o);
        k2 = *reinterpret_cast<const f32x4*>(ks + o + half);
        v1 = *reinterpret_cast<const f32x4*>(vs + o);
        v2 = *reinterpret_cast<const f32x4*>(vs + o + half);
      }
    } else if (j - W < T) {
      const int t = j - W;
      const size_t grow = (size_t)b * T + t;
      const float* row = qkv + grow * 3 * d + h * hd + c;
      k1 = *reinterpret_cast<const f32x4*>(row + d);
      k2 = *reinterpret_cast<const f32x4*>(row + d + half);
      v1 = *reinterpret_cast<const f32x4*>(row + 2 * d);
      v2 = *reinterpret_cast<const f32x4*>(row + 2 * d + half);
      rope4(k1, k2, tab, grow, half, c);
      if (W > 0 && t >= t0 && t < t0 + nq && t >= T - W) {
        const size_t o = (size_t)b * sstride + (size_t)(W - T + t) * d + h * hd + c;
        *reinterpret_cast<f32x4*>(ks_out + o) = k1;
        *reinterpret_cast<f32x4*>(ks_out + o + half) = k2;
        *reinterpret_cast<f32x4*>(vs_out + o) = v1;
        *reinterpret_cast<f32x4*>(vs_out + o + half) = v2;
      }
    }
    float* kd = Ks + r * ldk + c;
    kd[0] = k1.x; kd[1] = k1.y; kd[2] = k1.z; kd[3] = k1.w;
    kd[half] = k2.x; kd[half + 1] = k2.y; kd[half + 2] = k2.z; kd[half + 3] = k2.w;
    *reinterpret_cast<f32x4*>(Vs + r * hd + c) = v1;
    *reinterpret_cast<f32x4*>(Vs + r * hd + c + half) = v2;
  }
  for (int idx = tid; idx < nq * half4; idx += ATT_THREADS) {
    const int r = idx / half4, c = (idx - r * half4) * 4;
    const size_t grow = (size_t)b * T + t0 + r;
    const float* row = qkv + grow * 3 * d + h * hd + c;
    f32x4 q1 = *reinterpret_cast<const f32x4*>(row);
    f32x4 q2 = *reinterpret_cast<const f32x4*>(row + half);
    rope4(q1, q2, tab, grow, half, c);
    *reinterpret_cast<f32x4*>(Qs + r * hd + c) = q1;
    *reinterpret_cast<f32x4*>(Qs + r * hd + c + half) = q2;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const float scale = 1.0f / sqrtf((float)hd);
  for (int tl = wave; tl < nq; tl += ATT_THREADS / 64) {
    const long long P = (long long)p0 + t0 + tl;
    const float* qv = Qs + tl * hd;
    float e[4];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = lane + 64 * u;
      e[u] = -INFINITY;
      if (o <= W && P - W + o >= 0) {
        const float* kr = Ks + (tl + o) * ldk;
        float s = 0.f;
        for (int c = 0; c < hd; ++c) s += qv[c] * kr[c];
        e[u] = s * scale;
        m = fmaxf(m, e[u]);
      }
    }
    m = wave_max(m);
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = lane + 64 * u;
      e[u] = (o <= W && P - W + o >= 0) ? expf(e[u] - m) : 0.f;
      part += e[u];
    }
    const float denom = wave_sum(part);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
      for (int oo = 0; oo < 64; ++oo) {
        const int o = 64 * ub + oo;
        if (o > W) break;
        const float pw = __shfl(e[ub], oo, 64);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = lane + 64 * u;
          if (c < hd) acc[u] += pw * Vs[(tl + o) * hd + c];
        }
      }
    }
    float* orow = out + ((size_t)b * T + t0 + tl) * d + h * hd;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = lane + 64 * u;
      if (c < hd) orow[c] = acc[u] / denom;
    }
  }
}

// The same attention for a compile-time head size HD (a multiple of 4), with
// the compute loops vectorised: key rows padded to HD + 4 floats so that a
// lane reads its key in 16-byte pieces, and each wave's softmax weights
// staged in LDS so that the value loop reads them as broadcasts instead of
// lane shuffles, with a fixed trip count.  Every score, max, sum and
// accumulation takes the same operations in the same order as
// attention_kernel: the same bits.
template <int HD>
__global__ __launch_bounds__(ATT_THREADS) void attention_hd_kernel(
    const float* __restrict__ qkv, const float* __restrict__ ks, const float* __restrict__ vs, long long sstride,
    const int* __restrict__ pos, int T, int n_heads, int W, const float* __restrict__ tab,
    float* __restrict__ ks_out, float* __restrict__ vs_out, float* __restrict__ out) {
  static_assert(HD % 8 == 0 && HD <= 256, "head size");
  constexpr int LDK = HD + 4;
  constexpr int NU = (HD + 63) / 64;  // output channels per lane
  extern __shared__ float smem[];
  const int d = n_heads * HD;
  const int t0 = blockIdx.x * ATT_QT, h = blockIdx.y, b = blockIdx.z;
  const int p0 = pos[b];
  const int nq = min(ATT_QT, T - t0);
  const int nk = nq + W;
  const int es = (W + 4) & ~3;            // softmax weights per wave (W + 1, rounded up to 4)
  float* Ks = smem;                       // [(QT + W)][LDK]
  float* Vs = Ks + (ATT_QT + W) * LDK;    // [(QT + W)][HD]
  float* Qs = Vs + (ATT_QT + W) * HD;     // [QT][HD]
  float* Es = Qs + ATT_QT * HD;           // [waves][es]
  const int tid = threadIdx.x;
  constexpr int half = HD / 2, half4 = half / 4;
  for (int idx = tid; idx < nk * half4; idx += ATT_THREADS) {
    const int r = idx / half4, c = (idx - r * half4) * 4;
    const int j = t0 + r;  // concat index: j < W state row, else new frame j - W
    f32x4 k1 = {0.f, 0.f, 0.f, 0.f}, k2 = k1, v1 = k1, v2 = k1;
    if (j < W) {
      if (p0 - W + j >= 0) {
        const size_t o = (size_t)b * sstride + (size_t)j * d + h * HD + c;
        k1 = *reinterpret_cast<const f32x4*>(ks + o);
        k2 = *reinterpret_cast<const f32x4*>(ks + o + half);
        v1 = *reinterpret_cast<const f32x4*>(vs + o);
        v2 = *reinterpret_cast<const f32x4*>(vs + o + half);
      }
    } else if (j - W < T) {
      const int t = j - W;
      const size_t grow = (size_t)b * T + t;
      const float* row = qkv + grow * 3 * d + h * HD + c;
      k1 = *reinterpret_cast<const f32x4*>(row + d);
      k2 = *reinterpret_cast<const f32x4*>(row + d + half);
      v1 = *reinterpret_cast<const f32x4*>(row + 2 * d);
      v2 = *reinterpret_cast<const f32x4*>(row + 2 * d + half);
      rope4(k1, k2, tab, grow, half, c);
      if (W > 0 && t >= t0 && t < t0 + nq && t >= T - W) {
        const size_t o = (size_t)b * sstride + (size_t)(W - T + t) * d + h * HD + c;
        *reinterpret_cast<f32x4*>(ks_out + o) = k1;
        *reinterpret_cast<f32x4*>(ks_out + o + half) = k2;
        *reinterpret_cast<f32x4*>(vs_out + o) = v1;
        *reinterpret_cast<f32x4*>(vs_out + o + half) = v2;
      }
    }
    *reinterpret_cast<f32x4*>(Ks + r * LDK + c) = k1;
    *reinterpret_cast<f32x4*>(Ks + r * LDK + c + half) = k2;
    *reinterpret_cast<f32x4*>(Vs + r * HD + c) = v1;
    *reinterpret_cast<f32x4*>(Vs + r * HD + c + half) = v2;
  }
  for (int idx = tid; idx < nq * half4; idx += ATT_THREADS) {
    const int r = idx / half4, c = (idx - r * half4) * 4;
    const size_t grow = (size_t)b * T + t0 + r;
    const float* row = qkv + grow * 3 * d + h * HD + c;
    f32x4 q1 = *reinterpret_cast<const f32x4*>(row);
    f32x4 q2 = *reinterpret_cast<const f32x4*>(row + half);
    rope4(q1, q2, tab, grow, half, c);
    *reinterpret_cast<f32x4*>(Qs + r * HD + c) = q1;
    *reinterpret_cast<f32x4*>(Qs + r * HD + c + half) = q2;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const float scale = 1.0f / sqrtf((float)HD);
  float* Ew = Es + wave * es;
  for (int tl = wave; tl < nq; tl += ATT_THREADS / 64) {
    const long long P = (long long)p0 + t0 + tl;
    const f32x4* q4 = reinterpret_cast<const f32x4*>(Qs + tl * HD);
    float e[4];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = lane + 64 * u;
      e[u] = -INFINITY;
      if (o <= W && P - W + o >= 0) {
        const f32x4* k4 = reinterpret_cast<const f32x4*>(Ks + (tl + o) * LDK);
        float sc = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < HD / 4; ++c4) {
          const f32x4 qq = q4[c4], kk = k4[c4];
          sc += qq.x * kk.x;
          sc += qq.y * kk.y;
          sc += qq.z * kk.z;
          sc += qq.w * kk.w;
        }
        e[u] = sc * scale;
        m = fmaxf(m, e[u]);
      }
    }
    m = wave_max(m);
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = lane + 64 * u;
      e[u] = (o <= W && P - W + o >= 0) ? expf(e[u] - m) : 0.f;
      part += e[u];
      if (o <= W) Ew[o] = e[u];
    }
    const float denom = wave_sum(part);
    float acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = 0.f;
    const float* vrow = Vs + tl * HD;
#pragma unroll 8
    for (int o = 0; o <= W; ++o) {
      const float pw = Ew[o];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = lane + 64 * u;
        if (c < HD) acc[u] += pw * vrow[o * HD + c];
      }
    }
    float* orow = out + ((size_t)b * T + t0 + tl) * d + h * HD;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = lane + 64 * u;
      if (c < HD) orow[c] = acc[u] / denom;
    }
  }
}

// ---------------------------------------------------------------------------
// Final conv C -> 1 (kernel k, causal, history from the state) and tanh.
// A block owns POST_ROWS consecutive output samples: it stages those input
// rows and the k-1 rows before them in LDS with coalesced float4 loads (row
// stride C+1 so that lanes reading different rows hit different banks), then
// each thread reduces its own sample in a fixed (tap, channel) order.  Rows
// before a stream's chunk come from its history slot.
// ---------------------------------------------------------------------------
constexpr int POST_ROWS = 128;

__global__ __launch_bounds__(POST_ROWS) void conv_post_kernel(
    const float* __restrict__ x, const float* __restrict__ hin, long long sstride, int H,
    const float* __restrict__ w, const float* __restrict__ bias, int C, int k, int rows, int nin,
    float* __restrict__ pcm, float* __restrict__ pre) {
  extern __shared__ float sm[];
  const int ld = C + 1;
  float* ws = sm;                        // [k][C]
  float* xs = sm + k * C;                // [(POST_ROWS + k - 1)][ld]
  const int g0 = blockIdx.x * POST_ROWS;
  const int nr = min(POST_ROWS, rows - g0) + k - 1;
  for (int i = threadIdx.x; i < k * C; i += POST_ROWS) ws[i] = w[i];
  const int c4n = C / 4;
  for (int i = threadIdx.x; i < nr * c4n; i += POST_ROWS) {
    const int r = i / c4n, c = (i - r * c4n) * 4;
    const int g = g0 - (k - 1) + r;      // global input row; rows of another stream are staged but unused
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (g >= 0) v = ld4(x + (size_t)g * C + c);
    float* d = xs + r * ld + c;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int g = g0 + t;
  if (g >= rows) return;
  const int b = g / nin, n = g - b * nin;
  float acc = bias[0];
  for (int j = 0; j < k; ++j) {
    const int n2 = n - (k - 1 - j);
    const float* wj = ws + j * C;
    float dot = 0.f;
    if (n2 >= 0) {
      const float* xr = xs + (t + j) * ld;
      for (int c = 0; c < C; ++c) dot = fmaf(wj[c], xr[c], dot);
    } else {
      const float* xr = hin + (size_t)b * sstride + (size_t)(H + n2) * C;
      for (int c = 0; c < C; ++c) dot = fmaf(wj[c], xr[c], dot);
    }
    acc += dot;
  }
  if (pre) pre[g] = acc;
  pcm[g] = tanhf(acc);
}

// The same conv for a kernel size known at compile time, reading every input
// row from HBM once: thread t of a block sums its own input row against all K
// taps (K dot products over the channels, each a fused multiply-add chain in
// channel order), the block exchanges the tap sums through LDS, and output
// sample g adds bias + sum over taps j of the sum of row g-(K-1)+j, in tap
// order -- the operations and order of conv_post_kernel, so the same bits.
// A block covers POST_T input rows and emits the POST_T-(K-1) samples whose
// rows it holds; a tap reaching before the stream's chunk is summed from the
// history slot in place.  The rows are staged through LDS one channel slab at
// a time (slab channels of every row: a 128-byte line per row for 32-channel
// slabs), with loads that cover whole lines, so each line is fetched from HBM
// once instead of being revisited by one lane across its row.
constexpr int POST_T = 256;
constexpr int POST_SLAB_F4 = 8;  // float4 per row of the widest slab (32 channels)

template <int K>
__global__ __launch_bounds__(POST_T) void conv_post_rows_kernel(
    const float* __restrict__ x, const float* __restrict__ hin, long long sstride, int H,
    const float* __restrict__ w, const float* __restrict__ bias, int C, int slab, int rows, int nin,
    float* __restrict__ pcm, float* __restrict__ pre) {
  extern __shared__ float sm[];
  const int ld = slab + 4;   // padded slab row (floats)
  float* ws = sm;            // [K][C]
  float* ys = sm + K * C;    // [POST_T][K]: tap sums of each row
  float* xs = ys + POST_T * K;  // [POST_T][ld]: one channel slab of the block's rows
  constexpr int OUT = POST_T - (K - 1);
  const int t = threadIdx.x;
  const int g_out0 = blockIdx.x * OUT;
  const int row0 = g_out0 - (K - 1);
  for (int i = t; i < K * C; i += POST_T) ws[i] = w[i];
  const int gr = row0 + t;  // input row of this thread
  const bool mine = gr >= 0 && gr < rows;
  float dot[K];
#pragma unroll
  for (int j = 0; j < K; ++j) dot[j] = 0.f;
  // slab c0's loads go to registers (thread t: float4 t, t + POST_T, ... of
  // the slab's [POST_T][slab] tile) while the previous slab is summed from LDS
  const int q4 = slab / 4;  // float4 per row per slab, at most POST_SLAB_F4
  f32x4 buf[POST_SLAB_F4];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < POST_SLAB_F4; ++u) {
      if (u >= q4) break;
      const int i = t + u * POST_T, r = i / q4, q = i - r * q4;
      const int g = row0 + r;
      buf[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (g >= 0 && g < rows) buf[u] = ld4(x + (size_t)g * C + c0 + 4 * q);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < POST_SLAB_F4; ++u) {
      if (u >= q4) break;
      const int i = t + u * POST_T, r = i / q4, q = i - r * q4;
      st4(xs + r * ld + 4 * q, buf[u]);
    }
  };
  load(0);
  for (int c0 = 0; c0 < C; c0 += slab) {
    store();
    __syncthreads();
    if (c0 + slab < C) load(c0 + slab);
    if (mine) {
      const float* xr = xs + t * ld;
      for (int c = 0; c < slab; c += 4) {
        const f32x4 v = ld4(xr + c);
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const f32x4 wv = ld4(ws + j * C + c0 + c);
          dot[j] = fmaf(wv.x, v.x, dot[j]);
          dot[j] = fmaf(wv.y, v.y, dot[j]);
          dot[j] = fmaf(wv.z, v.z, dot[j]);
          dot[j] = fmaf(wv.w, v.w, dot[j]);
        }
      }
    }
    __syncthreads();
  }
  if (mine) {
#pragma unroll
    for (int j = 0; j < K; ++j) ys[t * K + j] = dot[j];
  }
  __syncthreads();
  if (t < K - 1) return;
  const int g = g_out0 + (t - (K - 1));
  if (g >= rows) return;
  const int b = g / nin, n = g - b * nin;
  float acc = bias[0];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int n2 = n - (K - 1 - j);
    if (n2 >= 0) {
      acc += ys[(t - (K - 1) + j) * K + j];
    } else {
      const float* wj = ws + j * C;
      const float* hr = hin + (size_t)b * sstride + (size_t)(H + n2) * C;
      float dot = 0.f;
      for (int c = 0; c < C; ++c) dot = fmaf(wj[c], hr[c], dot);
      acc += dot;
    }
  }
  if (pre) pre[g] = acc;
  pcm[g] = tanhf(acc);
}

// ---------------------------------------------------------------------------
// weight repacking (create time)
// ---------------------------------------------------------------------------
// Row m of the packed weights at position idx: tap j and input channel c.
// Tap-major rows are [k][cin]; slab-ordered rows are [cin / 32][k][32] (the
// 32-channel slabs of the fp16 GEMMs' channel-major reduction order).
__device__ __forceinline__ void packed_pos(long long idx, int cin, int k, bool slab, int& m, int& j, int& c) {
  if (slab) {
    const int e = (int)(idx & 31);
    const long long r1 = idx >> 5;
    j = (int)(r1 % k);
    const long long r2 = r1 / k;
    const int nb = cin / 32;
    c = (int)(r2 % nb) * 32 + e;
    m = (int)(r2 / nb);
  } else {
    c = (int)(idx % cin);
    const long long r = idx / cin;
    j = (int)(r % k);
    m = (int)(r / k);
  }
}

// Store one packed value: T is the packed element type (float, or _Float16
// rounded to nearest even); fp16 with lo_off > 0 stores the split of v times
// sc (a power of two: exact), its lo half lo_off elements further on, and
// flags a value whose hi half is not finite (|v sc| >= 65520, or NaN).
template <typename T>
__device__ __forceinline__ void put_packed(T* dst, long long idx, float v, long long lo_off, float sc,
                                           int* range_flag) {
  if constexpr (std::is_same<T, _Float16>::value) {
    if (lo_off > 0) {
      v *= sc;
      const _Float16 h = (_Float16)v;
      dst[idx] = h;
      dst[idx + lo_off] = split_lo(v, h);
      if (!(fabsf(v) < 65520.f)) *range_flag = 1;  // every writer stores the same value
      return;
    }
  }
  dst[idx] = (T)v;
}

// Conv1d / Linear [M][cin][k] -> [Mpad] packed rows, zero rows past M.
template <typename T>
__global__ void repack_conv_kernel(const float* __restrict__ src, T* __restrict__ dst, int M, int Mpad,
                                   int cin, int k, int slab, long long lo_off, float sc, int* range_flag) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)Mpad * k * cin;
  if (idx >= total) return;
  int m, j, c;
  packed_pos(idx, cin, k, slab != 0, m, j, c);
  put_packed(dst, idx, m < M ? src[((size_t)m * cin + c) * k + j] : 0.f, lo_off, sc, range_flag);
}

// ConvTranspose1d [cin][cout][2s] -> [Mpad][2][cin] with row m = p*cout + o:
// tap 0 (input row t-1) takes kernel index p + s, tap 1 (row t) takes p.
template <typename T>
__global__ void repack_convT_kernel(const float* __restrict__ src, T* __restrict__ dst, int cin, int cout,
                                    int s, int Mpad, int slab, long long lo_off, float sc, int* range_flag) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)Mpad * 2 * cin;
  if (idx >= total) return;
  int m, j, c;
  packed_pos(idx, cin, 2, slab != 0, m, j, c);
  float v = 0.f;
  if (m < s * cout) {
    const int p = m / cout, o = m - p * cout;
    const int kk = j == 0 ? p + s : p;
    v = src[((size_t)c * cout + o) * (2 * s) + kk];
  }
  put_packed(dst, idx, v, lo_off, sc, range_flag);
}

// int8 quantization of one group of 32 consecutive values of a row ("blixt/
// phonon", section Weights): the values rounded to fp16, scale = fp16(max |v| /
// 127), each value rint(v / scale) (ties to even); divisions correctly rounded
// in fp32; a zero group keeps scale 0 and values 0.  One thread per group.
// int8 weights back to the GEMM operand: value = q * scale of its group of 32
// (exact in fp32), stored as fp32 or rounded once to fp16 -- what the int8
// GEMM kernels compute per tile.  One thread per 8 values.
__global__ void dequant_rows_kernel(const int8_t* __restrict__ q, const _Float16* __restrict__ scale,
                                    long long units, void* __restrict__ dst, int half) {
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const uint2 w = *reinterpret_cast<const uint2*>(q + u * 8);
  const float sc = (float)scale[u >> 2];
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (float)(int8_t)(w.x >> (8 * i)) * sc;
    v[4 + i] = (float)(int8_t)(w.y >> (8 * i)) * sc;
  }
  if (half) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)v[i];
    reinterpret_cast<h8*>(dst)[u] = r;
  } else {
    f32x4* o = reinterpret_cast<f32x4*>(dst) + 2 * u;
    o[0] = (f32x4){v[0], v[1], v[2], v[3]};
    o[1] = (f32x4){v[4], v[5], v[6], v[7]};
  }
}

__global__ void quantize_rows_kernel(const float* __restrict__ src, long long groups, int8_t* __restrict__ q,
                                     _Float16* __restrict__ scale) {
  const long long gi = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= groups) return;
  const float* x = src + gi * 32;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = (float)(_Float16)x[i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const _Float16 sh = (_Float16)__fdiv_rn(amax, 127.0f);
  const float sc = (float)sh;
  uint32_t words[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t packed = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int qi = sc > 0.f ? (int)rintf(__fdiv_rn(v[4 * w + b], sc)) : 0;
      packed |= (uint32_t)(qi & 0xff) << (8 * b);
    }
    words[w] = packed;
  }
  uint4* qd = reinterpret_cast<uint4*>(q + gi * 32);
  qd[0] = make_uint4(words[0], words[1], words[2], words[3]);
  qd[1] = make_uint4(words[4], words[5], words[6], words[7]);
  scale[gi] = sh;
}

// per-channel vector [C] -> [Mpad] indexed by GEMM column m = p*C + c
__global__ void expand_vec_kernel(const float* __restrict__ src, float* __restrict__ dst, int C, int phases,
                                  int Mpad) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= Mpad) return;
  dst[m] = m < C * phases ? src[m % C] : 0.f;
}

__global__ void fill_kernel(uint32_t* __restrict__ dst, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = 0u;
}

__global__ void copy_kernel(f32x4* __restrict__ dst, const f32x4* __restrict__ src, long long n4) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long long)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void reset_headers_kernel(float* __restrict__ state, long long sstride, int batch, uint64_t hash) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  StateHeader* h = reinterpret_cast<StateHeader*>(state + (size_t)b * sstride);
  h->magic = VOC_STATE_MAGIC;
  h->version = VOC_STATE_VERSION;
  h->cfg_hash = hash;
  h->pos = 0;
  for (int i = 0; i < 5; ++i) h->reserved[i] = 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_begin(const void* state_in, void* state_out, long long sstride, int batch, int T,
                        uint64_t cfg_hash, const double* inv_freq, int half, float* rope_tab, int* pos,
                        int* status, hipStream_t s) {
  const long long n = (long long)batch * T * (half > 0 ? half : 1);
  hipLaunchKernelGGL(begin_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, (const float*)state_in,
                     (float*)state_out, sstride, batch, T, cfg_hash, inv_freq, half, rope_tab, pos, status);
  return hipGetLastError();
}

hipError_t launch_state_shift(const Slot* slots, int nslots, int max_h, const float* state_in, float* state_out,
                              long long sstride, int batch, int T, hipStream_t s) {
  (void)max_h;
  if (nslots == 0) return hipSuccess;
  hipLaunchKernelGGL(state_shift_kernel, dim3(nslots, batch, 16), dim3(256), 0, s, slots, state_in, state_out,
                     sstride, T);
  return hipGetLastError();
}

hipError_t launch_gather(const int32_t* codes, const float* codebooks, int Q, int V, int D, int rows, int T,
                         float* out, float* hist, int H, long long sstride, int* status, hipStream_t s) {
  const long long n = (long long)rows * (D / 4);
  hipLaunchKernelGGL(gather_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, codes, codebooks, Q, V, D, rows, T, out,
                     hist, H, sstride, status);
  return hipGetLastError();
}

int layernorm_nv(int d) {
  const int need = cdiv(d / 4, 64);
  int nv = 1;
  while (nv < need) nv *= 2;
  return d % 4 == 0 && nv <= LN_MAX_NV ? nv : 0;
}

hipError_t launch_layernorm(const float* x, const float* g, const float* b, float eps, int rows, int d, float* out,
                            int T, float* hist, int H, long long sstride, hipStream_t s) {
  const LnArgs a{g, b, eps, d, out, T, hist, H, sstride};
  if (rows <= 0) return hipSuccess;
  const int nv = layernorm_nv(d);
  const dim3 grid(rows), block(64 * nv);
  switch (nv) {
    case 1: hipLaunchKernelGGL(layernorm_kernel<1>, grid, block, 0, s, x, a); break;
    case 2: hipLaunchKernelGGL(layernorm_kernel<2>, grid, block, 0, s, x, a); break;
    case 4: hipLaunchKernelGGL(layernorm_kernel<4>, grid, block, 0, s, x, a); break;
    case 8: hipLaunchKernelGGL(layernorm_kernel<8>, grid, block, 0, s, x, a); break;
    case 16: hipLaunchKernelGGL(layernorm_kernel<16>, grid, block, 0, s, x, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
hipError_t launch_attention_hd(const float* qkv, const float* k_state, const float* v_state, long long sstride,
                               const int* pos, int batch, int T, int n_heads, int W, const float* rope_tab,
                               float* k_state_out, float* v_state_out, float* out, hipStream_t s) {
  const size_t smem = ((size_t)(ATT_QT + W) * (HD + 4) + (size_t)(ATT_QT + W) * HD + (size_t)ATT_QT * HD +
                       (size_t)(ATT_THREADS / 64) * ((W + 4) & ~3)) *
                      sizeof(float);
  if (smem > 64 * 1024 || W > 255) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_hd_kernel<HD>, dim3(cdiv(T, ATT_QT), n_heads, batch), dim3(ATT_THREADS), smem, s, qkv,
                     k_state, v_state, sstride, pos, T, n_heads, W, rope_tab, k_state_out, v_state_out, out);
  return hipGetLastError();
}

hipError_t launch_attention(const float* qkv, const float* k_state, const float* v_state, long long sstride,
                            const int* pos, int batch, int T, int n_heads, int hd, int W, const float* rope_tab,
                            float* k_state_out, float* v_state_out, float* out, hipStream_t s) {
  switch (hd) {
    case 16: return launch_attention_hd<16>(qkv, k_state, v_state, sstride, pos, batch, T, n_heads, W, rope_tab,
                                            k_state_out, v_state_out, out, s);
    case 32: return launch_attention_hd<32>(qkv, k_state, v_state, sstride, pos, batch, T, n_heads, W, rope_tab,
                                            k_state_out, v_state_out, out, s);
    case 64: return launch_attention_hd<64>(qkv, k_state, v_state, sstride, pos, batch, T, n_heads, W, rope_tab,
                                            k_state_out, v_state_out, out, s);
    case 128: return launch_attention_hd<128>(qkv, k_state, v_state, sstride, pos, batch, T, n_heads, W, rope_tab,
                                              k_state_out, v_state_out, out, s);
    default: break;
  }
  const size_t smem = ((size_t)(ATT_QT + W) * (hd + 1) + (size_t)(ATT_QT + W) * hd + (size_t)ATT_QT * hd) *
                      sizeof(float);
  if (smem > 64 * 1024 || hd % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_kernel, dim3(cdiv(T, ATT_QT), n_heads, batch), dim3(ATT_THREADS), smem, s, qkv,
                     k_state, v_state, sstride, pos, T, n_heads, hd, W, rope_tab, k_state_out, v_state_out, out);
  return hipGetLastError();
}

hipError_t launch_conv_post(const float* x, const float* hin, long long sstride, int H, const float* w,
                            const float* bias, int C, int k, int rows, int nin, float* pcm, float* pre_tanh,
                            hipStream_t s) {
  if (k == 7 && C % 4 == 0) {
    const int slab = C % 32 == 0 ? 32 : C % 16 == 0 ? 16 : C % 8 == 0 ? 8 : 4;
    const size_t smem7 = ((size_t)7 * C + (size_t)POST_T * 7 + (size_t)POST_T * (slab + 4)) * sizeof(float);
    if (smem7 > 64 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(conv_post_rows_kernel<7>, dim3(cdiv(rows, POST_T - 6)), dim3(POST_T), smem7, s, x, hin,
                       sstride, H, w, bias, C, slab, rows, nin, pcm, pre_tanh);
    return hipGetLastError();
  }
  const size_t smem = ((size_t)k * C + (size_t)(POST_ROWS + k - 1) * (C + 1)) * sizeof(float);
  if (smem > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(conv_post_kernel, dim3(cdiv(rows, POST_ROWS)), dim3(POST_ROWS), smem, s, x, hin, sstride, H, w,
                     bias, C, k, rows, nin, pcm, pre_tanh);
  return hipGetLastError();
}

hipError_t launch_repack_conv(const float* src, void* dst, int M, int Mpad, int cin, int k, bool half_out,
                              bool slab, hipStream_t s, long long lo_off, float split_scale, int* range_flag) {
  const long long n = (long long)Mpad * k * cin;
  if (slab && cin % 32) return hipErrorInvalidValue;
  if (lo_off < 0 || (lo_off > 0 && (!half_out || !range_flag))) return hipErrorInvalidValue;
  if (half_out)
    hipLaunchKernelGGL(repack_conv_kernel<_Float16>, dim3(cdiv(n, 256)), dim3(256), 0, s, src, (_Float16*)dst, M,
                       Mpad, cin, k, slab ? 1 : 0, lo_off, split_scale, range_flag);
  else
    hipLaunchKernelGGL(repack_conv_kernel<float>, dim3(cdiv(n, 256)), dim3(256), 0, s, src, (float*)dst, M, Mpad,
                       cin, k, slab ? 1 : 0, 0LL, 1.f, nullptr);
  return hipGetLastError();
}

hipError_t launch_repack_convT(const float* src, void* dst, int cin, int cout, int stride, int Mpad, bool half_out,
                               bool slab, hipStream_t s, long long lo_off, float split_scale, int* range_flag) {
  const long long n = (long long)Mpad * 2 * cin;
  if (slab && cin % 32) return hipErrorInvalidValue;
  if (lo_off < 0 || (lo_off > 0 && (!half_out || !range_flag))) return hipErrorInvalidValue;
  if (half_out)
    hipLaunchKernelGGL(repack_convT_kernel<_Float16>, dim3(cdiv(n, 256)), dim3(256), 0, s, src, (_Float16*)dst, cin,
                       cout, stride, Mpad, slab ? 1 : 0, lo_off, split_scale, range_flag);
  else
    hipLaunchKernelGGL(repack_convT_kernel<float>, dim3(cdiv(n, 256)), dim3(256), 0, s, src, (float*)dst, cin, cout,
                       stride, Mpad, slab ? 1 : 0, 0LL, 1.f, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* src, long long rows, int K, void* q, void* scale, hipStream_t s) {
  if (K <= 0 || K % 32 != 0 || rows < 0) return hipErrorInvalidValue;
  const long long groups = rows * (K / 32);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)cdiv(groups, 256)), dim3(256), 0, s, src, groups,
                     (int8_t*)q, (_Float16*)scale);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const void* q, const void* scale, long long values, void* dst, bool half,
                               hipStream_t s) {
  if (values <= 0) return hipSuccess;
  if (values % 32) return hipErrorInvalidValue;
  const long long units = values / 8;
  hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)cdiv(units, 256)), dim3(256), 0, s, (const int8_t*)q,
                     (const _Float16*)scale, units, dst, half ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_expand_vec(const float* src, float* dst, int C, int phases, int Mpad, hipStream_t s) {
  hipLaunchKernelGGL(expand_vec_kernel, dim3(cdiv(Mpad, 256)), dim3(256), 0, s, src, dst, C, phases, Mpad);
  return hipGetLastError();
}

hipError_t launch_fill(void* dst, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 65536);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)dst, words);
  return hipGetLastError();
}

hipError_t launch_copy(float* dst, const float* src, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15)) return hipErrorInvalidValue;
  const long long n4 = n / 4;
  const unsigned blocks = (unsigned)std::min<long long>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<f32x4*>(dst),
                     reinterpret_cast<const f32x4*>(src), n4);
  return hipGetLastError();
}

hipError_t launch_reset_headers(void* state, long long sstride, int batch, uint64_t cfg_hash, hipStream_t s) {
  hipLaunchKernelGGL(reset_headers_kernel, dim3(cdiv(batch, 256)), dim3(256), 0, s, (float*)state, sstride, batch,
                     cfg_hash);
  return hipGetLastError();
}

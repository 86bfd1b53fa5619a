// Shared device-side definitions of the code2wav decoder library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// LayerNorm over d channels of one row by one block of 64 * NV threads
// (NV = layernorm_nv(d)): thread t holds channels 4t..4t+3 (t < d/4).  Biased
// variance, two passes; each pass sums the per-thread partials of lane l in
// thread order l, l + 64, ... in wave 0, then across the wave.  Optionally
// the last H rows of each stream (T rows per stream) also go to a state slot.
// Shared by the LayerNorm kernel and the split-K fold that feeds one, so both
// give the same bits.
struct LnArgs {
  const float* g;
  const float* b;
  float eps;
  int d;
  float* out;
  int T;
  float* hist;
  int H;
  long long sstride;
};

// Widest row: 64 x LN_MAX_NV float4 (one thread each).
#define LN_MAX_NV 16

// red: LDS of at least 64 * NV + 1 floats.  Every thread of the block calls it.
template <int NV>
__device__ __forceinline__ void layernorm_block(const LnArgs& a, f32x4 x, int row, float* red) {
  const int t = threadIdx.x, lane = t & 63;
  const int d4 = a.d / 4;
  const bool have = t < d4;
  if (have) red[t] = (x.x + x.y) + (x.z + x.w);
  __syncthreads();
  if (t < 64) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (64 * i + lane < d4) s += red[64 * i + lane];
    s = wave_sum(s);
    if (t == 0) red[64 * NV] = s / (float)a.d;
  }
  __syncthreads();
  const float mean = red[64 * NV];
  const f32x4 v = x - mean;
  if (have) red[t] = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  __syncthreads();
  if (t < 64) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (64 * i + lane < d4) q += red[64 * i + lane];
    q = wave_sum(q);
    if (t == 0) red[64 * NV] = 1.0f / sqrtf(q / (float)a.d + a.eps);
  }
  __syncthreads();
  const float rstd = red[64 * NV];
  if (!have) return;
  const int b = row / a.T, tt = row - b * a.T;
  const f32x4 y = v * rstd * *reinterpret_cast<const f32x4*>(a.g + 4 * t) + *reinterpret_cast<const f32x4*>(a.b + 4 * t);
  *reinterpret_cast<f32x4*>(a.out + (size_t)row * a.d + 4 * t) = y;
  if (a.hist && tt >= a.T - a.H)
    *reinterpret_cast<f32x4*>(a.hist + (size_t)b * a.sstride + (size_t)(a.H - a.T + tt) * a.d + 4 * t) = y;
}

// ---------------------------------------------------------------------------
// implicit-GEMM convolution (conv1d, transposed conv, linear)
// ---------------------------------------------------------------------------
//
// out[g][m] = epi( sum_{tap, c} W[m][tap][c] * X[g - (k-1-tap)*dil][c] )
// GEMM rows g run over (stream, row) pairs, channels-last.  Rows before the
// start of a stream's chunk come from that stream's history slot in state_in.

struct EpiOut {
  float* dst;           // [rows_out][cout] or nullptr
  const float* alpha;   // Snake alpha per GEMM column, nullptr = no Snake
  float* hist;          // state_out slot of stream 0 ([H][cout]) or nullptr
  int H;                // slot rows
  int src;              // 0: the conv value v, 1: the multi-receptive-field value s
  int half;             // store dst as fp16 (a tensor read only as an fp16 GEMM operand)
};

enum { MRF_NONE = 0, MRF_FIRST = 1, MRF_ACCUM = 2, MRF_LAST = 3, MRF_ONLY = 4 };
enum { ACT_NONE = 0, ACT_GELU = 1 };

struct ConvParams {
  const float* w;       // packed [Mpad][k][cin] (fp32, fp16, or int8 when wscale is set)
  const void* wscale;   // int8 weights: fp16 scales [Mpad][k*cin/32], else nullptr
  const void* w_lo;     // split fp16 weights: the lo plane (w holds the hi plane), else nullptr
  float acc_scale;      // power of two applied to the reduced sum before the bias (1 unless split)
  int M;                // GEMM columns (= phases * cout)
  int k, cin, dil;
  const float* x;       // [rows][cin], fp32 or (x_half) fp16
  int x_half;           // x holds fp16 values (fp16-operand kernel only); history rows stay fp32
  const float* hin;     // state_in slot of stream 0 ([hin_rows][cin])
  long long sstride;    // state floats per stream
  int hin_rows;         // (k-1)*dil history rows
  int rows;             // GEMM rows = batch * nin
  int nin;              // GEMM rows per stream
  // epilogue
  const float* bias;    // [M]
  int act;
  const float* resid;   // [rows_out][cout] or nullptr
  int phases, cout;     // output row = g*phases + m/cout, channel = m % cout
  int mrf_mode;
  float mrf_div;        // divisor of the MRF mean
  float* mrf;           // running MRF sum [rows_out][cout] (read in ACCUM/LAST)
  const float* mrf2;    // LAST only, or nullptr: a second block's output, added after mrf
  int nout;
  EpiOut out[4];
  // split-K: splits > 1 stores per-group partials to `partial`
  // ([ceil(k*cin/256)][rows][M] floats), folded by a second kernel
  int splits;
  float* partial;
};

// reduction values per split-K group (and per accumulation group)
#define VOC_GROUP_K 256
// chunks of at most this many frames (over the batch) run a stage's AMP
// blocks concurrently
#define VOC_CONC_FRAMES 64

// ---------------------------------------------------------------------------
// state layout
// ---------------------------------------------------------------------------

#define VOC_STATE_MAGIC 0x56434453u  // "SDCV"
#define VOC_STATE_VERSION 1u
#define VOC_STATE_HEADER_FLOATS 64   // 256 bytes

struct StateHeader {
  uint32_t magic;
  uint32_t version;
  uint64_t cfg_hash;
  int64_t pos;        // frames decoded since reset
  int64_t reserved[5];
};

// A state slot: the last H rows (oldest first) of a tensor with C channels,
// which gains `rate` rows per frame.
struct Slot {
  long long off;   // float offset inside one stream's state
  long long cap;   // floats reserved for the slot (H*C rounded up to 64)
  int H;
  int C;
  int rate;
  int pad;
};

// status bits in the workspace status word
#define VOC_STATUS_CODE 1
#define VOC_STATUS_STATE 2

// ---------------------------------------------------------------------------
// launchers (defined in conv_gemm.hip / kernels.hip)
// ---------------------------------------------------------------------------

// tile configuration ids for the implicit-GEMM kernel
// TILE_S64x16 / TILE_S64x32: skinny tiles for launches of a few rows (small
// chunks), 128-deep K-steps so that few load round trips cover a group.
enum GemmTile { TILE_128x128 = 0, TILE_64x64 = 1, TILE_96x128 = 2, TILE_S64x16 = 3, TILE_S64x32 = 4, TILE_COUNT = 5 };
int gemm_tile_bm(int tile);
int gemm_tile_bn(int tile);
int gemm_tile_bk(int tile, int cin, bool half);
// the fp16-operand GEMM of this tile loads its operands straight into LDS
// (float or fp16 weights, channel count a multiple of 32, 128x128 or 96x128)
bool gemm_f16_direct(bool int8, int cin, int tile);
// ... and stages each 32-channel slab's input rows once for all its taps
// (fp16 rows, k >= 3, unsplit, history in the state; p.splits already set)
bool gemm_f16_window(const ConvParams& p, int tile);
// ln: for a split launch (p.splits > 1) whose first output (fp32, one phase,
// M = ln.d) feeds a LayerNorm, fold the partials, run the epilogue and
// normalise each row in one kernel (the same bits as the reduction followed
// by the LayerNorm kernel); null otherwise.
hipError_t launch_conv_gemm(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln = nullptr);
// Few-row fp32 GEMM (at most 16 GEMM rows, cin a multiple of 16, float or
// int8 weights): whether a launch fits it.
bool conv_gemm_rows_ok(const ConvParams& p);
hipError_t launch_conv_gemm_rows(const ConvParams& p, hipStream_t s);
// fp16-operand GEMM: p.w points at fp16 weights [Mpad][k][cin]; tiles 128x128, 96x128, 64x64
hipError_t launch_conv_gemm_f16(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln = nullptr);
// split-fp16 GEMM (fp32 accuracy from three fp16 products per pair): p.w and
// p.w_lo are the hi and lo planes of fp16 weights in 32-channel slab order,
// p.x fp32 rows; cin a multiple of 32, tiles 128x128, 96x128, 64x64, 64x32, 64x16
hipError_t launch_conv_gemm_split(const ConvParams& p, int tile, hipStream_t s, const LnArgs* ln = nullptr);

// The two-term fp16 split of an fp32 value: hi = fp16(v), lo = fp16(v - hi),
// both rounded to nearest even (v - hi is exact in fp32).
__device__ __forceinline__ _Float16 split_lo(float v, _Float16 hi) { return (_Float16)(v - (float)hi); }

hipError_t launch_begin(const void* state_in, void* state_out, long long sstride, int batch, int T,
                        uint64_t cfg_hash, const double* inv_freq, int half, float* rope_tab, int* pos,
                        int* status, hipStream_t s);
hipError_t launch_state_shift(const Slot* slots, int nslots, int max_h, const float* state_in,
                              float* state_out, long long sstride, int batch, int T, hipStream_t s);
hipError_t launch_gather(const int32_t* codes, const float* codebooks, int Q, int V, int D, int rows,
                         int T, float* out, float* hist, int H, long long sstride, int* status,
                         hipStream_t s);
// waves per LayerNorm row of d channels (a power of two, one float4 per
// thread), 0 if d is not a multiple of 4 or wider than 64 x LN_MAX_NV float4
int layernorm_nv(int d);
hipError_t launch_layernorm(const float* x, const float* g, const float* b, float eps, int rows, int d,
                            float* out, int T, float* hist, int H, long long sstride, hipStream_t s);
// Windowed attention of the new frames; RoPE is applied to their q and k as
// they are staged, and their rotated keys and values (the last W frames of
// each stream) go to k_state_out / v_state_out.
hipError_t launch_attention(const float* qkv, const float* k_state, const float* v_state, long long sstride,
                            const int* pos, int batch, int T, int n_heads, int hd, int W, const float* rope_tab,
                            float* k_state_out, float* v_state_out, float* out, hipStream_t s);
hipError_t launch_conv_post(const float* x, const float* hin, long long sstride, int H, const float* w,
                            const float* bias, int C, int k, int rows, int nin, float* pcm,
                            float* pre_tanh, hipStream_t s);
// Weight repacking into GEMM rows [Mpad][k * cin]: tap-major ([k][cin]) or,
// with slab (cin a multiple of 32; the fp16 GEMMs), [cin / 32][k][32].
// lo_off > 0 (fp16 output only): split each value times split_scale (a
// power of two) into hi and lo halves, the lo half lo_off elements after its
// hi half, and set *range_flag to 1 if a scaled value's hi half is not finite.
hipError_t launch_repack_conv(const float* src, void* dst, int M, int Mpad, int cin, int k, bool half_out,
                              bool slab, hipStream_t s, long long lo_off = 0, float split_scale = 1.f,
                              int* range_flag = nullptr);
hipError_t launch_repack_convT(const float* src, void* dst, int cin, int cout, int stride, int Mpad,
                               bool half_out, bool slab, hipStream_t s, long long lo_off = 0,
                               float split_scale = 1.f, int* range_flag = nullptr);
hipError_t launch_expand_vec(const float* src, float* dst, int C, int phases, int Mpad, hipStream_t s);
// int8 with one fp16 scale per 32 values of each row of a [rows][K] fp32 matrix
hipError_t launch_quantize_rows(const float* src, long long rows, int K, void* q, void* scale, hipStream_t s);
// int8 values q (groups of 32 with one fp16 scale each, values % 32 == 0) to
// fp32, or fp16 when half: q * scale, as the int8 GEMM kernels dequantize
hipError_t launch_dequant_rows(const void* q, const void* scale, long long values, void* dst, bool half,
                               hipStream_t s);
hipError_t launch_fill(void* dst, size_t bytes, hipStream_t s);
// dst[i] = src[i] for i < n floats (n a multiple of 4, both 16-byte aligned)
hipError_t launch_copy(float* dst, const float* src, long long n, hipStream_t s);
hipError_t launch_reset_headers(void* state, long long sstride, int batch, uint64_t cfg_hash,
                                hipStream_t s);

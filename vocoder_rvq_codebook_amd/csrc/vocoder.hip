// Host side of the code2wav decoder library: config checks, the packed-weight,
// state and workspace layouts, create / reset / decode_chunk.
//
// The decoder ("Edge TTS design (vLLM-Omni-compatible)", section 1.3): RVQ
// embedding sum -> causal conv -> sliding-window transformer -> 2x2 transposed
// conv upsampling -> BigVGAN Snake/AMP stack -> tanh, with the conv context and
// the attention window carried across chunks as explicit state (sections 2.2,
// 2.3 and the ExecuTorch note of section 4).

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "vocoder.h"  // include/, on the compiler include path
#include "common.h"

namespace {

constexpr long long ALIGN = 64;  // floats (256 bytes)
inline long long align_up(long long x, long long a = ALIGN) { return (x + a - 1) / a * a; }
inline int round_up_i(int x, int a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// config
// ---------------------------------------------------------------------------

bool config_valid(const vocoder_config* c) {
  if (!c) return false;
  auto m16 = [](int v) { return v > 0 && v % 16 == 0; };
  if (c->n_codebooks < 1 || c->n_codebooks > 64 || c->codebook_size < 1) return false;
  if (!m16(c->embed_dim) || !m16(c->model_dim) || !m16(c->ffn_dim)) return false;
  if (c->n_layers < 0 || c->n_layers > 64 || c->n_heads < 1 || c->model_dim % c->n_heads) return false;
  const int hd = c->model_dim / c->n_heads;
  if (hd % 8 || hd > 256) return false;  // rotate-half pairs of 16-byte pieces
  if (c->model_dim > 4096) return false;  // a LayerNorm row is held in one wave's registers
  if (c->window < 0 || c->window > 255) return false;
  // the attention kernel stages (16 + window) keys and values plus 16 queries in 64 KB of LDS
  if ((16LL + c->window) * (2LL * hd + 1) + 16LL * hd > 16384) return false;
  if (!(c->ln_eps > 0.f) || !(c->rope_theta > 0.f)) return false;
  if (c->pre_kernel < 1 || c->pre_kernel > 64) return false;
  if (c->n_up < 0 || c->n_up > VOCODER_MAX_UP) return false;
  for (int i = 0; i < c->n_up; ++i)
    if (c->up_strides[i] < 1 || c->up_strides[i] > 64) return false;
  if (c->n_stages < 1 || c->n_stages > VOCODER_MAX_STAGES) return false;
  if (c->voc_ch0 <= 0 || c->voc_ch0 % (16 << c->n_stages)) return false;
  if (c->conv_pre_kernel < 1 || c->conv_pre_kernel > 64) return false;
  for (int s = 0; s < c->n_stages; ++s)
    if (c->rates[s] < 1 || c->rates[s] > 64) return false;
  if (c->n_res < 1 || c->n_res > VOCODER_MAX_RES || c->n_dil < 1 || c->n_dil > VOCODER_MAX_DIL) return false;
  for (int j = 0; j < c->n_res; ++j)
    if (c->res_kernels[j] < 1 || c->res_kernels[j] > 64) return false;
  for (int i = 0; i < c->n_dil; ++i)
    if (c->dilations[i] < 1 || c->dilations[i] > 64) return false;
  if (c->post_kernel < 1 || c->post_kernel > 64) return false;
  {
    // the final conv stages 128 + post_kernel - 1 rows of the last stage's channels in 64 KB of LDS
    const long long cl = c->voc_ch0 >> c->n_stages;
    if ((long long)c->post_kernel * cl + (128LL + c->post_kernel - 1) * (cl + 1) > 16384) return false;
  }
  if (c->max_batch < 1 || c->max_frames < 1) return false;
  if (c->precision != VOCODER_PRECISION_F32 && c->precision != VOCODER_PRECISION_F16 &&
      c->precision != VOCODER_PRECISION_SPLIT16)
    return false;
  if (c->weight_format != VOCODER_WEIGHTS_FLOAT && c->weight_format != VOCODER_WEIGHTS_INT8) return false;
  if (c->precision == VOCODER_PRECISION_SPLIT16 && c->weight_format != VOCODER_WEIGHTS_FLOAT) return false;
  // every GEMM row count must fit in int
  long long hop = 1;
  for (int i = 0; i < c->n_up; ++i) hop *= c->up_strides[i];
  for (int s = 0; s < c->n_stages; ++s) hop *= c->rates[s];
  if (hop > (1 << 20)) return false;
  if ((long long)c->max_batch * c->max_frames * hop >= (1LL << 31) / 4) return false;
  return true;
}

uint64_t config_hash(const vocoder_config* c) {
  // FNV-1a over the model fields (max_batch / max_frames excluded: they size
  // the workspace, not the state)
  vocoder_config k = *c;
  k.max_batch = 0;
  k.max_frames = 0;
  const unsigned char* b = reinterpret_cast<const unsigned char*>(&k);
  uint64_t h = 1469598103934665603ULL;
  for (size_t i = 0; i < sizeof(k); ++i) {
    h ^= b[i];
    h *= 1099511628211ULL;
  }
  return h;
}

int hop_of(const vocoder_config& c) {
  int h = 1;
  for (int i = 0; i < c.n_up; ++i) h *= c.up_strides[i];
  for (int s = 0; s < c.n_stages; ++s) h *= c.rates[s];
  return h;
}

// ---------------------------------------------------------------------------
// layout plan (shared by size queries and create)
// ---------------------------------------------------------------------------

struct GemmW {
  long long w = -1, bias = -1;  // packed float offsets
  long long scale = -1;         // int8 weights: fp16 scales (packed float offset)
  long long raw_w = -1, raw_b = -1;
  int M = 0, Mpad = 0, k = 1, cin = 0, phases = 1, cout = 0;
  bool q8 = false;              // weights stored as int8 with one fp16 scale per 32
  bool split = false;           // split fp16: hi plane, then lo plane, in 32-channel slab order
  long long lo_halves() const { return (long long)Mpad * k * cin; }  // hi plane -> lo plane
};

// Split fp16: the weights are scaled by 2^SPLIT_W_EXP before their split (a
// power of two: exact) and the sum scaled back before the bias.  Unscaled, the
// lo half of a weight below 2^-3 is an fp16 subnormal (spacing 2^-24), which
// for weights of typical size (~0.02) costs about 2^-19 of their value and
// made the decoder's error 4x the fp32 path's; scaled, lo halves stay normal
// down to 2^-11, and weights up to 2^8 keep their hi half finite.
constexpr int SPLIT_W_EXP = 8;

// Tensors of at least this many values whose input channel count is a
// multiple of 32 are stored as int8 ("blixt/phonon", section Weights).
constexpr long long INT8_MIN_VALUES = 16384;

struct LayerP {
  long long ln1_g, ln1_b, ln2_g, ln2_b;         // packed
  long long raw_ln1_g, raw_ln1_b, raw_ln2_g, raw_ln2_b;
  long long raw_q_w, raw_q_b, raw_k_w, raw_k_b, raw_v_w, raw_v_b;
  GemmW qkv, o, fc1, fc2;
  int slot_k, slot_v;
};

struct AmpP {
  GemmW conv1, conv2;
  long long act1 = -1, act2 = -1;          // packed alpha [C]
  long long raw_act1 = -1, raw_act2 = -1;
  int slot1 = -1, slot2 = -1;              // conv1 / conv2 input slots
};

struct StageP {
  GemmW up;                                // transposed conv, M = r * C
  std::vector<long long> up_alpha;         // expanded act1 alpha of dilation 0, per AMP block
  int slot_up = -1;                        // ConvT input slot (1 row)
  std::vector<AmpP> amp;                   // [n_res * n_dil]
  int cin = 0, c = 0, r = 1;
  long long rate = 1;                      // rows per frame at the output
};

// Float offsets of the per-call buffers inside a workspace laid out for
// `rows` = batch x frames frame-rows (layout_workspace).
struct WsLayout {
  long long status = 0, pos = 0, rope = 0, emb = 0, h = 0, u = 0, qkv = 0, att = 0, ffn = 0;
  long long up[VOCODER_MAX_UP] = {0, 0, 0, 0};
  long long X0 = 0, T = 0, Xr = 0, An = 0, S[2] = {0, 0};
  long long A[VOCODER_MAX_RES] = {0, 0, 0, 0};
  long long partial = 0, partial_floats = 0;  // split-K group partials
  // concurrent AMP blocks (chunks of at most conc_frames frames over the
  // batch): per extra block its own inner buffers and split-K partials, and
  // the middle block's output
  long long conc_frames = 0;
  long long conc_T[2] = {0, 0}, conc_Xr[2] = {0, 0}, conc_An[2] = {0, 0}, conc_B1 = 0;
  long long partial_aux[2] = {0, 0}, partial_aux_floats = 0;
  long long wdeq = 0;   // an int8 layer expanded to the GEMM operand type (0: none, dequantize per tile)
  long long snap = 0;   // a batch of states: the input of an in-place decode
  long long floats = 0;
};

struct Plan {
  vocoder_config cfg{};
  int d = 0, hd = 0, half = 0, hop = 0;
  bool f16 = false;    // fp16 GEMM operands (packed weights in fp16)
  bool split = false;  // split-fp16 GEMMs (fp32 values; weights as fp16 hi + lo planes)
  long long max_gemm_values = 0;  // largest packed GEMM weight (values)
  long long max_q8_values = 0;    // largest int8 GEMM weight (values)
  long long ws_wdeq = 0;          // an int8 layer expanded to the GEMM operand type
  long long raw_count = 0;
  // packed
  long long raw_codebooks = 0, codebooks = 0;
  GemmW pre;
  int slot_pre = -1;
  std::vector<LayerP> layers;
  long long raw_fln_g = 0, raw_fln_b = 0, fln_g = 0, fln_b = 0;
  std::vector<GemmW> ups;
  std::vector<int> slot_ups;               // input slot of each up
  GemmW conv_pre;
  int slot_conv_pre = -1;
  std::vector<StageP> stages;
  long long raw_post_alpha = 0, post_alpha = 0, raw_post_w = 0, raw_post_b = 0, post_w = 0, post_b = 0;
  int slot_post = -1;
  long long inv_freq = 0;                  // packed doubles (offset in floats)
  long long slots_off = 0;                 // packed Slot table (offset in floats)
  long long packed_floats = 0;
  // state
  std::vector<Slot> slots;
  long long state_floats = 0;
  // workspace layout of the handle (max_batch x max_frames) and its size,
  // which also covers the float repack staged there by an int8 create
  WsLayout ws;
  long long ws_floats = 0;
  // largest split-K partial of any GEMM per frame-row of a chunk: groups x
  // (GEMM rows per frame) x M
  long long partial_per_row = 0;
  // frames at the end of a chunk that determine every carried row after the
  // transformer (prefill decodes only these through the upsampling stack)
  int tail_frames = 0;
};

int add_slot(Plan& P, int H, int C, long long rate) {
  Slot s{};
  s.off = P.state_floats;
  s.H = H;
  s.C = C;
  s.rate = (int)rate;
  s.cap = align_up((long long)H * C);
  P.slots.push_back(s);
  P.state_floats += align_up((long long)H * C);
  return (int)P.slots.size() - 1;
}

// Lay out the per-call buffers of decodes of up to `batch` streams x `frames`
// frames.  compact: the layout of the static scratch of the no-allocation
// entry point -- split-K partial room in proportion to the rows (launches
// whose partials do not fit are not split: the same bits) and no room for an
// expanded int8 layer (int8 weights are dequantized per tile: the same bits);
// otherwise the handle's workspace layout.  Needs P's layers and stages.
void layout_workspace(const Plan& P, long long batch, long long frames, bool compact, WsLayout& L) {
  const vocoder_config& c = P.cfg;
  const int d = P.d, De = c.embed_dim, F = c.ffn_dim;
  const long long Rr = batch * frames;
  L = WsLayout{};
  long long ws = 0;
  auto Wk = [&](long long n) { long long o = ws; ws += align_up(n); return o; };
  L.status = Wk(64);
  L.pos = Wk(batch);
  L.rope = Wk(Rr * std::max(P.half, 1) * 2);
  L.emb = Wk(Rr * De);
  L.h = Wk(Rr * d);
  L.u = Wk(Rr * d);
  L.qkv = Wk(Rr * 3 * d);
  L.att = Wk(Rr * d);
  L.ffn = Wk(Rr * F);
  long long ur = 1;
  for (int i = 0; i < c.n_up; ++i) {
    ur *= c.up_strides[i];
    L.up[i] = Wk(Rr * ur * d);
  }
  long long big = Rr * ur * c.voc_ch0;  // conv_pre output
  for (const StageP& S : P.stages) big = std::max(big, Rr * S.rate * S.c);
  L.X0 = Wk(big);
  for (int j = 0; j < c.n_res; ++j) L.A[j] = Wk(big);
  L.T = Wk(big);
  L.Xr = Wk(big);
  L.An = Wk(big);
  L.S[0] = Wk(big);
  L.S[1] = Wk(big);
  // split-K partials: used only by launches with few output tiles, which are
  // small; 32 M floats (128 MB) bounds the split factor of the rest
  L.partial_floats = compact ? std::min<long long>(32LL << 20, Rr * P.partial_per_row) : 32LL << 20;
  L.partial = Wk(L.partial_floats);
  if (c.n_res >= 2 && c.n_res <= 3) {
    L.conc_frames = std::min<long long>(Rr, VOC_CONC_FRAMES);
    long long bigc = 0;
    for (const StageP& S : P.stages) bigc = std::max(bigc, L.conc_frames * S.rate * S.c);
    for (int j = 0; j < 2; ++j) {
      L.conc_T[j] = Wk(bigc);
      L.conc_Xr[j] = Wk(bigc);
      L.conc_An[j] = Wk(bigc);
    }
    L.conc_B1 = Wk(bigc);
    L.partial_aux_floats = compact ? std::min<long long>(8LL << 20, Rr * P.partial_per_row) : 8LL << 20;
    for (int j = 0; j < 2; ++j) L.partial_aux[j] = Wk(L.partial_aux_floats);
  }
  if (P.max_q8_values > 0 && !compact) L.wdeq = Wk(P.f16 ? (P.max_q8_values + 1) / 2 : P.max_q8_values);
  L.snap = Wk(batch * P.state_floats);
  L.floats = ws;
}

bool make_plan(const vocoder_config* cp, Plan& P) {
  if (!config_valid(cp)) return false;
  const vocoder_config& c = *cp;
  P.cfg = c;
  P.d = c.model_dim;
  P.hd = c.model_dim / c.n_heads;
  P.half = P.hd / 2;
  P.hop = hop_of(c);
  P.f16 = c.precision == VOCODER_PRECISION_F16;
  P.split = c.precision == VOCODER_PRECISION_SPLIT16;
  const int d = P.d, De = c.embed_dim, F = c.ffn_dim;

  long long raw = 0, pk = 0;
  auto R = [&](long long n) { long long o = raw; raw += n; return o; };
  auto K = [&](long long n) { long long o = pk; pk += align_up(n); return o; };
  // tensor_values: values of the source tensor (one of q, k, v for the stacked
  // projection), which decides int8 storage
  auto gemm = [&](GemmW& g, int M, int k, int cin, int phases, int cout, long long tensor_values) {
    g.M = M;
    g.Mpad = round_up_i(M, 128);
    g.k = k;
    g.cin = cin;
    g.phases = phases;
    g.cout = cout;
    const long long welems = (long long)g.Mpad * k * cin;
    g.q8 = c.weight_format == VOCODER_WEIGHTS_INT8 && tensor_values >= INT8_MIN_VALUES && cin % 32 == 0;
    if (g.q8) {
      g.w = K((welems + 3) / 4);          // int8 values
      g.scale = K((welems / 32 + 1) / 2);  // fp16 scales, one per 32 values
    } else {
      // fp16 weights take half the floats; split weights two fp16 planes
      g.split = P.split && cin % 32 == 0;
      g.w = K(P.f16 ? (welems + 1) / 2 : welems);
    }
    g.bias = K(g.Mpad);
    P.max_gemm_values = std::max(P.max_gemm_values, welems);
    if (g.q8) P.max_q8_values = std::max(P.max_q8_values, welems);
  };

  P.state_floats = VOC_STATE_HEADER_FLOATS;

  // codebooks and pre-conv
  P.raw_codebooks = R((long long)c.n_codebooks * c.codebook_size * De);
  P.codebooks = K((long long)c.n_codebooks * c.codebook_size * De);
  gemm(P.pre, d, c.pre_kernel, De, 1, d, (long long)d * De * c.pre_kernel);
  P.pre.raw_w = R((long long)d * De * c.pre_kernel);
  P.pre.raw_b = R(d);
  P.slot_pre = add_slot(P, c.pre_kernel - 1, De, 1);

  // transformer
  P.layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    LayerP& L = P.layers[l];
    L.raw_ln1_g = R(d); L.raw_ln1_b = R(d);
    L.raw_q_w = R((long long)d * d); L.raw_q_b = R(d);
    L.raw_k_w = R((long long)d * d); L.raw_k_b = R(d);
    L.raw_v_w = R((long long)d * d); L.raw_v_b = R(d);
    gemm(L.o, d, 1, d, 1, d, (long long)d * d);
    L.o.raw_w = R((long long)d * d); L.o.raw_b = R(d);
    L.raw_ln2_g = R(d); L.raw_ln2_b = R(d);
    gemm(L.fc1, F, 1, d, 1, F, (long long)F * d);
    L.fc1.raw_w = R((long long)F * d); L.fc1.raw_b = R(F);
    gemm(L.fc2, d, 1, F, 1, d, (long long)d * F);
    L.fc2.raw_w = R((long long)d * F); L.fc2.raw_b = R(d);
    gemm(L.qkv, 3 * d, 1, d, 1, 3 * d, (long long)d * d);
    L.ln1_g = K(d); L.ln1_b = K(d); L.ln2_g = K(d); L.ln2_b = K(d);
    L.slot_k = add_slot(P, c.window, d, 1);
    L.slot_v = add_slot(P, c.window, d, 1);
  }
  P.raw_fln_g = R(d);
  P.raw_fln_b = R(d);
  P.fln_g = K(d);
  P.fln_b = K(d);

  // 2x2 upsampling
  long long rate = 1;
  P.ups.resize(c.n_up);
  for (int i = 0; i < c.n_up; ++i) {
    const int s = c.up_strides[i];
    gemm(P.ups[i], s * d, 2, d, s, d, (long long)d * d * 2 * s);
    P.ups[i].raw_w = R((long long)d * d * 2 * s);
    P.ups[i].raw_b = R(d);
    P.slot_ups.push_back(add_slot(P, 1, d, rate));
    rate *= s;
  }
  // conv_pre
  const int C0 = c.voc_ch0;
  gemm(P.conv_pre, C0, c.conv_pre_kernel, d, 1, C0, (long long)C0 * d * c.conv_pre_kernel);
  P.conv_pre.raw_w = R((long long)C0 * d * c.conv_pre_kernel);
  P.conv_pre.raw_b = R(C0);
  P.slot_conv_pre = add_slot(P, c.conv_pre_kernel - 1, d, rate);

  // BigVGAN stages
  P.stages.resize(c.n_stages);
  int cin = C0;
  for (int si = 0; si < c.n_stages; ++si) {
    StageP& S = P.stages[si];
    const int r = c.rates[si], co = cin / 2;
    S.cin = cin;
    S.c = co;
    S.r = r;
    gemm(S.up, r * co, 2, cin, r, co, (long long)cin * co * 2 * r);
    S.up.raw_w = R((long long)cin * co * 2 * r);
    S.up.raw_b = R(co);
    S.slot_up = add_slot(P, 1, cin, rate);
    rate *= r;
    S.rate = rate;
    S.amp.resize((size_t)c.n_res * c.n_dil);
    for (int j = 0; j < c.n_res; ++j) {
      const int k = c.res_kernels[j];
      for (int i = 0; i < c.n_dil; ++i) {
        AmpP& A = S.amp[(size_t)j * c.n_dil + i];
        A.raw_act1 = R(co);
        gemm(A.conv1, co, k, co, 1, co, (long long)co * co * k);
        A.conv1.raw_w = R((long long)co * co * k);
        A.conv1.raw_b = R(co);
        A.raw_act2 = R(co);
        gemm(A.conv2, co, k, co, 1, co, (long long)co * co * k);
        A.conv2.raw_w = R((long long)co * co * k);
        A.conv2.raw_b = R(co);
        A.act1 = K(co);
        A.act2 = K(co);
        A.slot1 = add_slot(P, (k - 1) * c.dilations[i], co, rate);
        A.slot2 = add_slot(P, k - 1, co, rate);
      }
    }
    for (int j = 0; j < c.n_res; ++j) S.up_alpha.push_back(K(S.up.Mpad));
    cin = co;
  }
  P.raw_post_alpha = R(cin);
  P.raw_post_w = R((long long)cin * c.post_kernel);
  P.raw_post_b = R(1);
  P.post_alpha = K(cin);
  P.post_w = K((long long)cin * c.post_kernel);
  P.post_b = K(4);
  P.slot_post = add_slot(P, c.post_kernel - 1, cin, rate);

  P.inv_freq = K(2LL * std::max(P.half, 1));
  P.slots_off = K((long long)(sizeof(Slot) / 4) * (long long)P.slots.size());
  P.raw_count = raw;
  P.packed_floats = pk;

  {
    auto need = [&](const GemmW& g, long long rows_per_frame) {
      const long long ngroups = ((long long)g.k * g.cin + VOC_GROUP_K - 1) / VOC_GROUP_K;
      P.partial_per_row = std::max(P.partial_per_row, ngroups * rows_per_frame * g.M);
    };
    need(P.pre, 1);
    for (const LayerP& L : P.layers) {
      need(L.qkv, 1); need(L.o, 1); need(L.fc1, 1); need(L.fc2, 1);
    }
    long long r = 1;
    for (int i = 0; i < c.n_up; ++i) {
      need(P.ups[i], r);
      r *= c.up_strides[i];
    }
    need(P.conv_pre, r);
    for (const StageP& S : P.stages) {
      need(S.up, S.rate / S.r);
      for (const AmpP& A : S.amp) {
        need(A.conv1, S.rate);
        need(A.conv2, S.rate);
      }
    }
  }
  // workspace, sized for max_batch x max_frames
  layout_workspace(P, c.max_batch, c.max_frames, false, P.ws);
  P.ws_floats = P.ws.floats;
  // int8 weights are quantized at create time from a float repack staged in
  // the workspace
  if (c.weight_format == VOCODER_WEIGHTS_INT8) P.ws_floats = std::max(P.ws_floats, align_up(P.max_gemm_values));
  {
    // Walk back from conv_post's carried rows: a causal conv of kernel k and
    // dilation d reaches (k-1)*d input rows further back, an AMP block the sum
    // over its dilations of both convs, a stage's blocks the longest of them;
    // m trailing output rows of a transposed conv of stride s need the last
    // ceil(m/s)+1 input rows.  The count at the transformer output, in frames,
    // covers every carried row of the stack.
    long long need = c.post_kernel - 1;
    for (int si = c.n_stages - 1; si >= 0; --si) {
      long long look = 0;
      for (int j = 0; j < c.n_res; ++j) {
        long long lj = 0;
        for (int i = 0; i < c.n_dil; ++i) lj += (long long)(c.res_kernels[j] - 1) * (c.dilations[i] + 1);
        look = std::max(look, lj);
      }
      need += look;
      need = (need + c.rates[si] - 1) / c.rates[si] + 1;
    }
    need += c.conv_pre_kernel - 1;
    for (int i = c.n_up - 1; i >= 0; --i) need = (need + c.up_strides[i] - 1) / c.up_strides[i] + 1;
    P.tail_frames = (int)std::min<long long>(need, 1 << 30);
  }
  return true;
}

}  // namespace

// ---------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------

struct GraphKey {
  const void* codes;
  const void* state_in;
  const void* state_out;
  const void* pcm;
  int batch, frames;
  bool operator==(const GraphKey& o) const {
    return codes == o.codes && state_in == o.state_in && state_out == o.state_out && pcm == o.pcm &&
           batch == o.batch && frames == o.frames;
  }
};

struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec;
  uint64_t last_use;
};

struct vocoder {
  Plan P;
  uint64_t hash = 0;
  float* packed = nullptr;
  float* ws = nullptr;
  std::map<std::string, std::pair<float*, size_t>> taps;
  // measurement: event pairs around each launch while profiling is on
  struct Rec {
    int name;
    double flops, bytes;
  };
  bool prof = false;
  bool no_events = false;  // a no-allocation call: no profiling events
  float* scratch = nullptr;  // device address of the static scratch on the handle's device (or null)
  std::vector<hipEvent_t> events;
  std::vector<Rec> recs;
  std::vector<std::string> prof_names;
  // decode graphs, one per (buffers, batch, frames), least recently used evicted
  std::vector<GraphEntry> graphs;
  uint64_t graph_clock = 0;
  hipStream_t capture_stream = nullptr;
  bool capturing = false;  // recording a graph: no profiling events, no taps
  // side streams (default priority) for concurrent AMP blocks, fork/join events
  hipStream_t aux[2] = {nullptr, nullptr};
  hipEvent_t ev_fork = nullptr, ev_join[2] = {nullptr, nullptr};
  ~vocoder() {
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    for (GraphEntry& g : graphs) (void)hipGraphExecDestroy(g.exec);
    if (capture_stream) (void)hipStreamDestroy(capture_stream);
    for (hipStream_t a : aux)
      if (a) (void)hipStreamDestroy(a);
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    for (hipEvent_t e : ev_join)
      if (e) (void)hipEventDestroy(e);
  }
};

namespace {

#define HIP_OK(x)                          \
  do {                                     \
    if ((x) != hipSuccess) return VOCODER_EHIP; \
  } while (0)

// Brackets one kernel launch with HIP events while profiling is on.
class Prof {
 public:
  Prof(vocoder* v, hipStream_t s, const char* name, double flops, double bytes) : v_(v), s_(s) {
    if (!v->prof || v->capturing || v->no_events) return;
    int id = -1;
    for (size_t i = 0; i < v->prof_names.size(); ++i)
      if (v->prof_names[i] == name) id = (int)i;
    if (id < 0) {
      v->prof_names.push_back(name);
      id = (int)v->prof_names.size() - 1;
    }
    const size_t k = v->recs.size();
    while (v->events.size() < 2 * (k + 1)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      v->events.push_back(e);
    }
    if (hipEventRecord(v->events[2 * k], s) != hipSuccess) return;
    v->recs.push_back({id, flops, bytes});
    idx_ = (long long)k;
  }
  ~Prof() {
    if (idx_ >= 0) (void)hipEventRecord(v_->events[2 * idx_ + 1], s_);
  }

 private:
  vocoder* v_;
  hipStream_t s_;
  long long idx_ = -1;
};

// Tile per GEMM shape: skinny 64x16 / 64x32 tiles up to 32 rows (the
// transformer and first stages of one- and two-frame chunks: weight streaming),
// 64x64 up to 2048 rows (transformer linears, the first stages of short
// chunks), 96x128 when M is 96, 192 or 288 (BigVGAN stages 3-4), 128x128
// otherwise.  Launches with few tiles are split along K.  Every tile reduces
// each output in the same order, so the choice never changes a bit.
int pick_tile(int M, long long rows) {
  if (rows <= 16) return TILE_S64x16;
  if (rows <= 32) return TILE_S64x32;
  if (rows <= 2048) return TILE_64x64;
  if (M % 96 == 0 && M <= 288) return TILE_96x128;
  return TILE_128x128;
}

struct Ctx {
  vocoder* v;
  hipStream_t s;
  const float* sin_;
  float* sout;
  long long sstride;
  int B, T;
  bool quiet = false;  // no taps
  float* partial = nullptr;       // split-K partials of launches on this stream
  long long partial_floats = 0;
  float* wdeq = nullptr;          // room for one expanded int8 layer (caller's stream only)
};

ConvParams base_params(const Ctx& cx, const GemmW& g, const float* x, int rows, int nin, int dil,
                       int hslot) {
  const Plan& P = cx.v->P;
  ConvParams p{};
  p.w = cx.v->packed + g.w;
  p.wscale = g.q8 ? (const void*)(cx.v->packed + g.scale) : nullptr;
  p.w_lo = g.split ? (const void*)(reinterpret_cast<const _Float16*>(p.w) + g.lo_halves()) : nullptr;
  p.acc_scale = g.split ? std::ldexp(1.f, -SPLIT_W_EXP) : 1.f;
  p.M = g.M;
  p.k = g.k;
  p.cin = g.cin;
  p.dil = dil;
  p.x = x;
  p.sstride = cx.sstride;
  if (hslot >= 0) {
    p.hin = cx.sin_ + P.slots[hslot].off;
    p.hin_rows = P.slots[hslot].H;
  }
  p.rows = rows;
  p.nin = nin;
  p.bias = cx.v->packed + g.bias;
  p.act = ACT_NONE;
  p.phases = g.phases;
  p.cout = g.cout;
  p.mrf_mode = MRF_NONE;
  p.mrf_div = 1.f;
  p.nout = 0;
  p.splits = 1;
  p.partial = nullptr;
  return p;
}

void add_out(const Ctx& cx, ConvParams& p, float* dst, const float* alpha, int hslot, int src = 0,
             bool half = false) {
  EpiOut& o = p.out[p.nout++];
  o.dst = dst;
  o.alpha = alpha;
  o.src = src;
  o.half = half ? 1 : 0;
  if (hslot >= 0) {
    o.hist = cx.sout + cx.v->P.slots[hslot].off;
    o.H = cx.v->P.slots[hslot].H;
  } else {
    o.hist = nullptr;
    o.H = 0;
  }
}

// Split a launch along K (at accumulation-group boundaries) when it has too
// few output tiles to fill the GPU: up to ~1024 blocks, if the group partials
// fit the workspace.  The result is bitwise the same either way.
int pick_splits(long long partial_floats, int tile, int M, long long rows, int k, int cin) {
  const long long tiles = (long long)((M + gemm_tile_bm(tile) - 1) / gemm_tile_bm(tile)) *
                          ((rows + gemm_tile_bn(tile) - 1) / gemm_tile_bn(tile));
  const long long ngroups = ((long long)k * cin + VOC_GROUP_K - 1) / VOC_GROUP_K;
  if (tiles >= 256 || ngroups < 2) return 1;
  if (ngroups * rows * M > partial_floats) return 1;
  long long splits = std::min<long long>(ngroups, (1024 + tiles - 1) / tiles);
  // every split owns at least one group
  const long long gps = (ngroups + splits - 1) / splits;
  splits = (ngroups + gps - 1) / gps;
  return (int)std::max<long long>(splits, 1);
}

// ln: the GEMM's first output feeds this LayerNorm (its input is that output).
// A split GEMM normalises in its fold kernel; otherwise the LayerNorm kernel follows.
int run_gemm(const Ctx& cx, const ConvParams& pin, const LnArgs* ln = nullptr) {
  ConvParams p = pin;
  // split fp16: one kernel family at every size (the same bits on every
  // tile); the few-row tiles as in fp32, else 96-row tiles where the padded
  // weight rows cover them (128x128 needs more registers)
  const bool x3 = p.w_lo != nullptr;
  int tile = pick_tile(p.M, p.rows);
  if (x3 && (tile == TILE_96x128 || tile == TILE_128x128))
    tile = (long long)((p.M + 95) / 96) * 96 <= round_up_i(p.M, 128) ? TILE_96x128 : TILE_128x128;
  const int bm = gemm_tile_bm(tile);
  const int mt = (p.M + bm - 1) / bm;
  const bool f16 = cx.v->P.f16;
  if (!f16 && !x3 && !ln && conv_gemm_rows_ok(p)) {
    // few rows (short chunks): one launch, no split-K partials, the same bits.
    // (A launch whose output feeds a LayerNorm keeps the split-K path, whose
    // fold normalises: measured faster than this kernel plus a LayerNorm.)
    if (p.hin_rows < (p.k - 1) * p.dil) return VOCODER_EINVAL;
    const double K = (double)p.k * p.cin;
    double bytes = (p.wscale ? 1.0625 : 4.0) * p.M * K + 4.0 * p.rows * K;
    for (int o = 0; o < p.nout; ++o)
      if (p.out[o].dst) bytes += (p.out[o].half ? 2.0 : 4.0) * (double)p.rows * p.M;
    if (p.resid) bytes += 4.0 * p.rows * p.M;
    Prof pr(cx.v, cx.s, p.wscale ? "conv_gemm_rows16_q8" : "conv_gemm_rows16", 2.0 * p.M * K * p.rows, bytes);
    HIP_OK(launch_conv_gemm_rows(p, cx.s));
    return VOCODER_OK;
  }
  if (p.wscale && cx.wdeq && (tile == TILE_128x128 || tile == TILE_96x128)) {
    // int8 weights of a many-row launch: expand the layer once into the
    // workspace (q * scale, rounded to fp16 in fp16 mode, exactly what the
    // int8 kernels stage per tile) and run the float-weight kernel on it, so
    // the operands and the bits are the same
    const long long values = (long long)round_up_i(p.M, 128) * p.k * p.cin;
    if (values > cx.v->P.max_q8_values) return VOCODER_EINVAL;
    {
      Prof pr(cx.v, cx.s, "dequant_int8", 0, values * (1.0 + 2.0 / 32 + (f16 ? 2.0 : 4.0)));
      HIP_OK(launch_dequant_rows(p.w, p.wscale, values, cx.wdeq, f16, cx.s));
    }
    p.w = cx.wdeq;
    p.wscale = nullptr;
  }
  p.splits = pick_splits(cx.partial_floats, tile, p.M, p.rows, p.k, p.cin);
  p.partial = p.splits > 1 ? cx.partial : nullptr;
  // A-tile rows read must lie inside the packed (zero-padded) weight rows
  if ((long long)mt * bm > round_up_i(p.M, 128)) return VOCODER_EINVAL;
  if (p.hin_rows < (p.k - 1) * p.dil) return VOCODER_EINVAL;
  const double K = (double)p.k * p.cin;
  const double flops = 2.0 * p.M * K * p.rows;
  double bytes = 4.0 * (double)p.M * K + (p.x_half ? 2.0 : 4.0) * (double)p.rows * p.cin;
  for (int o = 0; o < p.nout; ++o)
    if (p.out[o].dst) bytes += (p.out[o].half ? 2.0 : 4.0) * (double)p.rows * p.M;
  if (p.resid) bytes += 4.0 * p.rows * p.M;
  if (p.mrf_mode == MRF_ACCUM || p.mrf_mode == MRF_LAST) bytes += 4.0 * p.rows * p.M;
  if (p.wscale) bytes -= (4.0 - 1.0625) * p.M * K;  // int8 weights and their scales
  else if (f16) bytes -= 2.0 * p.M * K;             // fp16 weights
  const bool fuse_ln = ln && p.splits > 1;
  if (fuse_ln) bytes += 8.0 * p.rows * ln->d;
  char name[48] = "";
  if (cx.v->prof && !cx.v->capturing && !cx.v->no_events) {  // (named only while profiling: host time per launch)
    const bool direct = f16 && gemm_f16_direct(p.wscale != nullptr, p.cin, tile);
    const bool window = direct && gemm_f16_window(p, tile);
    snprintf(name, sizeof(name), "conv_gemm_%s%s%dx%d_bk%d%s", x3 ? "x3_" : direct ? "f16_dma_" : f16 ? "f16_" : "",
             p.wscale ? "q8_" : "", bm, gemm_tile_bn(tile), direct || x3 ? 32 : gemm_tile_bk(tile, p.cin, f16),
             p.splits > 1 ? (fuse_ln ? "_splitk_ln" : "_splitk") : window ? "_win" : "");
  }
  {
    Prof pr(cx.v, cx.s, name, flops, bytes);
    if (x3)
      HIP_OK(launch_conv_gemm_split(p, tile, cx.s, fuse_ln ? ln : nullptr));
    else if (f16)
      HIP_OK(launch_conv_gemm_f16(p, tile, cx.s, fuse_ln ? ln : nullptr));
    else
      HIP_OK(launch_conv_gemm(p, tile, cx.s, fuse_ln ? ln : nullptr));
  }
  if (ln && !fuse_ln) {
    Prof pr(cx.v, cx.s, "layernorm", 0, 8.0 * p.rows * ln->d);
    HIP_OK(launch_layernorm(p.out[0].dst, ln->g, ln->b, ln->eps, p.rows, ln->d, ln->out, ln->T, ln->hist, ln->H,
                            ln->sstride, cx.s));
  }
  return VOCODER_OK;
}

void tap(const Ctx& cx, const char* name, const float* src, long long count) {
  if (cx.v->capturing || cx.quiet || cx.v->taps.empty()) return;
  auto it = cx.v->taps.find(name);
  if (it == cx.v->taps.end() || !it->second.first) return;
  if ((size_t)count > it->second.second) return;
  (void)hipMemcpyAsync(it->second.first, src, (size_t)count * sizeof(float), hipMemcpyDeviceToDevice, cx.s);
}

// int8 weights: the float repack goes to the (still unused) workspace, then
// each [Mpad][k*cin] row is quantized per 32 values into the packed region.
int quantize_packed(vocoder* v, const GemmW& g, hipStream_t s) {
  HIP_OK(launch_quantize_rows(v->ws, g.Mpad, g.k * g.cin, v->packed + g.w, v->packed + g.scale, s));
  return VOCODER_OK;
}

int repack_gemm(vocoder* v, const float* raw, const GemmW& g, bool transposed, hipStream_t s) {
  float* pk = v->packed;
  void* dst = g.q8 ? (void*)v->ws : (void*)(pk + g.w);
  const bool half = (v->P.f16 && !g.q8) || g.split;
  // the fp16 and split GEMMs reduce in channel-major 32-channel slabs: pack in that order
  const bool slab = (v->P.f16 || g.split) && g.cin % 32 == 0;
  const long long lo = g.split ? g.lo_halves() : 0;
  const float sc = std::ldexp(1.f, SPLIT_W_EXP);
  int* flag = reinterpret_cast<int*>(v->ws + v->P.ws.status);  // cleared before the repacks
  if (transposed) {
    HIP_OK(launch_repack_convT(raw + g.raw_w, dst, g.cin, g.cout, g.phases, g.Mpad, half, slab, s, lo, sc, flag));
    HIP_OK(launch_expand_vec(raw + g.raw_b, pk + g.bias, g.cout, g.phases, g.Mpad, s));
  } else {
    HIP_OK(launch_repack_conv(raw + g.raw_w, dst, g.M, g.Mpad, g.cin, g.k, half, slab, s, lo, sc, flag));
    HIP_OK(launch_expand_vec(raw + g.raw_b, pk + g.bias, g.M, 1, g.Mpad, s));
  }
  if (g.q8) return quantize_packed(v, g, s);
  return VOCODER_OK;
}

int copy_d2d(float* dst, const float* src, long long n, hipStream_t s) {
  HIP_OK(hipMemcpyAsync(dst, src, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, s));
  return VOCODER_OK;
}

#define CHECK(x)                   \
  do {                             \
    int _r = (x);                  \
    if (_r != VOCODER_OK) return _r; \
  } while (0)

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of the no-allocation entry point: the per-call buffers of a
// vocoder_decode_chunk_noalloc call, laid out for that call's batch x frames
// (layout_workspace, compact).  Each GPU the library runs on holds its own
// copy until the process ends; host code uses the device address looked up
// once per device (never the array's name, which on the host is only a
// stand-in).  Every no-allocation call on a GPU shares that GPU's copy.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[VOCODER_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
float* scratch_addr[SCRATCH_MAX_DEVICES] = {};
bool scratch_looked_up[SCRATCH_MAX_DEVICES] = {};

// The device address of `scratch` on the current device (looked up on the
// first call for that device), or null if it could not be obtained.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_looked_up[dev]) {
    scratch_looked_up[dev] = true;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr) scratch_addr[dev] = (float*)ptr;
  }
  return scratch_addr[dev];
}

}  // namespace

extern "C" {

size_t vocoder_raw_weights_count(const vocoder_config* cfg) {
  Plan P;
  return make_plan(cfg, P) ? (size_t)P.raw_count : 0;
}

size_t vocoder_packed_weights_bytes(const vocoder_config* cfg) {
  Plan P;
  return make_plan(cfg, P) ? (size_t)P.packed_floats * 4 : 0;
}

size_t vocoder_weights_bytes(const vocoder_config* cfg) { return vocoder_packed_weights_bytes(cfg); }

size_t vocoder_workspace_bytes(const vocoder_config* cfg) {
  Plan P;
  return make_plan(cfg, P) ? (size_t)P.ws_floats * 4 : 0;
}

size_t vocoder_state_bytes(const vocoder_config* cfg) {
  Plan P;
  return make_plan(cfg, P) ? (size_t)P.state_floats * 4 : 0;
}

int vocoder_create(const vocoder_config* cfg, const float* raw_weights, void* packed_weights, void* workspace,
                   void* stream, vocoder** out) {
  if (!out) return VOCODER_EINVAL;
  *out = nullptr;
  if (!raw_weights || !packed_weights || !workspace) return VOCODER_EINVAL;
  if (((uintptr_t)packed_weights & 255) || ((uintptr_t)workspace & 255)) return VOCODER_EINVAL;
  vocoder* v = new (std::nothrow) vocoder();
  if (!v) return VOCODER_EINVAL;
  if (!make_plan(cfg, v->P)) {
    delete v;
    return VOCODER_EINVAL;
  }
  v->hash = config_hash(cfg);
  v->packed = (float*)packed_weights;
  v->ws = (float*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const Plan& P = v->P;
  const vocoder_config& c = P.cfg;
  const float* raw = raw_weights;
  float* pk = v->packed;
  int rc = VOCODER_OK;
  auto fail = [&](int r) { delete v; return r; };

  if (launch_fill(pk, (size_t)P.packed_floats * 4, s) != hipSuccess) return fail(VOCODER_EHIP);
  // the split repacks flag weights out of range in the status word
  if (launch_fill(v->ws + P.ws.status, 256, s) != hipSuccess) return fail(VOCODER_EHIP);
  if ((rc = copy_d2d(pk + P.codebooks, raw + P.raw_codebooks,
                     (long long)c.n_codebooks * c.codebook_size * c.embed_dim, s))) return fail(rc);
  if ((rc = repack_gemm(v, raw, P.pre, false, s))) return fail(rc);
  const int d = P.d;
  for (const LayerP& L : P.layers) {
    if ((rc = copy_d2d(pk + L.ln1_g, raw + L.raw_ln1_g, d, s))) return fail(rc);
    if ((rc = copy_d2d(pk + L.ln1_b, raw + L.raw_ln1_b, d, s))) return fail(rc);
    if ((rc = copy_d2d(pk + L.ln2_g, raw + L.raw_ln2_g, d, s))) return fail(rc);
    if ((rc = copy_d2d(pk + L.ln2_b, raw + L.raw_ln2_b, d, s))) return fail(rc);
    // q, k, v stacked along M into one [3d][1][d] GEMM
    const long long raw_w[3] = {L.raw_q_w, L.raw_k_w, L.raw_v_w};
    const long long raw_b[3] = {L.raw_q_b, L.raw_k_b, L.raw_v_b};
    for (int t = 0; t < 3; ++t) {
      const long long off = (long long)t * d * d;  // elements
      const bool half = (P.f16 && !L.qkv.q8) || L.qkv.split;
      void* dst = L.qkv.q8 ? (void*)(v->ws + off)
                  : half   ? (void*)(reinterpret_cast<_Float16*>(pk + L.qkv.w) + off)
                           : (void*)(pk + L.qkv.w + off);
      // (one tap: the tap-major and slab orders coincide; a split's lo plane
      // follows the whole stacked hi plane)
      if (launch_repack_conv(raw + raw_w[t], dst, d, d, d, 1, half, false, s,
                             L.qkv.split ? L.qkv.lo_halves() : 0, std::ldexp(1.f, SPLIT_W_EXP),
                             reinterpret_cast<int*>(v->ws + P.ws.status)) != hipSuccess)
        return fail(VOCODER_EHIP);
      if ((rc = copy_d2d(pk + L.qkv.bias + (long long)t * d, raw + raw_b[t], d, s))) return fail(rc);
    }
    if (L.qkv.q8) {
      // rows past the three stacked projections are padding: zero
      const long long used = 3LL * d * d, all = (long long)L.qkv.Mpad * d;
      if (all > used && launch_fill(v->ws + used, (size_t)(all - used) * 4, s) != hipSuccess)
        return fail(VOCODER_EHIP);
      if ((rc = quantize_packed(v, L.qkv, s))) return fail(rc);
    }
    if ((rc = repack_gemm(v, raw, L.o, false, s))) return fail(rc);
    if ((rc = repack_gemm(v, raw, L.fc1, false, s))) return fail(rc);
    if ((rc = repack_gemm(v, raw, L.fc2, false, s))) return fail(rc);
  }
  if ((rc = copy_d2d(pk + P.fln_g, raw + P.raw_fln_g, d, s))) return fail(rc);
  if ((rc = copy_d2d(pk + P.fln_b, raw + P.raw_fln_b, d, s))) return fail(rc);
  for (const GemmW& g : P.ups)
    if ((rc = repack_gemm(v, raw, g, true, s))) return fail(rc);
  if ((rc = repack_gemm(v, raw, P.conv_pre, false, s))) return fail(rc);
  for (const StageP& S : P.stages) {
    if ((rc = repack_gemm(v, raw, S.up, true, s))) return fail(rc);
    for (int j = 0; j < c.n_res; ++j) {
      const AmpP& A0 = S.amp[(size_t)j * c.n_dil];
      if (launch_expand_vec(raw + A0.raw_act1, pk + S.up_alpha[j], S.c, S.r, S.up.Mpad, s) != hipSuccess)
        return fail(VOCODER_EHIP);
    }
    for (const AmpP& A : S.amp) {
      if ((rc = repack_gemm(v, raw, A.conv1, false, s))) return fail(rc);
      if ((rc = repack_gemm(v, raw, A.conv2, false, s))) return fail(rc);
      if ((rc = copy_d2d(pk + A.act1, raw + A.raw_act1, S.c, s))) return fail(rc);
      if ((rc = copy_d2d(pk + A.act2, raw + A.raw_act2, S.c, s))) return fail(rc);
    }
  }
  const int CL = P.stages.back().c;
  if ((rc = copy_d2d(pk + P.post_alpha, raw + P.raw_post_alpha, CL, s))) return fail(rc);
  // conv_post [1][C][k] -> [k][C]
  if (launch_repack_conv(raw + P.raw_post_w, pk + P.post_w, 1, 1, CL, c.post_kernel, false, false, s) != hipSuccess)
    return fail(VOCODER_EHIP);
  if ((rc = copy_d2d(pk + P.post_b, raw + P.raw_post_b, 1, s))) return fail(rc);

  // RoPE inverse frequencies (float64) and the slot table, staged from the host
  std::vector<double> inv(std::max(P.half, 1), 0.0);
  for (int i = 0; i < P.half; ++i) inv[i] = std::pow((double)c.rope_theta, -2.0 * i / (double)P.hd);
  if (hipMemcpyAsync(pk + P.inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice, s) !=
      hipSuccess)
    return fail(VOCODER_EHIP);
  if (!P.slots.empty() && hipMemcpyAsync(pk + P.slots_off, P.slots.data(), P.slots.size() * sizeof(Slot),
                                         hipMemcpyHostToDevice, s) != hipSuccess)
    return fail(VOCODER_EHIP);
  // the host vectors above are released on return: wait for the copies
  if (hipStreamSynchronize(s) != hipSuccess) return fail(VOCODER_EHIP);
  if (P.split) {
    int range = 0;
    if (hipMemcpy(&range, v->ws + P.ws.status, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(VOCODER_EHIP);
    if (range) return fail(VOCODER_EINVAL);  // a weight beyond the split's range
  }
  if (launch_fill(v->ws + P.ws.status, 256, s) != hipSuccess) return fail(VOCODER_EHIP);
  if (P.ws.conc_frames > 0) {
    bool ok = hipEventCreateWithFlags(&v->ev_fork, hipEventDisableTiming) == hipSuccess;
    for (int j = 0; j < 2 && ok; ++j)
      ok = hipStreamCreateWithFlags(&v->aux[j], hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&v->ev_join[j], hipEventDisableTiming) == hipSuccess;
    if (!ok) return fail(VOCODER_EHIP);
  }
  // the no-allocation entry point's scratch on this (the handle's) device;
  // if it cannot be had, that entry point reports VOCODER_EHIP
  v->scratch = scratch_on_current_device();
  *out = v;
  return VOCODER_OK;
}

int vocoder_reset(vocoder* v, void* state, int batch, void* stream) {
  if (!v || !state || batch < 1) return VOCODER_EINVAL;
  if ((uintptr_t)state & 255) return VOCODER_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  HIP_OK(launch_fill(state, (size_t)batch * v->P.state_floats * 4, s));
  HIP_OK(launch_reset_headers(state, v->P.state_floats, batch, v->hash, s));
  return VOCODER_OK;
}

}  // extern "C"

namespace {

// Host-side argument checks shared by the eager and the graph entry points.
// state_out may be state_in itself (an in-place decode) but must not overlap
// it otherwise.
bool decode_args_ok(const vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                    const void* state_out, const float* pcm, bool need_pcm = true) {
  if (!v || !codes || !state_in || !state_out || (need_pcm && !pcm)) return false;
  const Plan& P = v->P;
  const vocoder_config& c = P.cfg;
  if (batch < 1 || batch > c.max_batch || n_frames < 1 || n_frames > c.max_frames) return false;
  if (((uintptr_t)state_in & 255) || ((uintptr_t)state_out & 255)) return false;
  if (state_in == state_out) return true;
  const char* a = (const char*)state_in;
  const char* b = (const char*)state_out;
  const size_t n = (size_t)batch * P.state_floats * 4;
  return !(a < b + n && b < a + n);
}

// Every launch of one decode call, in order, on stream `stream`.  Launches
// and device-to-device copies only: no host synchronisation, allocation or
// memset, so the sequence can be recorded into a HIP graph as it stands.
// prefill: produce state_out only (no PCM, no taps), taking the stack after
// the transformer through the chunk's last tail_frames frames alone.
// L / wsb: the layout and base of the per-call buffers (the handle's
// workspace, or the static scratch of the no-allocation entry point); the
// status word is always the handle's.
int decode_launches(vocoder* v, const WsLayout& L, float* wsb, const int32_t* codes, int batch, int n_frames,
                    const void* state_in, void* state_out, float* pcm, void* stream, bool prefill = false) {
  const Plan& P = v->P;
  const vocoder_config& c = P.cfg;
  // In place (state_out == state_in): every kernel below reads the old state
  // while others write the new one, so the batch's states are first copied to
  // the workspace and read from there.
  if (state_in == state_out) {
    float* snap = wsb + L.snap;
    const long long n = (long long)batch * P.state_floats;
    {
      Prof pr(v, (hipStream_t)stream, "state_snapshot", 0, 8.0 * n);
      HIP_OK(launch_copy(snap, (const float*)state_in, n, (hipStream_t)stream));
    }
    state_in = snap;
  }
  Ctx cx;
  cx.quiet = prefill;
  cx.partial = wsb + L.partial;
  cx.partial_floats = L.partial_floats;
  cx.wdeq = L.wdeq ? wsb + L.wdeq : nullptr;
  cx.v = v;
  cx.s = (hipStream_t)stream;
  cx.sin_ = (const float*)state_in;
  cx.sout = (float*)state_out;
  cx.sstride = P.state_floats;
  cx.B = batch;
  cx.T = n_frames;
  const int B = batch, T = n_frames, d = P.d;
  const int R = B * T;
  float* ws = wsb;
  const float* pk = v->packed;
  int* status = reinterpret_cast<int*>(v->ws + P.ws.status);
  int* pos = reinterpret_cast<int*>(ws + L.pos);
  float* rope = ws + L.rope;

  {
  Prof pr(v, cx.s, "begin", 0, 4.0 * B * (double)T * P.half * 2);
  HIP_OK(launch_begin(cx.sin_, cx.sout, cx.sstride, B, T, v->hash,
                      reinterpret_cast<const double*>(pk + P.inv_freq), P.half, rope, pos, status, cx.s));
  }
  {
  Prof pr(v, cx.s, "state_shift", 0, 0);
  HIP_OK(launch_state_shift(reinterpret_cast<const Slot*>(pk + P.slots_off), (int)P.slots.size(), 0, cx.sin_,
                            cx.sout, cx.sstride, B, T, cx.s));
  }

  // RVQ embedding sum
  float* emb = ws + L.emb;
  const Slot& spre = P.slots[P.slot_pre];
  {
  Prof pr(v, cx.s, "gather", 0, (double)R * c.n_codebooks * (4.0 + 4.0 * c.embed_dim) + 4.0 * R * c.embed_dim);
  HIP_OK(launch_gather(codes, pk + P.codebooks, c.n_codebooks, c.codebook_size, c.embed_dim, R, T, emb,
                       spre.H > 0 ? cx.sout + spre.off : nullptr, spre.H, cx.sstride, status, cx.s));
  }
  tap(cx, "embed", emb, (long long)R * c.embed_dim);

  // Each LayerNorm runs with the GEMM that produces its input (the pre-conv
  // or a residual projection): the next layer's first norm, or the final
  // norm, whose last row feeds the first transposed conv's history.
  float* h = ws + L.h;
  float* u = ws + L.u;
  auto ln_after = [&](int l) {
    if (l < c.n_layers) return LnArgs{pk + P.layers[l].ln1_g, pk + P.layers[l].ln1_b, c.ln_eps, d, u, T, nullptr, 0, 0};
    const Slot& so = P.slots[c.n_up > 0 ? P.slot_ups[0] : P.slot_conv_pre];
    return LnArgs{pk + P.fln_g, pk + P.fln_b, c.ln_eps, d, u, T, cx.sout + so.off, so.H, cx.sstride};
  };

  // causal conv before the transformer
  {
    ConvParams p = base_params(cx, P.pre, emb, R, T, 1, P.slot_pre);
    add_out(cx, p, h, nullptr, -1);
    const LnArgs ln = ln_after(0);
    CHECK(run_gemm(cx, p, &ln));
  }
  tap(cx, "pre_conv", h, (long long)R * d);

  // transformer
  float* qkv = ws + L.qkv;
  float* att = ws + L.att;
  float* ffn = ws + L.ffn;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerP& L = P.layers[l];
    {
      ConvParams p = base_params(cx, L.qkv, u, R, T, 1, -1);
      add_out(cx, p, qkv, nullptr, -1);
      CHECK(run_gemm(cx, p));
    }
    const Slot& sk = P.slots[L.slot_k];
    const Slot& sv = P.slots[L.slot_v];
    {
      // RoPE on the new frames' q and k, and their K/V into the state tail, happen in the staging
      const double keys = (double)c.window + 1;
      const double tail = (double)B * std::min(T, c.window) * 2 * d;
      Prof pr(v, cx.s, "attention", 4.0 * R * keys * d,
              4.0 * ((double)B * c.window * 2 * d + 3.0 * R * d + R * d + tail) + 8.0 * R * (P.hd / 2));
      HIP_OK(launch_attention(qkv, cx.sin_ + sk.off, cx.sin_ + sv.off, cx.sstride, pos, B, T, c.n_heads, P.hd,
                              c.window, rope, cx.sout + sk.off, cx.sout + sv.off, att, cx.s));
    }
    {
      ConvParams p = base_params(cx, L.o, att, R, T, 1, -1);
      p.resid = h;
      add_out(cx, p, h, nullptr, -1);
      const LnArgs ln{pk + L.ln2_g, pk + L.ln2_b, c.ln_eps, d, u, T, nullptr, 0, 0};
      CHECK(run_gemm(cx, p, &ln));
    }
    {
      ConvParams p = base_params(cx, L.fc1, u, R, T, 1, -1);
      p.act = ACT_GELU;
      add_out(cx, p, ffn, nullptr, -1);
      CHECK(run_gemm(cx, p));
    }
    {
      ConvParams p = base_params(cx, L.fc2, ffn, R, T, 1, -1);
      p.resid = h;
      add_out(cx, p, h, nullptr, -1);
      const LnArgs ln = ln_after(l + 1);
      CHECK(run_gemm(cx, p, &ln));
    }
    char nm[32];
    snprintf(nm, sizeof(nm), "layer%d", l);
    tap(cx, nm, h, (long long)R * d);
  }
  tap(cx, "final_ln", u, (long long)R * d);

  // Prefill: every carried row from here on depends only on the last
  // tail_frames frames (each row's value is computed by the same operations
  // whatever rows precede it), so run the rest on those frames alone; the
  // rows they would have read from earlier frames never reach a carried row.
  const int F = prefill ? std::min(T, P.tail_frames) : T;
  const float* x = u;
  if (F < T) {
    // the residual stream h is dead after the final LayerNorm: gather the
    // tail rows [B][F][d] there
    HIP_OK(hipMemcpy2DAsync(h, (size_t)F * d * sizeof(float), u + (size_t)(T - F) * d,
                            (size_t)T * d * sizeof(float), (size_t)F * d * sizeof(float), B,
                            hipMemcpyDeviceToDevice, cx.s));
    x = h;
  }

  // 2x2 upsampling: transposed convs as phase-stacked 2-tap GEMMs
  long long nin = F;
  for (int i = 0; i < c.n_up; ++i) {
    const GemmW& g = P.ups[i];
    float* y = ws + L.up[i];
    ConvParams p = base_params(cx, g, x, (int)(B * nin), (int)nin, 1, P.slot_ups[i]);
    const int next = i + 1 < c.n_up ? P.slot_ups[i + 1] : P.slot_conv_pre;
    add_out(cx, p, y, nullptr, next);
    CHECK(run_gemm(cx, p));
    nin *= g.phases;
    char nm[32];
    snprintf(nm, sizeof(nm), "up%d", i);
    tap(cx, nm, y, B * nin * d);
    x = y;
  }
  // conv_pre into the first stage's input
  int sbuf = 0;
  float* S_in = ws + L.S[sbuf];
  {
    ConvParams p = base_params(cx, P.conv_pre, x, (int)(B * nin), (int)nin, 1, P.slot_conv_pre);
    add_out(cx, p, S_in, nullptr, P.stages[0].slot_up);
    CHECK(run_gemm(cx, p));
  }
  tap(cx, "conv_pre", S_in, B * nin * c.voc_ch0);

  // BigVGAN stages
  float* X0 = ws + L.X0;
  float* Tb = ws + L.T;
  float* Xr = ws + L.Xr;
  float* An = ws + L.An;
  for (int si = 0; si < c.n_stages; ++si) {
    const StageP& S = P.stages[si];
    const bool last_stage = si + 1 == c.n_stages;
    float* S_out = ws + L.S[sbuf ^ 1];
    // transposed conv: raw output + the first Snake of every AMP block
    {
      ConvParams p = base_params(cx, S.up, S_in, (int)(B * nin), (int)nin, 1, S.slot_up);
      add_out(cx, p, X0, nullptr, -1);
      // Snake outputs are read only as GEMM operands: fp16 in fp16 mode
      for (int j = 0; j < c.n_res; ++j)
        add_out(cx, p, ws + L.A[j], pk + S.up_alpha[j], S.amp[(size_t)j * c.n_dil].slot1, 0, P.f16);
      CHECK(run_gemm(cx, p));
    }
    nin *= S.r;
    const int rows = (int)(B * nin);
    {
      char nm[32];
      snprintf(nm, sizeof(nm), "stage%d.up", si);
      tap(cx, nm, X0, (long long)rows * S.c);
    }
    // AMP blocks.  A short chunk (at most conc_frames frames over the batch)
    // runs them concurrently: every block but the last on a side stream, each
    // with its own intermediates and split-K partials, the last on the
    // caller's stream, which waits for the others before its final conv and
    // sums the multi-receptive-field mean in the sequential order, ((block 0
    // + block 1) + block 2) / 3.  Longer chunks fill the GPU one block at a
    // time and run the blocks in order.
    const bool conc = L.conc_frames > 0 && (long long)B * T <= L.conc_frames && v->aux[0] && v->aux[1];
    if (conc) {
      HIP_OK(hipEventRecord(v->ev_fork, cx.s));
      for (int j = 0; j + 1 < c.n_res; ++j) HIP_OK(hipStreamWaitEvent(v->aux[j], v->ev_fork, 0));
    }
    for (int j = 0; j < c.n_res; ++j) {
      const bool side = conc && j + 1 < c.n_res;
      Ctx bc = cx;
      float* tb = Tb;
      float* xr = Xr;
      float* an = An;
      if (side) {
        bc.s = v->aux[j];
        bc.partial = ws + L.partial_aux[j];
        bc.partial_floats = L.partial_aux_floats;
        bc.wdeq = nullptr;  // the int8 kernels dequantize per tile
        tb = ws + L.conc_T[j];
        xr = ws + L.conc_Xr[j];
        an = ws + L.conc_An[j];
      }
      for (int i = 0; i < c.n_dil; ++i) {
        const AmpP& A = S.amp[(size_t)j * c.n_dil + i];
        const float* a_in = i == 0 ? ws + L.A[j] : an;
        // conv(k, d) of Snake_1(x), then Snake_2
        {
          ConvParams p = base_params(bc, A.conv1, a_in, rows, (int)nin, c.dilations[i], A.slot1);
          p.x_half = P.f16;
          add_out(bc, p, tb, pk + A.act2, A.slot2, 0, P.f16);
          CHECK(run_gemm(bc, p));
        }
        // conv(k, 1) + residual
        {
          ConvParams p = base_params(bc, A.conv2, tb, rows, (int)nin, 1, A.slot2);
          p.x_half = P.f16;
          p.resid = i == 0 ? X0 : xr;
          if (i + 1 < c.n_dil) {
            const AmpP& An1 = S.amp[(size_t)j * c.n_dil + i + 1];
            add_out(bc, p, xr, nullptr, -1);
            add_out(bc, p, an, pk + An1.act1, An1.slot1, 0, P.f16);
          } else {
            p.mrf = S_out;
            p.mrf_div = (float)c.n_res;
            if (c.n_res == 1) p.mrf_mode = MRF_ONLY;
            else if (j + 1 == c.n_res) p.mrf_mode = MRF_LAST;
            else if (j == 0 || conc) p.mrf_mode = MRF_FIRST;
            else p.mrf_mode = MRF_ACCUM;
            const bool fin = p.mrf_mode == MRF_LAST || p.mrf_mode == MRF_ONLY;
            if (!fin) {
              // concurrent: block 0 into S_out, block 1 into its own buffer
              add_out(bc, p, side && j == 1 ? ws + L.conc_B1 : S_out, nullptr, -1, 1);
            } else {
              if (conc) {
                for (int jj = 0; jj + 1 < c.n_res; ++jj) HIP_OK(hipStreamWaitEvent(cx.s, v->ev_join[jj], 0));
                if (c.n_res == 3) p.mrf2 = ws + L.conc_B1;
              }
              if (!last_stage)
                add_out(bc, p, S_out, nullptr, P.stages[si + 1].slot_up, 1);
              else
                add_out(bc, p, S_out, pk + P.post_alpha, P.slot_post, 1);
            }
          }
          CHECK(run_gemm(bc, p));
          if (side && i + 1 == c.n_dil) HIP_OK(hipEventRecord(v->ev_join[j], bc.s));
        }
      }
    }
    {
      char nm[32];
      snprintf(nm, sizeof(nm), "stage%d", si);
      tap(cx, nm, S_out, (long long)rows * S.c);
    }
    sbuf ^= 1;
    S_in = S_out;
  }
  // final Snake is already applied: conv_post + tanh
  if (!prefill) {
    const Slot& sp = P.slots[P.slot_post];
    auto it = v->taps.find("pre_tanh");
    float* pre = nullptr;
    const long long rows = B * nin;
    if (!v->capturing && it != v->taps.end() && it->second.first && (size_t)rows <= it->second.second)
      pre = it->second.first;
    const double C = P.stages.back().c;
    Prof pr(v, cx.s, "conv_post", 2.0 * rows * C * c.post_kernel, 4.0 * rows * (C + 1 + (pre ? 1 : 0)));
    HIP_OK(launch_conv_post(S_in, cx.sin_ + sp.off, cx.sstride, sp.H, pk + P.post_w, pk + P.post_b,
                            P.stages.back().c, c.post_kernel, (int)rows, (int)nin, pcm, pre, cx.s));
  }
  return VOCODER_OK;
}

}  // namespace

extern "C" {

int vocoder_decode_chunk(vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                         void* state_out, float* pcm, void* stream) {
  if (!decode_args_ok(v, codes, batch, n_frames, state_in, state_out, pcm)) return VOCODER_EINVAL;
  return decode_launches(v, v->P.ws, v->ws, codes, batch, n_frames, state_in, state_out, pcm, stream);
}

int vocoder_decode_chunk_graph(vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                               void* state_out, float* pcm, void* stream) {
  if (!decode_args_ok(v, codes, batch, n_frames, state_in, state_out, pcm)) return VOCODER_EINVAL;
  const GraphKey key{codes, state_in, state_out, pcm, batch, n_frames};
  ++v->graph_clock;
  for (GraphEntry& e : v->graphs)
    if (e.key == key) {
      e.last_use = v->graph_clock;
      HIP_OK(hipGraphLaunch(e.exec, (hipStream_t)stream));
      return VOCODER_OK;
    }
  // record the launch sequence on the library's own capture stream (nothing
  // runs while recording), then instantiate and launch on the caller's stream
  if (!v->capture_stream) HIP_OK(hipStreamCreateWithFlags(&v->capture_stream, hipStreamNonBlocking));
  HIP_OK(hipStreamBeginCapture(v->capture_stream, hipStreamCaptureModeThreadLocal));
  v->capturing = true;
  const int rc =
      decode_launches(v, v->P.ws, v->ws, codes, batch, n_frames, state_in, state_out, pcm, v->capture_stream);
  v->capturing = false;
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(v->capture_stream, &graph);
  if (rc != VOCODER_OK || ec != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc != VOCODER_OK ? rc : VOCODER_EHIP;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return VOCODER_EHIP;
  if ((int)v->graphs.size() >= VOCODER_GRAPH_CACHE) {
    size_t lru = 0;
    for (size_t i = 1; i < v->graphs.size(); ++i)
      if (v->graphs[i].last_use < v->graphs[lru].last_use) lru = i;
    (void)hipGraphExecDestroy(v->graphs[lru].exec);
    v->graphs.erase(v->graphs.begin() + lru);
  }
  v->graphs.push_back({key, exec, v->graph_clock});
  HIP_OK(hipGraphLaunch(exec, (hipStream_t)stream));
  return VOCODER_OK;
}

int vocoder_decode_chunk_noalloc(vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                                 void* state_out, float* pcm, void* stream) {
  if (!decode_args_ok(v, codes, batch, n_frames, state_in, state_out, pcm)) return VOCODER_EINVAL;
  WsLayout L;
  layout_workspace(v->P, batch, n_frames, true, L);
  if ((unsigned long long)L.floats * 4 > (unsigned long long)VOCODER_NOALLOC_SCRATCH_BYTES) return VOCODER_ESCRATCH;
  if (!v->scratch) return VOCODER_EHIP;
  v->no_events = true;
  const int rc = decode_launches(v, L, v->scratch, codes, batch, n_frames, state_in, state_out, pcm, stream);
  v->no_events = false;
  return rc;
}

int vocoder_quantize_int8(const float* src, long long rows, int K, int8_t* q, uint16_t* scale, void* stream) {
  if (!src || !q || !scale || rows < 0 || K <= 0 || K % 32 != 0) return VOCODER_EINVAL;
  HIP_OK(launch_quantize_rows(src, rows, K, q, scale, (hipStream_t)stream));
  return VOCODER_OK;
}

int vocoder_graph_cache_size(const vocoder* v) { return v ? (int)v->graphs.size() : -1; }

int vocoder_prefill(vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                    void* state_out, void* stream) {
  if (!decode_args_ok(v, codes, batch, n_frames, state_in, state_out, nullptr, false)) return VOCODER_EINVAL;
  return decode_launches(v, v->P.ws, v->ws, codes, batch, n_frames, state_in, state_out, nullptr, stream, true);
}

int vocoder_prefill_tail_frames(const vocoder* v) { return v ? v->P.tail_frames : 0; }

int vocoder_profile_begin(vocoder* v) {
  if (!v) return VOCODER_EINVAL;
  v->prof = true;
  v->recs.clear();
  return VOCODER_OK;
}

int vocoder_profile_end(vocoder* v, void* stream, vocoder_kernel_stat* out, int max_entries, int* n_entries) {
  if (!v || max_entries < 0 || (max_entries > 0 && !out)) return VOCODER_EINVAL;
  v->prof = false;
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  std::vector<vocoder_kernel_stat> agg(v->prof_names.size());
  for (size_t i = 0; i < agg.size(); ++i) {
    memset(&agg[i], 0, sizeof(agg[i]));
    snprintf(agg[i].name, sizeof(agg[i].name), "%s", v->prof_names[i].c_str());
  }
  for (size_t k = 0; k < v->recs.size(); ++k) {
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, v->events[2 * k], v->events[2 * k + 1]));
    vocoder_kernel_stat& a = agg[v->recs[k].name];
    a.launches += 1;
    a.total_ms += ms;
    a.flops += v->recs[k].flops;
    a.bytes += v->recs[k].bytes;
  }
  v->recs.clear();
  int n = 0;
  for (const auto& a : agg) {
    if (a.launches == 0) continue;
    if (n < max_entries) out[n] = a;
    ++n;
  }
  if (n_entries) *n_entries = n;
  return VOCODER_OK;
}

int vocoder_hop(const vocoder* v) { return v ? v->P.hop : 0; }

int vocoder_left_context_frames(const vocoder* v) { return v ? v->P.cfg.window : 0; }

int vocoder_get_status(vocoder* v, void* stream) {
  if (!v) return VOCODER_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int st = 0;
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(&st, v->ws + v->P.ws.status, sizeof(int), hipMemcpyDeviceToHost));
  HIP_OK(launch_fill(v->ws + v->P.ws.status, 256, s));
  HIP_OK(hipStreamSynchronize(s));
  if (st & VOC_STATUS_CODE) return VOCODER_ECODE;
  if (st & VOC_STATUS_STATE) return VOCODER_ESTATE;
  return VOCODER_OK;
}

int vocoder_set_tap(vocoder* v, const char* name, float* dst, size_t dst_floats) {
  if (!v || !name) return VOCODER_EINVAL;
  if (!dst) {
    v->taps.erase(name);
    return VOCODER_OK;
  }
  v->taps[name] = {dst, dst_floats};
  return VOCODER_OK;
}

void vocoder_destroy(vocoder* v) { delete v; }

const char* vocoder_strerror(int status) {
  switch (status) {
    case VOCODER_OK: return "ok";
    case VOCODER_EINVAL: return "invalid argument";
    case VOCODER_ESTATE: return "state does not belong to this decoder";
    case VOCODER_EHIP: return "HIP error";
    case VOCODER_ECODE: return "code out of range";
    case VOCODER_ESCRATCH: return "chunk needs more than the static scratch of the no-allocation entry point";
  }
  return "unknown status";
}

}  // extern "C"

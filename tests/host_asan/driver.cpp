// Host-side driver for the sanitizer build of the library: exercises the
// config validation, the packed-weight / state / workspace layout planning
// and the host-side argument checks of every entry point -- everything that
// runs before (or instead of) a HIP call -- on known decoder shapes and on
// fuzzed configs with extreme field values.  No call here reaches the GPU.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "vocoder.h"

static int failures = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static vocoder_config qwen3(int max_batch, int max_frames) {
  vocoder_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_codebooks = 16; c.codebook_size = 2048; c.embed_dim = 512; c.model_dim = 1024;
  c.n_layers = 8; c.n_heads = 16; c.window = 72; c.ffn_dim = 4096;
  c.rope_theta = 10000.f; c.ln_eps = 1e-5f; c.pre_kernel = 3;
  c.n_up = 2; c.up_strides[0] = 2; c.up_strides[1] = 2;
  c.voc_ch0 = 1536; c.conv_pre_kernel = 7; c.n_stages = 4;
  c.rates[0] = 8; c.rates[1] = 5; c.rates[2] = 4; c.rates[3] = 3;
  c.n_res = 3; c.res_kernels[0] = 3; c.res_kernels[1] = 7; c.res_kernels[2] = 11;
  c.n_dil = 3; c.dilations[0] = 1; c.dilations[1] = 3; c.dilations[2] = 5;
  c.post_kernel = 7; c.max_batch = max_batch; c.max_frames = max_frames;
  c.precision = VOCODER_PRECISION_F32; c.weight_format = VOCODER_WEIGHTS_FLOAT;
  return c;
}

static void sizes(const vocoder_config& c, size_t out[4]) {
  out[0] = vocoder_raw_weights_count(&c);
  out[1] = vocoder_packed_weights_bytes(&c);
  out[2] = vocoder_workspace_bytes(&c);
  out[3] = vocoder_state_bytes(&c);
}

int main() {
  size_t s[4];
  // known shapes, every precision and weight format
  for (int prec = 0; prec < 3; ++prec)
    for (int wf = 0; wf < 2; ++wf) {
      vocoder_config c = qwen3(64, 25);
      c.precision = prec;
      c.weight_format = wf;
      sizes(c, s);
      const bool ok = !(prec == VOCODER_PRECISION_SPLIT16 && wf == VOCODER_WEIGHTS_INT8);
      EXPECT(ok == (s[0] != 0) && ok == (s[1] != 0) && ok == (s[2] != 0) && ok == (s[3] != 0));
      if (ok) {
        EXPECT(s[0] == 259806497u);
        EXPECT(s[1] % 256 == 0 && s[2] % 256 == 0 && s[3] % 256 == 0);
      }
    }
  // workspace grows with max_batch x max_frames, the state does not
  {
    size_t a[4], b[4];
    sizes(qwen3(1, 1), a);
    sizes(qwen3(64, 25), b);
    EXPECT(a[2] < b[2] && a[3] == b[3] && a[1] == b[1]);
  }
  // fuzzed configs: every field from a set of ordinary and extreme values;
  // the four size queries must agree on validity and never misbehave
  std::mt19937 rng(12345);
  const int32_t ints[] = {INT_MIN, -1, 0, 1, 2, 3, 4, 7, 11, 16, 31, 32, 48, 64, 65, 72, 96, 255, 256,
                          1024, 1536, 2048, 4096, 4352, 65536, 1 << 20, INT_MAX};
  const float floats[] = {0.f, -1.f, 1e-5f, 1.f, 1e4f, 3.4e38f};
  auto pick = [&](auto& arr) { return arr[rng() % (sizeof(arr) / sizeof(arr[0]))]; };
  int valid = 0;
  for (int it = 0; it < 20000; ++it) {
    vocoder_config c = qwen3(1 + (int)(rng() % 8), 1 + (int)(rng() % 8));
    int32_t* f = reinterpret_cast<int32_t*>(&c);
    const int nfields = (int)(sizeof(c) / sizeof(int32_t));
    const int nmut = 1 + (int)(rng() % 3);
    for (int m = 0; m < nmut; ++m) {
      const int k = (int)(rng() % nfields);
      if (k == 8 || k == 9) {  // rope_theta, ln_eps
        const float v = pick(floats);
        std::memcpy(&f[k], &v, sizeof(v));
      } else {
        f[k] = pick(ints);
      }
    }
    sizes(c, s);
    const bool any = s[0] || s[1] || s[2] || s[3];
    const bool all = s[0] && s[1] && s[2] && s[3];
    EXPECT(any == all);
    valid += all ? 1 : 0;
  }
  EXPECT(valid > 100);
  // host-side argument errors of every entry point (no handle, bad pointers)
  vocoder* h = nullptr;
  vocoder_config c = qwen3(2, 4);
  EXPECT(vocoder_create(&c, nullptr, nullptr, nullptr, nullptr, &h) == VOCODER_EINVAL && h == nullptr);
  EXPECT(vocoder_create(&c, nullptr, nullptr, nullptr, nullptr, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_create(nullptr, nullptr, nullptr, nullptr, nullptr, &h) == VOCODER_EINVAL);
  // misaligned packed / workspace pointers are refused before any HIP call
  EXPECT(vocoder_create(&c, reinterpret_cast<const float*>(256), reinterpret_cast<void*>(260),
                        reinterpret_cast<void*>(512), nullptr, &h) == VOCODER_EINVAL);
  vocoder_config bad = c;
  bad.n_heads = 3;  // invalid shape: refused before any HIP call
  EXPECT(vocoder_create(&bad, reinterpret_cast<const float*>(256), reinterpret_cast<void*>(256),
                        reinterpret_cast<void*>(512), nullptr, &h) == VOCODER_EINVAL);
  const int32_t* codes = reinterpret_cast<const int32_t*>(256);
  void* st = reinterpret_cast<void*>(512);
  float* pcm = reinterpret_cast<float*>(1024);
  EXPECT(vocoder_reset(nullptr, st, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_decode_chunk(nullptr, codes, 1, 1, st, st, pcm, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_decode_chunk_graph(nullptr, codes, 1, 1, st, st, pcm, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_decode_chunk_noalloc(nullptr, codes, 1, 1, st, st, pcm, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_prefill(nullptr, codes, 1, 1, st, st, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_quantize_int8(nullptr, 1, 32, nullptr, nullptr, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_quantize_int8(reinterpret_cast<const float*>(256), -1, 32, reinterpret_cast<int8_t*>(256),
                               reinterpret_cast<uint16_t*>(256), nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_quantize_int8(reinterpret_cast<const float*>(256), 1, 48, reinterpret_cast<int8_t*>(256),
                               reinterpret_cast<uint16_t*>(256), nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_get_status(nullptr, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_set_tap(nullptr, "embed", nullptr, 0) == VOCODER_EINVAL);
  EXPECT(vocoder_profile_begin(nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_profile_end(nullptr, nullptr, nullptr, 0, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_hop(nullptr) == 0 && vocoder_left_context_frames(nullptr) == 0);
  EXPECT(vocoder_graph_cache_size(nullptr) == -1 && vocoder_prefill_tail_frames(nullptr) == 0);
  EXPECT(vocoder_peak_mfma(0, nullptr, 1, 8, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_peak_mfma(2, reinterpret_cast<float*>(256), 1, 8, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_stream_read(nullptr, 4, nullptr, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_stream_copy(nullptr, nullptr, 4, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_grid_barrier(nullptr, nullptr, nullptr, 2, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_grid_barrier(reinterpret_cast<unsigned*>(256), reinterpret_cast<float*>(256),
                              reinterpret_cast<int*>(256), 1, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_empty_launches(nullptr, 1, 1, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_empty_launches(reinterpret_cast<int*>(256), 1, 0, nullptr) == VOCODER_EINVAL);
  EXPECT(vocoder_peak_mfma_flops(0, 1, 8) == 2.0 * 16 * 16 * 4 * 4 * 4 * 8);
  for (int code = -6; code <= 1; ++code) EXPECT(vocoder_strerror(code) != nullptr);
  vocoder_destroy(nullptr);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks passed (%d valid of 20000 fuzzed configs)\n", valid);
  return 0;
}

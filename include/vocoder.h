/*
 * vocoder.h -- C ABI of the streaming code2wav decoder on MI355X (gfx950).
 *
 * What it computes ("Edge TTS design (vLLM-Omni-compatible)", section 1.3,
 * Codec / vocoder): each 12.5 Hz codec frame carries one code per codebook
 * (16 codebooks); the decoder sums the selected RVQ codewords, runs a causal
 * conv, a stack of pre-norm transformer layers with a sliding attention window
 * (72 frames), two stride-2 transposed convs, a causal conv into the BigVGAN
 * stack (per stage: a causal transposed conv of kernel 2 x rate, then the mean
 * of AMP residual blocks of Snake -> dilated conv -> Snake -> conv), a final
 * Snake -> conv -> tanh, and emits `hop` fp32 samples per frame (1920 at 24 kHz
 * for the Qwen3-TTS-12Hz shape).  The call shape follows section 2.2
 * (IDecoderAdapter: decode(frames), reset(), left_context_frames()) with the
 * state made explicit as an input and an output, as section 4 proposes for the
 * ExecuTorch decoder, and section 2.3 (the decoder's conv context and attention
 * window live for an utterance and survive between calls).
 *
 * Conventions
 *  - Every data pointer is a DEVICE pointer on the current HIP device, except
 *    the vocoder_config pointer (host).  `stream` is a hipStream_t (NULL = the
 *    null stream).  Calls enqueue work on `stream` and never synchronise it,
 *    except vocoder_get_status.  A decode of a short chunk (at most 64 frames
 *    over the batch) also runs part of its work on two streams the handle
 *    owns, forked from `stream` and joined back into it by events: every
 *    call's work still starts after earlier work on `stream` and ends before
 *    later work on it.
 *  - The caller owns every device buffer (raw and packed weights, workspace,
 *    states, codes, PCM).  The library allocates no device memory; it owns its
 *    host-side handle, two streams and three events created by vocoder_create,
 *    and the graphs vocoder_decode_chunk_graph records, all released by
 *    vocoder_destroy.
 *  - Return values: VOCODER_OK (0) or a negative VOCODER_E* code.  Argument
 *    errors are detected on the host before any HIP call.  Errors the device
 *    detects (a code out of range, a state that belongs to another decoder) are
 *    recorded in a status word inside the workspace and reported by
 *    vocoder_get_status.
 *  - A handle is not thread-safe; calls on one handle must be ordered on one
 *    stream.  Distinct handles are independent.
 */
#ifndef VOCODER_H
#define VOCODER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VOCODER_OK 0
#define VOCODER_EINVAL (-1)       /* null pointer, bad size, unsupported config */
#define VOCODER_ESTATE (-2)       /* state header does not match this decoder (device-detected) */
#define VOCODER_EHIP (-3)         /* a HIP call or kernel launch failed */
#define VOCODER_ECODE (-4)        /* a code outside [0, codebook_size) (device-detected) */
#define VOCODER_ESCRATCH (-5)     /* vocoder_decode_chunk_noalloc: the chunk's buffers exceed its static scratch */

#define VOCODER_MAX_UP 4
#define VOCODER_MAX_STAGES 8
#define VOCODER_MAX_RES 4
#define VOCODER_MAX_DIL 4

/* Decoder shape.  All channel counts that feed a convolution or linear layer
 * must be multiples of 16; model_dim is at most 4096; model_dim / n_heads (the
 * head size) must be at most 256 and a multiple of 8.  Qwen3-TTS-12Hz shape: 16, 2048, 512, 1024, 8, 16, 72, 4096,
 * 10000, 1e-5, 3, 2, {2,2}, 1536, 7, 4, {8,5,4,3}, 3, {3,7,11}, 3, {1,3,5}, 7. */
typedef struct vocoder_config {
  int32_t n_codebooks;      /* codes per frame (16) */
  int32_t codebook_size;    /* entries per codebook (2048) */
  int32_t embed_dim;        /* codeword width (512) */
  int32_t model_dim;        /* transformer width d (1024) */
  int32_t n_layers;         /* transformer layers (8) */
  int32_t n_heads;          /* attention heads (16) */
  int32_t window;           /* attention window W in frames (72): a frame attends itself and the W before it */
  int32_t ffn_dim;          /* FFN hidden width (4096) */
  float rope_theta;         /* RoPE base (10000) */
  float ln_eps;             /* LayerNorm epsilon (1e-5) */
  int32_t pre_kernel;       /* causal conv kernel before the transformer (3) */
  int32_t n_up;             /* transposed convs after the transformer (2) */
  int32_t up_strides[VOCODER_MAX_UP];       /* their strides ({2,2}); kernel = 2 x stride, d -> d */
  int32_t voc_ch0;          /* BigVGAN input channels (1536) */
  int32_t conv_pre_kernel;  /* causal conv d -> voc_ch0 (7) */
  int32_t n_stages;         /* BigVGAN stages (4) */
  int32_t rates[VOCODER_MAX_STAGES];        /* stage strides ({8,5,4,3}); kernel 2 x rate, channels halve */
  int32_t n_res;            /* AMP blocks per stage (3) */
  int32_t res_kernels[VOCODER_MAX_RES];     /* their kernel sizes ({3,7,11}) */
  int32_t n_dil;            /* dilations per AMP block (3) */
  int32_t dilations[VOCODER_MAX_DIL];       /* ({1,3,5}) */
  int32_t post_kernel;      /* final conv kernel, C -> 1 (7) */
  int32_t max_batch;        /* largest batch a decode call may pass (sizes the workspace) */
  int32_t max_frames;       /* largest n_frames a decode call may pass (sizes the workspace) */
  int32_t precision;        /* VOCODER_PRECISION_F32 (0), _F16 (1) or _SPLIT16 (2), see below */
  int32_t weight_format;    /* VOCODER_WEIGHTS_FLOAT (0) or VOCODER_WEIGHTS_INT8 (1), see below */
} vocoder_config;

/* Arithmetic of the matrix products (every conv, transposed conv and linear
 * except the final C -> 1 conv).  F32: fp32 operands, fp32 MFMA.  F16: both
 * operands rounded to IEEE binary16 (ties to even) -- weights when packed,
 * activations as they are read -- and products summed in fp32 on the fp16
 * MFMA; everything else (embedding sum, LayerNorm, attention, GELU, Snake,
 * residuals, biases, the final conv, all stored activations and the state)
 * stays fp32.  The edge design page (section 1.5, quality row) allows the
 * decoder fp16 at most; activations must stay within fp16 range (|x| < 65504).
 * SPLIT16: fp32 values throughout, as F32, with the products of the matrix
 * products made on the fp16 MFMA: each fp32 operand v is written as hi + lo,
 * hi = fp16(v) and lo = fp16(v - hi) (both ties to even; the subtraction is
 * exact), and a product w*x as lo_w*hi_x + hi_w*lo_x + hi_w*hi_x, summed in
 * fp32 (lo_w*lo_x, below 2^-22 of w*x, is dropped).  This is the split of
 * Ootomo and Yokota (2022, single-precision accuracy from fp16 matrix units),
 * with one power-of-two scale per operand in place of their scaled lo term:
 * weights are split as w * 2^8 and sums scaled back by 2^-8 (exact), which
 * keeps their lo halves in fp16's normal range; inputs are split unscaled (the
 * fp16 MFMA keeps subnormal inputs exactly).  Weights are split when packed
 * (4 bytes per value, as fp32) and activations as they are read; layers whose
 * input channel count is not a multiple of 32 run the F32 kernels.  Weights
 * must lie within +-2^8 (vocoder_create returns VOCODER_EINVAL for a weight
 * whose scaled hi half would not be finite) and activations within the fp16
 * range (|v| < 65504).
 * Every product of a layer takes the same three MFMAs in the same order, so
 * decodes stay bitwise independent of batch and chunking.
 * The precision is part of the state's identity: states are not
 * interchangeable between precisions. */
#define VOCODER_PRECISION_F32 0
#define VOCODER_PRECISION_F16 1
#define VOCODER_PRECISION_SPLIT16 2

/* Storage of the matrix-product weights.  FLOAT: fp32 (precision F32) or
 * fp16 (F16).  INT8: the blixt/phonon page's weight format (section Weights):
 * a weight tensor of 16,384 values or more becomes int8 with one fp16 scale per
 * 32 values along its rows, the scale being max |value| / 127 of the 32 values
 * after rounding them to fp16, and each value round(v / scale), ties to even;
 * all arithmetic stays as `precision` says, on the dequantized value q * scale
 * (exact in fp32; rounded to fp16 for F16).  Here a row is one output channel
 * at one tap, its values the input channels, so the tensors quantized are the
 * conv, transposed-conv and linear weights of at least 16,384 values whose
 * input channel count is a multiple of 32 (all of them at the Qwen3-TTS-12Hz
 * shape); the others, the codebooks, the vectors and the final C -> 1 conv
 * keep their float storage.  Packed, every such weight takes 1.0625 bytes
 * per value; launches with few rows read it so, while a launch with many rows
 * first expands its layer into the workspace (4 or 2 bytes per value; the
 * workspace holds the largest int8 layer) and reads that.  Weights must lie
 * within the fp16 range.  INT8 is not offered with SPLIT16. */
#define VOCODER_WEIGHTS_FLOAT 0
#define VOCODER_WEIGHTS_INT8 1

typedef struct vocoder vocoder;

/* Number of floats in the raw weight vector vocoder_create reads: every
 * parameter, C-contiguous, in this order and these PyTorch-native layouts
 * (Linear [out][in], Conv1d [out][in][k], ConvTranspose1d [in][out][k]):
 *   codebooks [n_codebooks][codebook_size][embed_dim];
 *   pre_conv.weight [d][embed_dim][pre_kernel], pre_conv.bias [d];
 *   per layer: ln1.weight, ln1.bias [d]; q_proj, k_proj, v_proj, o_proj
 *     (.weight [d][d], .bias [d] each); ln2.weight, ln2.bias [d];
 *     fc1.weight [ffn][d], fc1.bias [ffn]; fc2.weight [d][ffn], fc2.bias [d];
 *   final_ln.weight, final_ln.bias [d];
 *   per up i: weight [d][d][2*up_strides[i]], bias [d];
 *   conv_pre.weight [voc_ch0][d][conv_pre_kernel], conv_pre.bias [voc_ch0];
 *   per stage s (C = voc_ch0 >> s input, C/2 output):
 *     up.weight [C][C/2][2*rates[s]], up.bias [C/2];
 *     per AMP block j, per dilation i: act1.alpha [C/2], conv1.weight
 *       [C/2][C/2][res_kernels[j]], conv1.bias [C/2], act2.alpha [C/2],
 *       conv2.weight [C/2][C/2][res_kernels[j]], conv2.bias [C/2];
 *   act_post.alpha [C_last]; conv_post.weight [1][C_last][post_kernel];
 *   conv_post.bias [1].
 * Returns 0 if the config is invalid. */
size_t vocoder_raw_weights_count(const vocoder_config* cfg);

/* Bytes of the packed-weight buffer (library-internal layout). 0 if invalid.
 * vocoder_weights_bytes is the same call under a second, shorter name. */
size_t vocoder_packed_weights_bytes(const vocoder_config* cfg);
size_t vocoder_weights_bytes(const vocoder_config* cfg);

/* Bytes of the workspace for max_batch streams x max_frames frames (including
 * room for one batch of states, the input copy of an in-place decode).  0 if
 * invalid. */
size_t vocoder_workspace_bytes(const vocoder_config* cfg);

/* Bytes of one stream's state (a header plus every carried row).  A batch of
 * states is [batch][state_bytes], stream b at offset b * state_bytes.  The
 * state holds the frame position, the last `window` RoPE-rotated keys and
 * values of every layer, and the last (k-1)*dilation input rows of every
 * convolution (one row per transposed conv).  0 if invalid. */
size_t vocoder_state_bytes(const vocoder_config* cfg);

/* Build a decoder.  `raw_weights` (device, vocoder_raw_weights_count floats)
 * is repacked into `packed_weights` (device, vocoder_packed_weights_bytes,
 * 256-byte aligned) by kernels on `stream`; raw_weights may be freed once
 * `stream` has completed that work.  `workspace` (device,
 * vocoder_workspace_bytes, 256-byte aligned) must stay valid and unshared for
 * the handle's life.  On success *out receives the handle.  It returns once
 * the repacking is done (it synchronizes `stream`).
 * Errors: VOCODER_EINVAL (bad config or pointer; SPLIT16 with a weight out of
 * its range), VOCODER_EHIP. */
int vocoder_create(const vocoder_config* cfg, const float* raw_weights, void* packed_weights,
                   void* workspace, void* stream, vocoder** out);

/* Reset `batch` consecutive states (device, [batch][state_bytes]) to a fresh
 * utterance: position 0, empty window, zero conv context (the decoder
 * adapter's reset() of section 2.2, which drops all carried context).  Errors: VOCODER_EINVAL,
 * VOCODER_EHIP. */
int vocoder_reset(vocoder* v, void* state, int batch, void* stream);

/* Decode one chunk of n_frames frames for each of `batch` streams.
 *   codes     int32 [batch][n_frames][n_codebooks] (device)
 *   state_in  [batch][state_bytes] (device), read
 *   state_out [batch][state_bytes] (device), written.  Either state_in itself
 *             (an in-place decode: the state the decoder adapter keeps across
 *             calls, "Edge TTS design", sections 2.3 and 4) or a buffer that
 *             does not overlap it (ping-pong two buffers across calls).  In
 *             place, the call first copies the batch's states into the
 *             workspace and reads the old state from that copy (one extra pass
 *             over batch * state_bytes); the results are bit for bit those of a
 *             ping-pong call.
 *   pcm       float [batch][n_frames * hop] (device), written
 * Streams may sit at different positions.  A chunk of T frames emits exactly
 * T * hop samples per stream; any chunking of a stream gives the same samples
 * as decoding it whole (each output element is reduced in the same order).
 * Errors: VOCODER_EINVAL (null pointer, batch not in [1, max_batch], n_frames
 * not in [1, max_frames], states that overlap without being the same buffer,
 * a state pointer not 256-byte aligned), VOCODER_EHIP.  Device-detected
 * errors (VOCODER_ECODE: that chunk's PCM is unspecified and no out-of-range
 * codeword is read; VOCODER_ESTATE: the stream is decoded from a fresh state)
 * are reported by vocoder_get_status. */
int vocoder_decode_chunk(vocoder* v, const int32_t* codes, int batch, int n_frames,
                         const void* state_in, void* state_out, float* pcm, void* stream);

/* Graph entries a handle keeps (least recently used evicted). */
#define VOCODER_GRAPH_CACHE 32

/* vocoder_decode_chunk replayed from a HIP graph: the server runs the decoder
 * with one stateful graph per reachable chunk length ("Edge TTS design",
 * section 1.3); small chunks are bound by launch overhead.  Same arguments,
 * checks, results (bit for bit) and error reporting as vocoder_decode_chunk.
 * The first call for a given (codes, state_in, state_out, pcm, batch,
 * n_frames) records the call's launch sequence into a graph (nothing runs
 * while recording), instantiates it and keeps it in the handle; later calls
 * with the same six values only launch that graph on `stream`.  A streaming
 * caller that ping-pongs two state buffers and reuses its code and PCM buffers
 * therefore holds two graphs per chunk length.  Buffers named by a kept graph
 * must stay allocated while the handle lives (or be re-used only at the same
 * address and size).  Taps and profiling apply to eager calls only.  Graphs
 * hold driver resources, released by vocoder_destroy.  Errors: as
 * vocoder_decode_chunk, and VOCODER_EHIP if recording or instantiation fails. */
int vocoder_decode_chunk_graph(vocoder* v, const int32_t* codes, int batch, int n_frames,
                               const void* state_in, void* state_out, float* pcm, void* stream);

/* Bytes of the static device scratch of vocoder_decode_chunk_noalloc (per GPU). */
#define VOCODER_NOALLOC_SCRATCH_BYTES (256u << 20)

/* vocoder_decode_chunk for callers that cannot allocate device memory at all
 * at call time (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, checks, results (bit for bit) and
 * error reporting as vocoder_decode_chunk, but the call's buffers
 * (activations, split-K partials, the copy of the states of an in-place call)
 * come from a fixed static device array of VOCODER_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends, laid out
 * for this call's batch x n_frames, instead of from the handle's workspace
 * (which still holds the status word).  The call allocates nothing and
 * creates no events (profiling does not apply to it); taps do.  At the
 * Qwen3-TTS-12Hz shape a chunk needs about 25 MB per frame of batch x
 * n_frames plus one state (6 MB) per stream, so one stream's chunks of up to
 * 10 frames fit; a larger chunk returns VOCODER_ESCRATCH before any launch.
 * Launches whose split-K partials would not fit the compact layout are not
 * split and int8 weights are dequantized per tile: the same bits either way.
 * Every call on one GPU, from any handle, shares that GPU's scratch, and
 * nothing in it needs to start at zero: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race and must be
 * ordered by the caller.  Errors: as vocoder_decode_chunk, VOCODER_ESCRATCH,
 * and VOCODER_EHIP if the scratch's device address could not be obtained
 * when the handle was created. */
int vocoder_decode_chunk_noalloc(vocoder* v, const int32_t* codes, int batch, int n_frames,
                                 const void* state_in, void* state_out, float* pcm, void* stream);

/* The int8 weight quantizer vocoder_create applies (see VOCODER_WEIGHTS_INT8),
 * on a caller's matrix: src fp32 [rows][K] (device, K a multiple of 32) ->
 * q int8 [rows][K] and scale fp16 [rows][K/32] (device, IEEE binary16 bits),
 * one scale per 32 consecutive values of a row.  Errors: VOCODER_EINVAL (null
 * pointer, K not a positive multiple of 32, rows < 0), VOCODER_EHIP. */
int vocoder_quantize_int8(const float* src, long long rows, int K, int8_t* q, uint16_t* scale, void* stream);

/* Graphs the handle currently keeps (0..VOCODER_GRAPH_CACHE), -1 for NULL. */
int vocoder_graph_cache_size(const vocoder* v);

/* Reference prefix: decode `codes` into the state without emitting audio.
 * The decoder's cross-chunk state includes a cache of the voice-clone
 * reference prefix ("Edge TTS design", section 1.3): the reference's codes are
 * run through the decoder before the utterance so that its window and conv
 * context start from them.  state_out is bit for bit the state_out of
 * vocoder_decode_chunk on the same arguments; no PCM is written.  The
 * transformer runs over all n_frames frames (its window of keys and values is
 * carried); the stack after it runs over the last
 * vocoder_prefill_tail_frames frames only, which determine every carried row
 * of that stack.  A prefix longer than max_frames is fed in several calls.
 * Arguments and errors as vocoder_decode_chunk without `pcm`. */
int vocoder_prefill(vocoder* v, const int32_t* codes, int batch, int n_frames, const void* state_in,
                    void* state_out, void* stream);

/* Frames at the end of a prefill call that go through the upsampling stack
 * (9 for the Qwen3-TTS-12Hz shape); 0 for NULL. */
int vocoder_prefill_tail_frames(const vocoder* v);

/* Samples per frame (product of up_strides and rates): 1920 for Qwen3-TTS-12Hz. */
int vocoder_hop(const vocoder* v);

/* Frames of attention left context the state carries (= window), as
 * IDecoderAdapter::left_context_frames(). */
int vocoder_left_context_frames(const vocoder* v);

/* Synchronise `stream`, return the first device-detected error since the last
 * call (VOCODER_ECODE or VOCODER_ESTATE) or VOCODER_OK, and clear it. */
int vocoder_get_status(vocoder* v, void* stream);

/* Debug taps: when set, each decode call also copies the named intermediate
 * tensor (channels-last, [batch][rows][channels]) to `dst` (device; NULL
 * clears).  Names: "embed", "pre_conv", "layer<l>", "final_ln", "up<i>",
 * "conv_pre", "stage<s>.up", "stage<s>" (for the last stage: after the final
 * Snake), "pre_tanh" ([batch][n_frames*hop]).  `dst_floats` is its capacity;
 * a decode whose tap would overflow it skips the copy.  Errors: VOCODER_EINVAL. */
int vocoder_set_tap(vocoder* v, const char* name, float* dst, size_t dst_floats);

/* Measurement.  Between vocoder_profile_begin and vocoder_profile_end, every
 * kernel a decode call launches is bracketed by HIP events recorded on the
 * caller's stream.  vocoder_profile_end synchronises the stream, stops
 * recording and aggregates per kernel: launches, total device time, and the
 * kernel's algorithmic work (FLOPs of the dense contraction it computes, and
 * the bytes it must read and write at least once).  Up to `max_entries`
 * records are written to `out`; *n_entries receives how many exist.  Events
 * are created by the library (host-side objects, no device allocation) and
 * released by vocoder_destroy.  Errors: VOCODER_EINVAL, VOCODER_EHIP. */
typedef struct vocoder_kernel_stat {
  char name[48];      /* kernel family, e.g. "conv_gemm_96x256_bk32" */
  int32_t launches;
  double total_ms;    /* sum of event-measured launch durations */
  double flops;       /* algorithmic FLOPs summed over launches */
  double bytes;       /* algorithmic bytes summed over launches */
} vocoder_kernel_stat;

int vocoder_profile_begin(vocoder* v);
int vocoder_profile_end(vocoder* v, void* stream, vocoder_kernel_stat* out, int max_entries, int* n_entries);

/* Roofline microbenchmarks: kernels of their own that measure, on the GPU at
 * hand, the two denominators the decoder's kernels are judged against (the
 * benchmark reports them beside the vendor's peaks).  None needs a handle.
 *
 * vocoder_peak_mfma: `blocks` workgroups of 4 waves, each wave issuing `iters`
 * rounds of 4 independent dependent-chain MFMAs on operands held in
 * registers -- v_mfma_f32_16x16x4_f32 (dtype 0) or v_mfma_f32_16x16x32_f16
 * (dtype 1) -- with no memory traffic but one float per thread written to
 * `out` (device, blocks * 256 floats).  iters: a positive multiple of 8.
 * vocoder_peak_mfma_flops gives the FLOPs such a launch performs.
 * vocoder_stream_read: sum n floats of `src` (device, 16-byte aligned, n a
 * multiple of 4) with `blocks` workgroups of 256 threads, grid-stride 16-byte
 * loads, one float per thread to `out` (blocks * 256 floats).
 * vocoder_stream_copy: dst[i] = src[i] for n floats (both 16-byte aligned).
 * All enqueue on `stream`.  Errors: VOCODER_EINVAL, VOCODER_EHIP. */
double vocoder_peak_mfma_flops(int dtype, int blocks, int iters);
int vocoder_peak_mfma(int dtype, float* out, int blocks, int iters, void* stream);
int vocoder_stream_read(const float* src, long long n, float* out, int blocks, void* stream);
int vocoder_stream_copy(const float* src, float* dst, long long n, int blocks, void* stream);

/* The price of an ordering point between dependent steps ("blixt/phonon",
 * Speed: its note on the cost of an empty dependent dispatch): a grid-wide
 * barrier inside one kernel, against a launch boundary.
 * vocoder_grid_barrier: a cooperative grid of `blocks` workgroups of 256
 * threads (2 <= blocks <= what the GPU holds at once, else VOCODER_EINVAL)
 * runs `rounds` rounds.  In each round every block writes 64 floats to its
 * slot of `slots`, crosses a barrier, reads another block's slot and checks it,
 * and crosses a second barrier: 2 * rounds barriers in all.  A barrier is a
 * flag per block, gathered by block 0, which then publishes the round; flags
 * and slots are written and read past the caches.  Device buffers, all the
 * caller's: `flags` blocks + 1 uint32, zero on entry (the call leaves them
 * non-zero); `slots` blocks * 64 floats; `err` one int32, zero on entry.
 * Every wait is bounded: a wait that runs out sets bit 0 of *err (the grid
 * then drains), and a check that fails sets bit 1.
 * vocoder_empty_launches: n back-to-back launches of a kernel of `blocks`
 * workgroups that does nothing observable; `scratch` is 2 device int32 it
 * reads.  Both enqueue on `stream`.  Errors: VOCODER_EINVAL, VOCODER_EHIP. */
int vocoder_grid_barrier(unsigned* flags, float* slots, int* err, int blocks, int rounds, void* stream);
int vocoder_empty_launches(int* scratch, int blocks, int n, void* stream);

/* Free the host handle (device buffers stay the caller's). */
void vocoder_destroy(vocoder* v);

/* Static text for a status code. */
const char* vocoder_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* VOCODER_H */

// Microbenchmarks that measure the two roofline denominators on the GPU at
// hand: the dense matrix-core rate (fp32 and fp16 MFMA, operands in
// registers, no memory traffic) and the HBM streaming rate (a read-only
// reduction and a copy).  Two more price the ordering points of a chain of
// dependent steps: a grid-wide barrier inside one kernel against a launch
// boundary.  They run nothing of the decoder; the benchmark reports their
// rates beside the vendor's peaks.

#include <algorithm>

#include "vocoder.h"  // include/, on the compiler include path
#include "common.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int PEAK_THREADS = 256;  // 4 waves: one per SIMD of a CU
constexpr int PEAK_CHAINS = 4;     // independent accumulators per wave (hides the MFMA latency)
constexpr int PEAK_UNROLL = 8;

// Each iteration issues PEAK_CHAINS independent v_mfma_f32_16x16x4_f32 per
// wave (2 * 16 * 16 * 4 FLOPs each) on operands held in registers.
__global__ __launch_bounds__(PEAK_THREADS) void peak_mfma_f32_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const float a = 1.0f + (float)lane * 1e-3f;
  const float b = 1.0f - (float)lane * 1e-3f;
  f32x4 acc[PEAK_CHAINS];
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, (float)c};
  for (int i = 0; i < iters; i += PEAK_UNROLL) {
#pragma unroll
    for (int u = 0; u < PEAK_UNROLL; ++u)
#pragma unroll
      for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) s += (acc[c].x + acc[c].y) + (acc[c].z + acc[c].w);
  out[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

// The same with v_mfma_f32_16x16x32_f16 (2 * 16 * 16 * 32 FLOPs each).
__global__ __launch_bounds__(PEAK_THREADS) void peak_mfma_f16_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(1.0f + (float)(lane + e) * 1e-3f);
    b[e] = (_Float16)(1.0f - (float)(lane + e) * 1e-3f);
  }
  f32x4 acc[PEAK_CHAINS];
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, (float)c};
  for (int i = 0; i < iters; i += PEAK_UNROLL) {
#pragma unroll
    for (int u = 0; u < PEAK_UNROLL; ++u)
#pragma unroll
      for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) s += (acc[c].x + acc[c].y) + (acc[c].z + acc[c].w);
  out[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

// Streaming read: every thread sums its 16-byte pieces, STREAM_UNROLL
// independent loads in flight (grid-stride: each wave reads 1 KB contiguous
// per load), and writes one float.
constexpr int STREAM_UNROLL = 8;

__global__ __launch_bounds__(PEAK_THREADS) void stream_read_kernel(const f32x4* __restrict__ src, long long n4,
                                                                   float* __restrict__ out) {
  f32x4 s[STREAM_UNROLL];
#pragma unroll
  for (int u = 0; u < STREAM_UNROLL; ++u) s[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const long long stride = (long long)gridDim.x * PEAK_THREADS;
  long long i = (long long)blockIdx.x * PEAK_THREADS + threadIdx.x;
  for (; i + (STREAM_UNROLL - 1) * stride < n4; i += STREAM_UNROLL * stride) {
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) s[u] += __builtin_nontemporal_load(src + i + u * stride);
  }
  for (; i < n4; i += stride) s[0] += src[i];
  f32x4 t = s[0];
#pragma unroll
  for (int u = 1; u < STREAM_UNROLL; ++u) t += s[u];
  out[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = (t.x + t.y) + (t.z + t.w);
}

// Streaming copy of 16-byte pieces (grid-stride), STREAM_UNROLL loads in
// flight per thread.
__global__ __launch_bounds__(PEAK_THREADS) void stream_copy_kernel(const f32x4* __restrict__ src,
                                                                   f32x4* __restrict__ dst, long long n4) {
  const long long stride = (long long)gridDim.x * PEAK_THREADS;
  long long i = (long long)blockIdx.x * PEAK_THREADS + threadIdx.x;
  for (; i + (STREAM_UNROLL - 1) * stride < n4; i += STREAM_UNROLL * stride) {
    f32x4 v[STREAM_UNROLL];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n4; i += stride) dst[i] = src[i];
}

// Grid-wide ordering against launch boundaries.  A decode of a few frames is
// a chain of dependent launches, and each boundary costs a dispatch on top of
// the work (the blixt/phonon page, Speed: its note on the cost of an empty
// dependent dispatch).  A persistent kernel would put a grid-wide barrier in
// each boundary's place; grid_barrier_kernel measures one.  Every block
// publishes the round in its own flag, block 0 gathers the flags and then
// publishes the round once for all.  Flags and the data checked across the
// barrier are written and read past the caches (relaxed system-scope
// accesses), so no cache writeback or invalidate is needed.  Every wait is
// bounded: one that runs out sets bit 0 of *err and its block leaves, so the
// grid always drains; a read of another block's data that does not hold that
// block's value of the round sets bit 1.
constexpr long BARRIER_SPIN_LIMIT = 1L << 22;
constexpr int BARRIER_THREADS = 256;
constexpr int BARRIER_SLOT = 64;  // floats each block writes per round

__device__ __forceinline__ bool grid_barrier(unsigned* flags, int* err, unsigned round) {
  __syncthreads();
  const unsigned nb = gridDim.x;
  unsigned* go = flags + nb;
  if (threadIdx.x == 0) __hip_atomic_store(flags + blockIdx.x, round, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (blockIdx.x == 0) {
    for (unsigned t = threadIdx.x; t < nb; t += BARRIER_THREADS) {
      long spins = 0;
      while (__hip_atomic_load(flags + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != round) {
        if (++spins > BARRIER_SPIN_LIMIT) {
          __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(go, round, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  } else if (threadIdx.x == 0) {
    long spins = 0;
    while (__hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != round) {
      if (++spins > BARRIER_SPIN_LIMIT) {
        __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
    }
  }
  __syncthreads();
  return (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) & 1) == 0;
}

// `rounds` rounds of: write this block's slot, barrier, read another block's
// slot and check it, barrier (before the next round overwrites the slots).
__global__ __launch_bounds__(BARRIER_THREADS) void grid_barrier_kernel(unsigned* flags, float* slots, int* err,
                                                                       int rounds) {
  const unsigned nb = gridDim.x;
  const unsigned other = (blockIdx.x + nb / 2 + 1) % nb;
  bool bad = false;
  unsigned round = 0;
  for (int r = 0; r < rounds; ++r) {
    if (threadIdx.x < BARRIER_SLOT) {
      __hip_atomic_store(slots + (size_t)blockIdx.x * BARRIER_SLOT + threadIdx.x, (float)(r * 7 + (int)blockIdx.x),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __builtin_amdgcn_s_waitcnt(0);  // the slot is written before the flag
    }
    if (!grid_barrier(flags, err, ++round)) return;
    if (threadIdx.x < BARRIER_SLOT) {
      const float v = __hip_atomic_load(slots + (size_t)other * BARRIER_SLOT + threadIdx.x, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_SYSTEM);
      bad |= v != (float)(r * 7 + (int)other);
    }
    if (!grid_barrier(flags, err, ++round)) return;
  }
  if (bad) __hip_atomic_fetch_or(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// A kernel that does nothing observable (its store never happens): the cost
// of a dependent launch on its own.
__global__ __launch_bounds__(BARRIER_THREADS) void empty_kernel(int* p) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && p[0] == 0x7fffffff) p[1] = 0;
}

}  // namespace

extern "C" {

double vocoder_peak_mfma_flops(int dtype, int blocks, int iters) {
  const double per_mfma = dtype == 1 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 4;
  return per_mfma * PEAK_CHAINS * (PEAK_THREADS / 64) * (double)blocks * (double)iters;
}

int vocoder_peak_mfma(int dtype, float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < PEAK_UNROLL || iters % PEAK_UNROLL || (dtype != 0 && dtype != 1))
    return VOCODER_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(peak_mfma_f32_kernel, dim3(blocks), dim3(PEAK_THREADS), 0, s, out, iters);
  else
    hipLaunchKernelGGL(peak_mfma_f16_kernel, dim3(blocks), dim3(PEAK_THREADS), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? VOCODER_OK : VOCODER_EHIP;
}

int vocoder_stream_read(const float* src, long long n, float* out, int blocks, void* stream) {
  if (!src || !out || n < 4 || n % 4 || blocks < 1 || ((uintptr_t)src & 15)) return VOCODER_EINVAL;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(PEAK_THREADS), 0, (hipStream_t)stream,
                     reinterpret_cast<const f32x4*>(src), n / 4, out);
  return hipGetLastError() == hipSuccess ? VOCODER_OK : VOCODER_EHIP;
}

int vocoder_stream_copy(const float* src, float* dst, long long n, int blocks, void* stream) {
  if (!src || !dst || n < 4 || n % 4 || blocks < 1 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return VOCODER_EINVAL;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(PEAK_THREADS), 0, (hipStream_t)stream,
                     reinterpret_cast<const f32x4*>(src), reinterpret_cast<f32x4*>(dst), n / 4);
  return hipGetLastError() == hipSuccess ? VOCODER_OK : VOCODER_EHIP;
}

int vocoder_grid_barrier(unsigned* flags, float* slots, int* err, int blocks, int rounds, void* stream) {
  if (!flags || !slots || !err || blocks < 2 || rounds < 1) return VOCODER_EINVAL;
  int dev = 0, cus = 0, per_cu = 0, coop = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)grid_barrier_kernel, BARRIER_THREADS, 0) !=
          hipSuccess)
    return VOCODER_EHIP;
  // every block must be resident at once, or the first barrier could not complete
  if (!coop || (long long)blocks > (long long)cus * per_cu) return VOCODER_EINVAL;
  void* args[] = {&flags, &slots, &err, &rounds};
  if (hipLaunchCooperativeKernel((const void*)grid_barrier_kernel, dim3(blocks), dim3(BARRIER_THREADS), args, 0,
                                 (hipStream_t)stream) != hipSuccess)
    return VOCODER_EHIP;
  return VOCODER_OK;
}

int vocoder_empty_launches(int* scratch, int blocks, int n, void* stream) {
  if (!scratch || blocks < 1 || n < 1) return VOCODER_EINVAL;
  for (int i = 0; i < n; ++i)
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(BARRIER_THREADS), 0, (hipStream_t)stream, scratch);
  return hipGetLastError() == hipSuccess ? VOCODER_OK : VOCODER_EHIP;
}

}  // extern "C"

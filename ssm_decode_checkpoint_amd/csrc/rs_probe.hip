// Measurement helper, not part of the decode library: a read-only stream with
// the decode kernels' access pattern (one tile of T threads x P 16-byte
// non-temporal loads per workgroup, summed and written as one float), to tell
// what fraction of the read bandwidth this chip reaches for such tiles the
// decode kernels achieve.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rs_probe.h"

namespace {

typedef float vf4 __attribute__((ext_vector_type(4)));

template <int T, int P>
__global__ __launch_bounds__(T) void read_tiles(const vf4* __restrict__ src, float* __restrict__ out) {
  const vf4* p = src + static_cast<size_t>(blockIdx.x) * (T * P) + threadIdx.x;
  vf4 r[P];
#pragma unroll
  for (int k = 0; k < P; ++k) r[k] = __builtin_nontemporal_load(p + k * T);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < P; ++k) s += (r[k].x + r[k].y) + (r[k].z + r[k].w);
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  __shared__ float w[T / 64];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int i = 0; i < T / 64; ++i) t += w[i];
    out[blockIdx.x] = t;
  }
}

template <int T, int P>
int32_t launch(const void* src, float* out, uint64_t bytes, hipStream_t st) {
  const uint64_t tile = static_cast<uint64_t>(T) * P * 16;
  if (bytes == 0 || bytes % tile != 0 || bytes / tile > 0x7FFFFFFFull) return -2;
  read_tiles<T, P><<<static_cast<unsigned>(bytes / tile), T, 0, st>>>(static_cast<const vf4*>(src), out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

extern "C" int32_t rs_probe_read(const void* src, float* out, uint64_t bytes, int32_t threads, int32_t per_thread,
                                 void* stream) {
  if (!src || !out || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (threads == 256 && per_thread == 8) return launch<256, 8>(src, out, bytes, st);
  if (threads == 256 && per_thread == 4) return launch<256, 4>(src, out, bytes, st);
  if (threads == 128 && per_thread == 16) return launch<128, 16>(src, out, bytes, st);
  return -4;
}

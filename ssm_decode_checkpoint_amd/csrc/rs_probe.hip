// Measurement helper, not part of the decode library: a read-only stream with
// the decode kernels' access pattern (one tile of T threads x P 16-byte
// non-temporal loads per workgroup, summed and written as one float), to tell
// what fraction of the read bandwidth this chip reaches for such tiles the
// decode kernels achieve; and the same stream with a few hundred bytes written
// per tile after its sum, as a decode step writes its output and appended
// record, to price those writes inside a saturated read stream.
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

// The same tile read; then lanes 0 .. wbytes/16 - 1 each store 16 bytes
// (non-temporal) of their wave's sum at dst + tile * wbytes.
template <int T, int P>
__global__ __launch_bounds__(T) void read_write_tiles(const vf4* __restrict__ src, vf4* __restrict__ dst,
                                                      int wvec) {
  const vf4* p = src + static_cast<size_t>(blockIdx.x) * (T * P) + threadIdx.x;
  vf4 r[P];
#pragma unroll
  for (int k = 0; k < P; ++k) r[k] = __builtin_nontemporal_load(p + k * T);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < P; ++k) s += (r[k].x + r[k].y) + (r[k].z + r[k].w);
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (static_cast<int>(threadIdx.x) < wvec) {
    const vf4 v = {s, s, s, s};
    __builtin_nontemporal_store(v, dst + static_cast<size_t>(blockIdx.x) * wvec + threadIdx.x);
  }
}

template <int T, int P>
int32_t launch_rw(const void* src, void* dst, uint64_t bytes, int32_t wbytes, hipStream_t st) {
  const uint64_t tile = static_cast<uint64_t>(T) * P * 16;
  if (bytes == 0 || bytes % tile != 0 || bytes / tile > 0x7FFFFFFFull) return -2;
  if (wbytes <= 0 || wbytes % 16 != 0 || wbytes > T * 16) return -5;
  read_write_tiles<T, P><<<static_cast<unsigned>(bytes / tile), T, 0, st>>>(static_cast<const vf4*>(src),
                                                                           static_cast<vf4*>(dst), wbytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
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

extern "C" int32_t rs_probe_read_write(const void* src, void* dst, uint64_t bytes, int32_t threads, int32_t per_thread,
                                       int32_t write_bytes, void* stream) {
  if (!src || !dst || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (threads == 256 && per_thread == 8) return launch_rw<256, 8>(src, dst, bytes, write_bytes, st);
  if (threads == 256 && per_thread == 4) return launch_rw<256, 4>(src, dst, bytes, write_bytes, st);
  if (threads == 128 && per_thread == 16) return launch_rw<128, 16>(src, dst, bytes, write_bytes, st);
  return -4;
}

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

// Variants of the read stream that move more bytes per workgroup or take
// another path into the compute unit; each sums its tile and writes one float
// per tile to out[tile], as read_tiles does.
typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16-byte global -> LDS direct loads (no registers hold the data in flight):
// wave w's k-th load fills LDS bytes [(k T + 64 w) 16, +1024), lane l the
// 16 bytes at +16 l, from the same addresses the register tile reads.
template <int T, int P>
__global__ __launch_bounds__(T) void read_tiles_lds(const vf4* __restrict__ src, float* __restrict__ out) {
  __shared__ vf4 buf[T * P];
  const vf4* p = src + static_cast<size_t>(blockIdx.x) * (T * P) + threadIdx.x;
  const int wave = static_cast<int>(threadIdx.x >> 6);
#pragma unroll
  for (int k = 0; k < P; ++k)
    __builtin_amdgcn_global_load_lds((gptr_t)(p + k * T), (lptr_t)(&buf[k * T + wave * 64]), 16, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const vf4 r = buf[k * T + threadIdx.x];
    s += (r.x + r.y) + (r.z + r.w);
  }
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
__device__ __forceinline__ float tile_sum(const vf4 (&r)[P]) {
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < P; ++k) s += (r[k].x + r[k].y) + (r[k].z + r[k].w);
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

// Persistent workgroups: workgroup g reads the tile pairs g, g + G, g + 2G,
// ... (G = gridDim.x; pair q = tiles 2q and 2q + 1), issuing both tiles of a
// pair before it sums the first, so no workgroup is launched per tile and two
// tiles per workgroup are in flight at a time. Nothing in flight is carried
// across iterations (the registers are reloaded each pair). Every workgroup
// leaves the loop once its pair index passes the last pair.
template <int T, int P>
__global__ __launch_bounds__(T) void read_tiles_persistent(const vf4* __restrict__ src, float* __restrict__ out,
                                                           unsigned npairs) {
  __shared__ float w[2][T / 64];
  for (unsigned q = blockIdx.x; q < npairs; q += gridDim.x) {
    const vf4* p0 = src + static_cast<size_t>(2 * q) * (T * P) + threadIdx.x;
    const vf4* p1 = p0 + T * P;
    vf4 r0[P], r1[P];
#pragma unroll
    for (int k = 0; k < P; ++k) r0[k] = __builtin_nontemporal_load(p0 + k * T);
#pragma unroll
    for (int k = 0; k < P; ++k) r1[k] = __builtin_nontemporal_load(p1 + k * T);
    __builtin_amdgcn_sched_barrier(0);   // both tiles issued before either is summed
    const float s0 = tile_sum<T, P>(r0);
    const float s1 = tile_sum<T, P>(r1);
    if ((threadIdx.x & 63) == 0) {
      w[0][threadIdx.x >> 6] = s0;
      w[1][threadIdx.x >> 6] = s1;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      float a = 0.0f;
      for (int i = 0; i < T / 64; ++i) a += w[threadIdx.x][i];
      out[2 * q + threadIdx.x] = a;
    }
    __syncthreads();
  }
}

template <int T, int P, bool PLAIN>
__global__ __launch_bounds__(T) void read_tiles_v(const vf4* __restrict__ src, float* __restrict__ out) {
  const vf4* p = src + static_cast<size_t>(blockIdx.x) * (T * P) + threadIdx.x;
  vf4 r[P];
#pragma unroll
  for (int k = 0; k < P; ++k) r[k] = PLAIN ? p[k * T] : __builtin_nontemporal_load(p + k * T);
  const float s = tile_sum<T, P>(r);
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
uint64_t tile_bytes() { return static_cast<uint64_t>(T) * P * 16; }

}  // namespace

extern "C" int32_t rs_probe_read_variant(const void* src, float* out, uint64_t bytes, int32_t variant,
                                         void* stream) {
  if (!src || !out || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const vf4* s = static_cast<const vf4*>(src);
  if (variant < RS_PROBE_REG_256X8 || variant > RS_PROBE_PERSISTENT_256X8) return -4;
  const uint64_t tb = variant == RS_PROBE_REG_256X16 || variant == RS_PROBE_LDS_256X16 ? tile_bytes<256, 16>()
                                                                                        : tile_bytes<256, 8>();
  if (bytes == 0 || bytes % tb != 0 || bytes / tb > 0x7FFFFFFFull) return -2;
  const unsigned n = static_cast<unsigned>(bytes / tb);
  if (variant == RS_PROBE_PERSISTENT_256X8 && n % 2 != 0) return -2;   // whole tile pairs
  switch (variant) {
    case RS_PROBE_REG_256X8: read_tiles_v<256, 8, false><<<n, 256, 0, st>>>(s, out); break;
    case RS_PROBE_PLAIN_256X8: read_tiles_v<256, 8, true><<<n, 256, 0, st>>>(s, out); break;
    case RS_PROBE_REG_256X16: read_tiles_v<256, 16, false><<<n, 256, 0, st>>>(s, out); break;
    case RS_PROBE_LDS_256X8: read_tiles_lds<256, 8><<<n, 256, 0, st>>>(s, out); break;
    case RS_PROBE_LDS_256X16: read_tiles_lds<256, 16><<<n, 256, 0, st>>>(s, out); break;
    case RS_PROBE_PERSISTENT_256X8: {
      // as many workgroups as fit on the chip at once, so none waits for a slot
      int dev = 0, cus = 0, per_cu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, read_tiles_persistent<256, 8>, 256, 0) !=
              hipSuccess || cus <= 0 || per_cu <= 0)
        return -3;
      const unsigned g = static_cast<unsigned>(cus) * static_cast<unsigned>(per_cu);
      read_tiles_persistent<256, 8><<<n / 2 < g ? n / 2 : g, 256, 0, st>>>(s, out, n / 2);
      break;
    }
    default: return -4;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

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

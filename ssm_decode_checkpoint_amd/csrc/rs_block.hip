// The Mamba-2 block's per-token work around the SSM step (Dao and Gu 2024):
// the short causal convolution over the concatenated x | B | C channels with
// its state kept as a ring of recent inputs, and the gated RMS norm of the SSM
// output.
//
// Convolution state. The decode state of a width-W causal convolution is the
// last W-1 inputs. They are kept in a 16-slot ring per sequence, input of
// absolute token position q in slot q mod 16, with the position taken from the
// SSM layer's counters (q = n_ckpt + len is the next committed position). Like
// the ReplaySSM buffer (sitech.ge ReplaySSM page, "Reducing state traffic and
// simplifying rollback"), drafts are written to the slots after the committed
// ones and a commit needs no work here: the SSM commit moves the position, and
// the slots of rejected drafts are overwritten later.
#include "rs_internal.h"

namespace rs {

namespace {

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// float -> bf16, round to nearest, ties to even (inputs here are finite)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// eight consecutive channels in the input type
template <typename TIN>
__device__ __forceinline__ void load8(const TIN* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename TIN>
__device__ __forceinline__ void store8(TIN* p, const float* v);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_rne(v[2 * i]) | (bf16_rne(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

// One thread per (sequence, 8 channels): the W-1 previous inputs from the
// ring, then for each of the K tokens the convolution, SiLU, the output into
// its x / B / C array and the input into the ring. Sequences whose SSM call
// will refuse the tokens (drafts pending, or no room for K entries) are left
// untouched, outputs included.
// UNI: a wavefront never straddles two sequences (chunks % 64 == 0), so the
// sequence index is wave-uniform and its counters are read through scalar
// loads, which do not queue behind the vector loads already in flight.
template <typename TIN, int W, bool UNI>
__global__ __launch_bounds__(kThreads) void conv_step_kernel(ConvArgs a) {
  const int chunks = a.channels / 8;
  const long long gid = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= static_cast<long long>(a.batch) * chunks) return;
  int b = static_cast<int>(gid / chunks);
  if constexpr (UNI) b = __builtin_amdgcn_readfirstlane(b);
  const int ch = static_cast<int>(gid - static_cast<long long>(b) * chunks) * 8;
  // weights, biases and the first token's input do not depend on the position:
  // their loads go out before the counters are read
  float wt[8 * W], bs[8], cur[8];
  load8(static_cast<const TIN*>(a.xbc) + static_cast<size_t>(b) * a.channels + ch, cur);
  const float4* wp = reinterpret_cast<const float4*>(a.w + static_cast<size_t>(ch) * W);
#pragma unroll
  for (int j = 0; j < 2 * W; ++j) {
    const float4 v = wp[j];
    wt[4 * j] = v.x; wt[4 * j + 1] = v.y; wt[4 * j + 2] = v.z; wt[4 * j + 3] = v.w;
  }
  if (a.bias) {
    const float4* bp = reinterpret_cast<const float4*>(a.bias + ch);
    const float4 b0 = bp[0], b1 = bp[1];
    bs[0] = b0.x; bs[1] = b0.y; bs[2] = b0.z; bs[3] = b0.w; bs[4] = b1.x; bs[5] = b1.y; bs[6] = b1.z; bs[7] = b1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) bs[i] = 0.0f;
  }
  const rs_meta* __restrict__ m = a.meta + b;
  const int len = m->len, nd = m->nd;
  if (nd != 0 || len + a.K > kRing) return;
  const long long p = m->n_ckpt + len;
  TIN* ring = static_cast<TIN*>(a.ring) + static_cast<size_t>(b) * kRing * a.channels + ch;
  float hist[W > 1 ? W - 1 : 1][8];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) load8(ring + ((p - (W - 1) + k) & (kRing - 1)) * a.channels, hist[k]);
  for (int d = 0; d < a.K; ++d) {
    const size_t row = static_cast<size_t>(d) * a.batch + b;
    const TIN* in = static_cast<const TIN*>(a.xbc) + row * a.channels + ch;
    float out[8];
    if (d > 0) load8(in, cur);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = bs[i];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) acc += wt[i * W + k] * hist[k][i];
      acc += wt[i * W + W - 1] * cur[i];
      out[i] = silu(acc);
    }
    TIN* dst;
    if (ch < a.d_inner) dst = static_cast<TIN*>(a.x) + row * a.d_inner + ch;
    else if (ch < a.d_inner + a.gn) dst = static_cast<TIN*>(a.B) + row * a.gn + (ch - a.d_inner);
    else dst = static_cast<TIN*>(a.C) + row * a.gn + (ch - a.d_inner - a.gn);
    store8(dst, out);
    store8(ring + ((p + d) & (kRing - 1)) * a.channels, cur);   // exact: cur holds input-type values
#pragma unroll
    for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) hist[k][i] = hist[k + 1][i];
    if constexpr (W > 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) hist[W - 2][i] = cur[i];
    }
  }
}

template <typename TIN>
void conv_step_t(const ConvArgs& a, hipStream_t st) {
  const long long threads = static_cast<long long>(a.batch) * (a.channels / 8);
  const int grid = static_cast<int>((threads + kThreads - 1) / kThreads);
  if ((a.channels / 8) % 64 == 0) {
    switch (a.width) {
      case 1: conv_step_kernel<TIN, 1, true><<<grid, kThreads, 0, st>>>(a); break;
      case 2: conv_step_kernel<TIN, 2, true><<<grid, kThreads, 0, st>>>(a); break;
      case 3: conv_step_kernel<TIN, 3, true><<<grid, kThreads, 0, st>>>(a); break;
      default: conv_step_kernel<TIN, 4, true><<<grid, kThreads, 0, st>>>(a); break;
    }
  } else {
    switch (a.width) {
      case 1: conv_step_kernel<TIN, 1, false><<<grid, kThreads, 0, st>>>(a); break;
      case 2: conv_step_kernel<TIN, 2, false><<<grid, kThreads, 0, st>>>(a); break;
      case 3: conv_step_kernel<TIN, 3, false><<<grid, kThreads, 0, st>>>(a); break;
      default: conv_step_kernel<TIN, 4, false><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
}

void conv_step(const ConvArgs& a, bool bf, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (bf) conv_step_t<bf16>(a, st);
  else conv_step_t<float>(a, st);
}

// Gated RMS norm: one wavefront per (row, channel group), four per workgroup.
// Each lane takes runs of 4 consecutive channels (16-byte y loads) and keeps
// v = y * silu(z) of up to kNormRuns runs in registers (groups up to
// 4 * 64 * kNormRuns channels; larger groups recompute v from the inputs,
// still in cache, in the second pass). Sum of squares by shuffles; then
// v / sqrt(mean + eps) * weight.
constexpr int kNormRuns = 8;

template <typename TIN>
__device__ __forceinline__ void load4(const TIN* p, float* v);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <>
__device__ __forceinline__ void load4<bf16>(const bf16* p, float* v) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
template <typename TIN>
__device__ __forceinline__ void store4(TIN* p, const float* v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float* v) {
  *reinterpret_cast<uint2*>(p) =
      make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
}

template <typename TIN>
__global__ __launch_bounds__(kThreads) void gated_norm_kernel(NormArgs a) {
  const int ng = a.d / a.gs;
  const long long item = static_cast<long long>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (item >= static_cast<long long>(a.rows) * ng) return;   // whole wavefronts leave together
  const int row = static_cast<int>(item / ng), g = static_cast<int>(item - static_cast<long long>(row) * ng);
  const int lane = threadIdx.x & 63;
  const size_t base = static_cast<size_t>(row) * a.d + static_cast<size_t>(g) * a.gs;
  const TIN* z = static_cast<const TIN*>(a.z) + base;
  const float* y = a.y + base;
  const float* wt = a.w + static_cast<size_t>(g) * a.gs;
  TIN* out = static_cast<TIN*>(a.out) + base;
  const int runs = a.gs / 4;                      // runs of 4 channels, lane takes runs lane, lane + 64, ...
  float v[kNormRuns][4];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormRuns; ++j) {
    const int r = lane + 64 * j;
    if (r < runs) {
      float yv[4], zv[4];
      load4(y + 4 * r, yv);
      load4(z + 4 * r, zv);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[j][k] = yv[k] * silu(zv[k]);
        ss += v[j][k] * v[j][k];
      }
    }
  }
  for (int r = lane + 64 * kNormRuns; r < runs; r += 64) {
    float yv[4], zv[4];
    load4(y + 4 * r, yv);
    load4(z + 4 * r, zv);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float t = yv[k] * silu(zv[k]);
      ss += t * t;
    }
  }
  ss = wave_sum_stride<1>(ss);
  const float rs_ = 1.0f / sqrtf(ss / static_cast<float>(a.gs) + a.eps);
#pragma unroll
  for (int j = 0; j < kNormRuns; ++j) {
    const int r = lane + 64 * j;
    if (r < runs) {
      float wv[4], o[4];
      load4(wt + 4 * r, wv);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = v[j][k] * rs_ * wv[k];
      store4(out + 4 * r, o);
    }
  }
  for (int r = lane + 64 * kNormRuns; r < runs; r += 64) {
    float yv[4], zv[4], wv[4], o[4];
    load4(y + 4 * r, yv);
    load4(z + 4 * r, zv);
    load4(wt + 4 * r, wv);
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = yv[k] * silu(zv[k]) * rs_ * wv[k];
    store4(out + 4 * r, o);
  }
}

void gated_norm(const NormArgs& a, bool bf, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long items = static_cast<long long>(a.rows) * (a.d / a.gs);
  const int grid = static_cast<int>((items + kThreads / 64 - 1) / (kThreads / 64));
  if (bf) gated_norm_kernel<bf16><<<grid, kThreads, 0, st>>>(a);
  else gated_norm_kernel<float><<<grid, kThreads, 0, st>>>(a);
}

}  // namespace rs

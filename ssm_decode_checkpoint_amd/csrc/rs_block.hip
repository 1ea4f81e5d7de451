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

// raw copy of eight channels (the ring keeps the inputs bit for bit)
template <typename TIN>
__device__ __forceinline__ void copy8(TIN* dst, const TIN* src) {
  constexpr int N = static_cast<int>(sizeof(TIN)) * 8 / 16;
#pragma unroll
  for (int i = 0; i < N; ++i) reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
}

}  // namespace

// One thread per (sequence, 8 channels): the W-1 previous inputs from the
// ring, then for each of the K tokens the convolution, SiLU, the output into
// its x / B / C array and the input into the ring. Sequences whose SSM call
// will refuse the tokens (drafts pending, or no room for K entries) are left
// untouched, outputs included.
template <typename TIN, int W>
__global__ __launch_bounds__(kThreads) void conv_step_kernel(ConvArgs a) {
  const int chunks = a.channels / 8;
  const long long gid = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= static_cast<long long>(a.batch) * chunks) return;
  const int b = static_cast<int>(gid / chunks);
  const int ch = static_cast<int>(gid - static_cast<long long>(b) * chunks) * 8;
  const rs_meta* m = a.meta + b;
  const int len = m->len, nd = m->nd;
  if (nd != 0 || len + a.K > kRing) return;
  const long long p = m->n_ckpt + len;
  float wt[8][W], bs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int k = 0; k < W; ++k) wt[i][k] = a.w[(ch + i) * W + k];
    bs[i] = a.bias ? a.bias[ch + i] : 0.0f;
  }
  TIN* ring = static_cast<TIN*>(a.ring) + static_cast<size_t>(b) * kRing * a.channels + ch;
  float hist[W > 1 ? W - 1 : 1][8];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) load8(ring + ((p - (W - 1) + k) & (kRing - 1)) * a.channels, hist[k]);
  for (int d = 0; d < a.K; ++d) {
    const size_t row = static_cast<size_t>(d) * a.batch + b;
    const TIN* in = static_cast<const TIN*>(a.xbc) + row * a.channels + ch;
    float cur[8], out[8];
    load8(in, cur);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = bs[i];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) acc += wt[i][k] * hist[k][i];
      acc += wt[i][W - 1] * cur[i];
      out[i] = silu(acc);
    }
    TIN* dst;
    if (ch < a.d_inner) dst = static_cast<TIN*>(a.x) + row * a.d_inner + ch;
    else if (ch < a.d_inner + a.gn) dst = static_cast<TIN*>(a.B) + row * a.gn + (ch - a.d_inner);
    else dst = static_cast<TIN*>(a.C) + row * a.gn + (ch - a.d_inner - a.gn);
    store8(dst, out);
    copy8(ring + ((p + d) & (kRing - 1)) * a.channels, in);
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
  switch (a.width) {
    case 1: conv_step_kernel<TIN, 1><<<grid, kThreads, 0, st>>>(a); break;
    case 2: conv_step_kernel<TIN, 2><<<grid, kThreads, 0, st>>>(a); break;
    case 3: conv_step_kernel<TIN, 3><<<grid, kThreads, 0, st>>>(a); break;
    default: conv_step_kernel<TIN, 4><<<grid, kThreads, 0, st>>>(a); break;
  }
}

void conv_step(const ConvArgs& a, bool bf, hipStream_t st) {
  if (bf) conv_step_t<bf16>(a, st);
  else conv_step_t<float>(a, st);
}

// Gated RMS norm: one workgroup per (row, channel group). First pass: the sum
// of squares of v = y * silu(z); second pass recomputes v (the group's inputs
// are still in cache) and writes v / sqrt(mean + eps) * weight.
template <typename TIN>
__global__ __launch_bounds__(kThreads) void gated_norm_kernel(NormArgs a) {
  __shared__ float part[kThreads / 64];
  const int ng = a.d / a.gs;
  const int row = blockIdx.x / ng, g = blockIdx.x - row * ng;
  const size_t base = static_cast<size_t>(row) * a.d + static_cast<size_t>(g) * a.gs;
  const TIN* z = static_cast<const TIN*>(a.z) + base;
  const float* y = a.y + base;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < a.gs; i += kThreads) {
    const float v = y[i] * silu(to_f(z[i]));
    ss += v * v;
  }
  ss = wave_sum_stride(ss, 1);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
  const float r = 1.0f / sqrtf(tot / static_cast<float>(a.gs) + a.eps);
  const float* wt = a.w + static_cast<size_t>(g) * a.gs;
  TIN* out = static_cast<TIN*>(a.out) + base;
  for (int i = threadIdx.x; i < a.gs; i += kThreads) {
    const float v = y[i] * silu(to_f(z[i])) * r * wt[i];
    if constexpr (sizeof(TIN) == 2) out[i] = bf16{static_cast<uint16_t>(bf16_rne(v))};
    else out[i] = v;
  }
}

void gated_norm(const NormArgs& a, bool bf, hipStream_t st) {
  const int grid = a.rows * (a.d / a.gs);
  if (bf) gated_norm_kernel<bf16><<<grid, kThreads, 0, st>>>(a);
  else gated_norm_kernel<float><<<grid, kThreads, 0, st>>>(a);
}

}  // namespace rs

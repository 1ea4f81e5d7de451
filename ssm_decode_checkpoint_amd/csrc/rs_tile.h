// Workgroup-level state-tile routines shared by the Mamba-2 and Gated DeltaNet
// kernels: load a stored matrix into registers, reduce it against vectors,
// round it to a checkpoint format, and store it (with the per-matrix and
// per-block scales that format needs).
#pragma once

#include "rs_device.h"

namespace rs {

// A stored rows x cols matrix held by one 256-thread workgroup:
// v[k][i] = M[row(k)][col0() + i] with c = tid % TPR, row(k) = tid / TPR + k*RPP.
// Rows past the matrix hold zeros.
template <int E, int NR, int NC>
struct RegTile {
  using TM = TileMap<E, NR, NC>;
  static constexpr int P = TM::PASSES;
  float v[P][E];

  __device__ __forceinline__ static int col0() { return static_cast<int>(threadIdx.x % TM::TPR) * E; }
  __device__ __forceinline__ static int row(int k) { return static_cast<int>(threadIdx.x / TM::TPR) + k * TM::RPP; }
};

template <int FMT, int E, int NR, int NC>
struct RawTile {
  using TM = TileMap<E, NR, NC>;
  Raw<FMT, E> r[TM::PASSES];
  float ms;

  // Every thread issues all its loads unconditionally (rows past a matrix
  // smaller than one pass are clamped to its last row and ignored when
  // decoding): loads under a branch would be merged through a wait, which
  // serialises the stream. The scheduling barrier keeps every load written
  // before the tile (the buffer records) ahead of it: returns come back in
  // issue order, so a record load moved behind the tile would wait for all of it.
  __device__ __forceinline__ void issue(const StateBuf& sb, size_t mat) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      int row = static_cast<int>(threadIdx.x / TM::TPR) + k * TM::RPP;
      if constexpr (NR % TM::RPP != 0 || TM::RPP > NR) row = row < NR ? row : NR - 1;
      r[k] = load_chunk<FMT, E, NC>(sb, mat, NR, row, static_cast<int>(threadIdx.x % TM::TPR));
    }
    ms = mat_scale<FMT>(sb, mat);
  }
  __device__ __forceinline__ void decode(RegTile<E, NR, NC>& dst, float mult = 1.0f) const {
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = static_cast<int>(threadIdx.x / TM::TPR) + k * TM::RPP;
      float t[E];
      decode_chunk<FMT, E>(r[k], ms, t);
      const bool in = (NR % TM::RPP == 0 && TM::RPP <= NR) || row < NR;
#pragma unroll
      for (int i = 0; i < E; ++i) dst.v[k][i] = in ? t[i] * mult : 0.0f;
    }
  }
};

// out[q][col] = sum_rows M[row][col] * w[q*ws + row] for Q weight vectors in
// LDS. `red` is LDS scratch of 4*Q*NC floats; `out` is LDS of Q*NC floats.
// Contains workgroup barriers; all threads must call.
template <int Q, int E, int NR, int NC>
__device__ __forceinline__ void tile_matvec(const RegTile<E, NR, NC>& M, const float* w, int ws, float* red,
                                            float* out) {
  using TM = TileMap<E, NR, NC>;
  float acc[Q][E];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < E; ++i) acc[q][i] = 0.0f;
#pragma unroll
  for (int k = 0; k < TM::PASSES; ++k) {
    const int row = static_cast<int>(threadIdx.x / TM::TPR) + k * TM::RPP;
    if (row < NR) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float wr = w[q * ws + row];
#pragma unroll
        for (int i = 0; i < E; ++i) acc[q][i] += M.v[k][i] * wr;
      }
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < E; ++i) acc[q][i] = wave_sum_stride<TM::TPR>(acc[q][i]);
  if (lane < TM::TPR) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < E; ++i) red[(wave * Q + q) * NC + lane * E + i] = acc[q][i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < Q * NC; idx += kThreads) {
    out[idx] = (red[idx] + red[Q * NC + idx]) + (red[2 * Q * NC + idx] + red[3 * Q * NC + idx]);
  }
  __syncthreads();
}

// out[t][col] = sum_rows M_t[row][col] * w[row] for T held matrices and one
// LDS weight vector; `red` is 4*T*NC floats of LDS, `out` T*NC. Barriers inside.
template <int T, int E, int NR, int NC>
__device__ __forceinline__ void tiles_matvec(const RegTile<E, NR, NC> (&M)[T], const float* w, float* red,
                                             float* out) {
  using TM = TileMap<E, NR, NC>;
  float acc[T][E];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < E; ++i) acc[t][i] = 0.0f;
#pragma unroll
  for (int k = 0; k < TM::PASSES; ++k) {
    const int row = static_cast<int>(threadIdx.x / TM::TPR) + k * TM::RPP;
    if (row < NR) {
      const float wr = w[row];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < E; ++i) acc[t][i] += M[t].v[k][i] * wr;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < E; ++i) acc[t][i] = wave_sum_stride<TM::TPR>(acc[t][i]);
  if (lane < TM::TPR) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < E; ++i) red[(wave * T + t) * NC + lane * E + i] = acc[t][i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * NC; idx += kThreads) {
    out[idx] = (red[idx] + red[T * NC + idx]) + (red[2 * T * NC + idx] + red[3 * T * NC + idx]);
  }
  __syncthreads();
}

// Workgroup max of |M|; every thread gets it. Contains barriers.
template <int E, int NR, int NC>
__device__ __forceinline__ float tile_absmax(const RegTile<E, NR, NC>& M, float* scratch4) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < RegTile<E, NR, NC>::P; ++k)
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(M.v[k][i]));
  m = wave_max(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch4[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(scratch4[0], scratch4[1]), fmaxf(scratch4[2], scratch4[3]));
}

// ----------------------------------------------------------------------------
// Encoders. Each element is divided by its scale first (correctly rounded, the
// order the format definitions use), the quotient is clamped to the format's
// largest finite magnitude (saturation: the E4M3FN conversion instruction would
// give the NaN code above about 464), then converted by gfx950's packed
// conversion at unit scale, which rounds to nearest with ties to even.
// ----------------------------------------------------------------------------
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float clamp_mag(float q, float m) { return fminf(fmaxf(q, -m), m); }

// The correctly rounded quotient x / d from y = RN(1/d), by Markstein's
// correction step (Markstein 1990; Muller et al., Handbook of Floating-Point
// Arithmetic): q = RN(x y) is within one ulp of x / d, the remainder x - d q is
// exact by FMA, and RN(q + (x - d q) y) = RN(x / d) when neither 1/d nor the
// quotient overflows or underflows. The remainder is formed negated, t = q d -
// x, and subtracted, RN(q - t y): the same value, and a zero quotient keeps
// the sign of x as the division gives it (for x = -0, q = -0 and t = +0, so
// -0 - (+0) y = -0; with the remainder added instead, +0 + -0 would give
// +0). Below the scale kRecipMin the callers divide: there 1/d could
// overflow. Subnormal quotients (|x / d| < 2^-126) cannot change a code.
constexpr float kRecipMin = 0x1p-125f;

// q[i] = RN(x[i] / d) for i < N, with y = RN(1/d) when d >= kRecipMin. The
// choice between the correction step and the division depends on d alone, so
// it is taken once for all N quotients (those sharing a scale).
template <int N>
__device__ __forceinline__ void quot_n(const float* x, float d, float y, float* q) {
  if (d >= kRecipMin) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float q0 = x[i] * y;
      const float t = fmaf(q0, d, -x[i]);
      q[i] = fmaf(-t, y, q0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = x[i] / d;
  }
}

// E4M3FN codes of x[0..N) / sc, element i in byte i of w (N a multiple of 4;
// y = RN(1/sc)), for a matrix scale sc = RN(amax / 448) of the same values:
// then |x / sc| <= 448 (1 + 2^-23) and its correctly rounded quotient stays far
// below 464, where the conversion would give the NaN code, and rounds to 448
// at most, as saturation would; so the quotients need no clamp.
template <int N>
__device__ __forceinline__ void fp8_codes(const float* x, float sc, float y, uint32_t* w) {
  float q[N];
  quot_n<N>(x, sc, y, q);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    s16x2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, q[4 * i], q[4 * i + 1], 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, q[4 * i + 2], q[4 * i + 3], 1.0f, true);
    w[i] = static_cast<uint32_t>(static_cast<uint16_t>(r.x)) | (static_cast<uint32_t>(static_cast<uint16_t>(r.y)) << 16);
  }
}

// E4M3FN code of a non-negative quotient q (an NVFP4 block scale).
__device__ __forceinline__ uint32_t e4m3_code_of(float q) {
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(q, 448.0f), 0.0f, 1.0f, false);
  return static_cast<uint32_t>(r.x) & 0xFFu;
}

// E2M1 codes of x[0..N) / sd (one block scale), element i in nibble i of w
// (N a multiple of 8; all 0 when sd = 0). One correctly rounded division per
// call gives the reciprocal.
template <int N>
__device__ __forceinline__ void nvfp4_codes(const float* x, float sd, uint32_t* w) {
  float q[N];
  quot_n<N>(x, sd, 1.0f / sd, q);
#pragma unroll
  for (int j = 0; j < N / 8; ++j) {
    const float* p = q + 8 * j;
    uint32_t v = 0u;
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(p[0], 6.0f), clamp_mag(p[1], 6.0f), 1.0f, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(p[2], 6.0f), clamp_mag(p[3], 6.0f), 1.0f, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(p[4], 6.0f), clamp_mag(p[5], 6.0f), 1.0f, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(p[6], 6.0f), clamp_mag(p[7], 6.0f), 1.0f, 3);
    w[j] = sd == 0.0f ? 0u : v;
  }
}

__device__ __forceinline__ float fp8_scale_of(float amax) {
  const float sc = amax / 448.0f;
  return sc == 0.0f ? 1.0f : sc;
}

__device__ __forceinline__ float nvfp4_tscale_of(float amax) {
  const float ts = amax / 2688.0f;
  return ts == 0.0f ? 1.0f : ts;
}

// NVFP4 block scale code of a block of sixteen columns held E per thread by
// 16 / E neighbouring lanes (E = 8: a lane pair; E = 4: a quad), which
// exchange their parts' maxima.
template <int E = 8>
__device__ __forceinline__ uint32_t nvfp4_block_code(const float* x, float ts) {
  static_assert(E == 4 || E == 8, "eight or four columns per thread");
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) bm = fmaxf(bm, fabsf(x[i]));
  bm = fmaxf(bm, dpp_mov<kDppXor1>(bm));
  if constexpr (E == 4) bm = fmaxf(bm, dpp_mov<kDppXor2>(bm));
  return e4m3_code_of(bm / (6.0f * ts));
}

// E2M1 codes of four values x[0..4) / sd in the low 16 bits (element i in
// nibble i; 0 when sd = 0), with the arithmetic of nvfp4_codes.
__device__ __forceinline__ uint32_t nvfp4_codes4(const float* x, float sd) {
  float q[4];
  quot_n<4>(x, sd, 1.0f / sd, q);
  uint32_t v = 0u;
  v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(q[0], 6.0f), clamp_mag(q[1], 6.0f), 1.0f, 0);
  v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, clamp_mag(q[2], 6.0f), clamp_mag(q[3], 6.0f), 1.0f, 1);
  return sd == 0.0f ? 0u : (v & 0xFFFFu);
}

// Replace M by the value it reads back as after being stored in FMT (scales
// computed from M itself, as tile_store does). All threads must call.
template <int FMT, int E, int NR, int NC>
__device__ __forceinline__ void tile_round_trip(RegTile<E, NR, NC>& M, float* scratch4) {
  if constexpr (FMT == FMT_F16) {
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k)
#pragma unroll
      for (int i = 0; i < E; ++i) M.v[k][i] = __half2float(__float2half_rn(M.v[k][i]));
  } else if constexpr (FMT == FMT_FP8) {
    static_assert(E == 8, "fp8 state chunks are eight elements");
    const float sc = fp8_scale_of(tile_absmax(M, scratch4));
    const float y = 1.0f / sc;
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
      Raw<FMT_FP8, 8> r;
      uint32_t w[2];
      fp8_codes<8>(M.v[k], sc, y, w);
      r.v = make_uint2(w[0], w[1]);
      decode_chunk<FMT_FP8, 8>(r, sc, M.v[k]);
    }
  } else if constexpr (FMT == FMT_NVFP4) {
    static_assert(E == 8, "NVFP4 blocks span two threads of eight columns");
    const float ts = nvfp4_tscale_of(tile_absmax(M, scratch4));
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
      Raw<FMT_NVFP4, 8> r;
      r.s = nvfp4_block_code(M.v[k], ts);
      nvfp4_codes<8>(M.v[k], e4m3_value(r.s) * ts, &r.v);
      decode_chunk<FMT_NVFP4, 8>(r, ts, M.v[k]);
    }
  }
}

template <int E, int NR, int NC>
__device__ __forceinline__ void tile_store_nvfp4(const StateBuf& sb, size_t mat, const RegTile<E, NR, NC>& M,
                                                 float amax);

// Store M into sb in format FMT. FP8 and NVFP4 compute their scales from M.
// All threads must call.
template <int FMT, int E, int NR, int NC>
__device__ __forceinline__ void tile_store(const StateBuf& sb, size_t mat, const RegTile<E, NR, NC>& M,
                                           float* scratch4) {
  using TM = TileMap<E, NR, NC>;
  const int c = static_cast<int>(threadIdx.x % TM::TPR);
  if constexpr (FMT == FMT_F32) {
    float* base = static_cast<float*>(sb.data) + mat * NR * NC;
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = RegTile<E, NR, NC>::row(k);
      if (row < NR) {
        float4* dst = reinterpret_cast<float4*>(base + row * NC + c * E);
        nt_store(make_float4(M.v[k][0], M.v[k][1], M.v[k][2], M.v[k][3]), dst);
        if constexpr (E == 8)
          nt_store(make_float4(M.v[k][4], M.v[k][5], M.v[k][6], M.v[k][7]), dst + 1);
      }
    }
  } else if constexpr (FMT == FMT_F16) {
    static_assert(E == 8, "fp16 state chunks are eight elements");
    __half* base = static_cast<__half*>(sb.data) + mat * NR * NC;
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = RegTile<E, NR, NC>::row(k);
      if (row < NR) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = __half_as_ushort(__float2half_rn(M.v[k][2 * i]));
          const uint32_t hi = __half_as_ushort(__float2half_rn(M.v[k][2 * i + 1]));
          w[i] = lo | (hi << 16);
        }
        nt_store(make_uint4(w[0], w[1], w[2], w[3]),
                                    reinterpret_cast<uint4*>(base + row * NC + c * E));
      }
    }
  } else if constexpr (FMT == FMT_FP8) {
    static_assert(E == 8, "fp8 state chunks are eight elements");
    const float sc = fp8_scale_of(tile_absmax(M, scratch4));
    const float y = 1.0f / sc;
    uint8_t* base = static_cast<uint8_t*>(sb.data) + mat * NR * NC;
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = RegTile<E, NR, NC>::row(k);
      if (row < NR) {
        uint32_t w[2];
        fp8_codes<8>(M.v[k], sc, y, w);
        nt_store(make_uint2(w[0], w[1]), reinterpret_cast<uint2*>(base + row * NC + c * E));
      }
    }
    if (threadIdx.x == 0) sb.tscale[mat] = sc;
  } else {
    tile_store_nvfp4(sb, mat, M, tile_absmax(M, scratch4));
  }
}

// NVFP4 store of M whose matrix |max| is amax (already reduced: no barrier here).
template <int E, int NR, int NC>
__device__ __forceinline__ void tile_store_nvfp4(const StateBuf& sb, size_t mat, const RegTile<E, NR, NC>& M,
                                                 float amax) {
  using TM = TileMap<E, NR, NC>;
  static_assert(E == 8 || E == 4, "NVFP4 blocks span two threads of eight columns or four of four");
  const int c = static_cast<int>(threadIdx.x % TM::TPR);
  const float ts = nvfp4_tscale_of(amax);
  uint8_t* base = static_cast<uint8_t*>(sb.data) + mat * NR * NC / 2;
  uint8_t* sbase = sb.nv_scale + mat * NR * NC / 16;
#pragma unroll
  for (int k = 0; k < TM::PASSES; ++k) {
    const int row = RegTile<E, NR, NC>::row(k);
    const uint32_t s = nvfp4_block_code<E>(M.v[k], ts);
    const float sd = e4m3_value(s) * ts;
    if constexpr (E == 8) {
      uint32_t w;
      nvfp4_codes<8>(M.v[k], sd, &w);
      if (row < NR) {
        nt_store(w, reinterpret_cast<uint32_t*>(base + (row * NC + c * 8) / 2));
        if ((c & 1) == 0) sbase[(row * NC + c * 8) / 16] = static_cast<uint8_t>(s);
      }
    } else {
      const uint32_t w = nvfp4_codes4(M.v[k], sd);
      if (row < NR) {
        *reinterpret_cast<uint16_t*>(base + (row * NC + c * 4) / 2) = static_cast<uint16_t>(w);
        if ((c & 3) == 0) sbase[(row * NC + c * 4) / 16] = static_cast<uint8_t>(s);
      }
    }
  }
  if (threadIdx.x == 0) sb.tscale[mat] = ts;
}

// H <- L*H + sum_{e<m} row[e][r] * col[e][c]: a rank-m update of the held
// matrix from LDS vectors (row: m x NR, stride rs; col: m x NC, stride cs),
// accumulated in entry order. No barriers.
template <int E, int NR, int NC>
__device__ __forceinline__ void tile_rank_update(RegTile<E, NR, NC>& H, float L, const float* row, int rs,
                                                 const float* col, int cs, int m) {
  const int c0 = RegTile<E, NR, NC>::col0();
#pragma unroll
  for (int k = 0; k < RegTile<E, NR, NC>::P; ++k)
#pragma unroll
    for (int i = 0; i < E; ++i) H.v[k][i] *= L;
  for (int e = 0; e < m; ++e) {
    float xc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) xc[i] = col[e * cs + c0 + i];
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
      const int r = RegTile<E, NR, NC>::row(k);
      if (r < NR) {
        const float br = row[e * rs + r];
#pragma unroll
        for (int i = 0; i < E; ++i) H.v[k][i] += br * xc[i];
      }
    }
  }
}

// The 16 / sizeof(T) floats at src as 16 bytes of T. Exact for values that
// came from T (bf16 keeps the upper half of the float's bits).
template <typename T>
__device__ __forceinline__ uint4 pack16(const float* src) {
  if constexpr (sizeof(T) == 4) {
    return make_uint4(__float_as_uint(src[0]), __float_as_uint(src[1]), __float_as_uint(src[2]),
                      __float_as_uint(src[3]));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (__float_as_uint(src[2 * k]) >> 16) | (__float_as_uint(src[2 * k + 1]) & 0xFFFF0000u);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Write n LDS floats that came from T back to a global T row (exact), 16 bytes
// per lane where the length allows (n % (16/sizeof(T)) == 0, dst 16-byte aligned).
template <typename T>
__device__ __forceinline__ void store_row_as(T* dst, const float* src, int n) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  if (n % V != 0) {
    for (int i = threadIdx.x; i < n; i += kThreads) dst[i] = from_f<T>(src[i]);
  } else {
    for (int i = threadIdx.x; i < n / V; i += kThreads) reinterpret_cast<uint4*>(dst)[i] = pack16<T>(src + V * i);
  }
}

// Rows r = 0..nrows-1 of n floats each (LDS, src + r * sstride) that came from
// T, to global T rows at dst + slot(r) * n, as one pass of 16-byte stores over
// all threads (n % (16/sizeof(T)) == 0, rows 16-byte aligned).
template <typename T, typename SLOT>
__device__ __forceinline__ void store_rows_as(T* dst, const float* src, int sstride, int nrows, int n, SLOT slot) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  const int per = n / V;
  for (int i = threadIdx.x; i < nrows * per; i += kThreads) {
    const int r = i / per, c = i - r * per;
    *reinterpret_cast<uint4*>(dst + static_cast<size_t>(slot(r)) * n + c * V) = pack16<T>(src + r * sstride + c * V);
  }
}

// Copy nrows rows of n T elements from global src (row r at src + r * sstride)
// to global dst rows (row r at dst + slot(r) * dstride), 16 bytes per lane over
// all threads (n % (16/sizeof(T)) == 0, rows 16-byte aligned).
template <typename T, typename SLOT>
__device__ __forceinline__ void copy_rows16(T* dst, size_t dstride, const T* src, size_t sstride, int nrows, int n,
                                            SLOT slot) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  const int per = n / V;
  for (int i = threadIdx.x; i < nrows * per; i += kThreads) {
    const int r = i / per, c = i - r * per;
    *reinterpret_cast<uint4*>(dst + static_cast<size_t>(slot(r)) * dstride + c * V) =
        *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r) * sstride + c * V);
  }
}

// Stream n floats from LDS to global with 16-byte non-temporal stores
// (n % 4 == 0, dst 16-byte aligned).
__device__ __forceinline__ void store_rows_nt(float* dst, const float* src, int n) {
  for (int i = threadIdx.x; i < n / 4; i += kThreads)
    nt_store(make_float4(src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]), reinterpret_cast<float4*>(dst) + i);
}

// Where buffer entry e of the current window comes from: the ring (e < nring)
// or a token array (entries nring.. come from `tok` stacked with stride tstride).
template <typename TIN>
struct EntrySrc {
  const TIN* ring;      // this sequence/head (or group) ring base: [kRing][len]
  const TIN* tok;       // first new token's record
  size_t tstride;       // elements between consecutive new tokens
  long long nck;        // n_ckpt
  int nring;            // entries held in the ring
  int width;            // record length
  __device__ __forceinline__ const TIN* at(int e) const {
    return e < nring ? ring + static_cast<size_t>((nck + e) & (kRing - 1)) * width
                     : tok + static_cast<size_t>(e - nring) * tstride;
  }
};

// 16-byte chunk of input elements -> floats
__device__ __forceinline__ void unpack16(const uint4& u, const float*, float* d) {
  d[0] = __uint_as_float(u.x); d[1] = __uint_as_float(u.y); d[2] = __uint_as_float(u.z); d[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack16(const uint4& u, const bf16*, float* d) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[2 * i] = __uint_as_float(w[i] << 16);
    d[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Up to CH 16-byte chunks per thread of a record region, loaded into registers.
template <typename TIN, int CH>
struct RegChunks {
  uint4 c[CH];
  // region of n records of `width` elements: record e comes from src(e)
  template <typename SRC>
  __device__ __forceinline__ void load(const SRC& src, int n, int width) {
    constexpr int V = 16 / static_cast<int>(sizeof(TIN));
    const int per = width / V;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      int q = static_cast<int>(threadIdx.x) + r * kThreads;
      q = q < n * per ? q : 0;   // unconditional load from a valid record (n >= 1)
      const int e = q / per, k = q - e * per;
      c[r] = *reinterpret_cast<const uint4*>(src.at(e) + k * V);
    }
  }
  __device__ __forceinline__ void to_lds(float* dst, int stride, int n, int width) const {
    constexpr int V = 16 / static_cast<int>(sizeof(TIN));
    const int per = width / V;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int q = static_cast<int>(threadIdx.x) + r * kThreads;
      if (q < n * per) {
        const int e = q / per, k = q - e * per;
        float t[V];
        unpack16(c[r], static_cast<const TIN*>(nullptr), t);
#pragma unroll
        for (int i = 0; i < V; ++i) dst[e * stride + k * V + i] = t[i];
      }
    }
  }
};

}  // namespace rs

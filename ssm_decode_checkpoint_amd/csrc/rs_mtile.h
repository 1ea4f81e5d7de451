// State tile in the matrix-core accumulator layout, for the rank-m fold.
//
// The flush folds the buffered entries into the checkpoint with one rank-m
// update, m <= 16 (sitech.ge ReplaySSM page, "How ReplaySSM works": the
// buffer is folded into the checkpoint once per window):
//   M[n][p] <- L * M[n][p] + sum_e rowv_e[n] * colv_e[p]
// over the stored rows x cols matrix (Mamba-2: rows = dstate n, cols = headdim
// p, rowv_e = B_e, colv_e = w_e dt_e x_e). That is a (cols x m) . (m x rows)
// product accumulated onto M^T, which v_mfma_f32_16x16x4f32 computes in
// 16 x 16 blocks, four entries per instruction, in fp32.
//
// Layout. Instruction operands and result, lane l (checked in the GDN matvec
// against a host product): A[l % 16][l / 16], B[l / 16][l % 16], result rows
// 4 (l / 16) + i, column l % 16. The result's columns index matrix rows n:
// wavefront w owns rows 16 (RB w + r) + l % 16, r < RB = rows / 64. The
// result's rows index matrix columns: lane l holds, in each 64-column group
// q of its row, the 16 consecutive columns 64 q + 16 (l / 16) .. + 15, so its
// element k = 4 cb + i is the instruction block cb's result row 4 (l / 16) + i
// (which fixes the A operand's column map, colv_col below). The four lanes
// l / 16 = 0..3 of a row cover 64 consecutive columns: one load or store
// instruction moves 64 contiguous bytes of each of 16 rows of an fp8 state,
// and each lane's 16 columns are exactly one NVFP4 block, whose scale is then
// lane-local. (An fp32 state in this layout moves 16-byte pieces of 64-byte
// row segments per instruction; its flush stays on the streaming layout.)
#pragma once

#include <type_traits>

#include "rs_device.h"
#include "rs_tile.h"

namespace rs {

typedef float mf32x4 __attribute__((ext_vector_type(4)));

template <int NR, int NC>
struct MTile {
  static_assert(NR % 64 == 0 && NC % 64 == 0, "rows: 16 per wavefront block; cols: groups of 64");
  static constexpr int RB = NR / 64;   // row blocks per wavefront
  static constexpr int CG = NC / 64;   // 64-column groups
  mf32x4 v[RB][CG][4];                 // v[r][q][k / 4][k % 4]: element k of row(r), group q

  __device__ __forceinline__ static int row(int r) {
    return 16 * (RB * static_cast<int>(threadIdx.x >> 6) + r) + static_cast<int>(threadIdx.x & 15);
  }
  // first of the lane's 16 columns in group q
  __device__ __forceinline__ static int col(int q) { return 64 * q + 16 * static_cast<int>((threadIdx.x >> 4) & 3); }
  // column of the A-operand element this lane supplies for block cb of group q:
  // the element 4 cb + i % 4 of the lanes with l / 16 = i / 4 (i = l % 16, the
  // operand's row, a result row)
  __device__ __forceinline__ static int colv_col(int q, int cb) {
    const int i = static_cast<int>(threadIdx.x & 15);
    return 64 * q + 16 * (i >> 2) + 4 * cb + (i & 3);
  }
  __device__ __forceinline__ float at(int r, int q, int k) const { return v[r][q][k >> 2][k & 3]; }
  __device__ __forceinline__ void set(int r, int q, int k, float x) { v[r][q][k >> 2][k & 3] = x; }
};

// ----------------------------------------------------------------------------
// 16-element row chunks in a stored format
// ----------------------------------------------------------------------------
template <int FMT>
constexpr int kChunkBytes = FMT == FMT_F32 ? 64 : FMT == FMT_F16 ? 32 : FMT == FMT_FP8 ? 16 : 8;

template <int N>
struct Bytes {
  uint32_t w[N / 4];
};

template <int N>
__device__ __forceinline__ void store_bytes(const Bytes<N>& b, void* p) {
  if constexpr (N == 8) {
    nt_store(make_uint2(b.w[0], b.w[1]), static_cast<uint2*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < N / 16; ++i)
      nt_store(make_uint4(b.w[4 * i], b.w[4 * i + 1], b.w[4 * i + 2], b.w[4 * i + 3]), static_cast<uint4*>(p) + i);
  }
}

template <int N>
__device__ __forceinline__ Bytes<N> load_bytes(const void* p) {
  Bytes<N> b;
  if constexpr (N == 8) {
    const uint2 u = nt_load(static_cast<const uint2*>(p));
    b.w[0] = u.x; b.w[1] = u.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const uint4 u = nt_load(static_cast<const uint4*>(p) + i);
      b.w[4 * i] = u.x; b.w[4 * i + 1] = u.y; b.w[4 * i + 2] = u.z; b.w[4 * i + 3] = u.w;
    }
  }
  return b;
}

// Encode 16 values in FMT (FP8: matrix scale sc with y = RN(1/sc); NVFP4: the
// block's decoded scale sd in sc), with the arithmetic of tile_store.
template <int FMT>
__device__ __forceinline__ Bytes<kChunkBytes<FMT>> encode16(const float* x, float sc, float y) {
  Bytes<kChunkBytes<FMT>> b;
  if constexpr (FMT == FMT_F32) {
#pragma unroll
    for (int i = 0; i < 16; ++i) b.w[i] = __float_as_uint(x[i]);
  } else if constexpr (FMT == FMT_F16) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      b.w[i] = static_cast<uint32_t>(__half_as_ushort(__float2half_rn(x[2 * i]))) |
               (static_cast<uint32_t>(__half_as_ushort(__float2half_rn(x[2 * i + 1]))) << 16);
  } else if constexpr (FMT == FMT_FP8) {
    fp8_codes<16>(x, sc, y, b.w);
  } else {
    nvfp4_codes<16>(x, sc, b.w);
  }
  return b;
}

// Decode 16 elements, each multiplied by mult (the matrix scale of FP8 / NVFP4
// is applied in the same product).
template <int FMT>
__device__ __forceinline__ void decode16(const Bytes<kChunkBytes<FMT>>& b, uint32_t scode, float ms, float mult,
                                         float* v) {
  if constexpr (FMT == FMT_F32) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(b.w[i]) * mult;
  } else if constexpr (FMT == FMT_F16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(b.w[i] & 0xFFFFu))) * mult;
      v[2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(b.w[i] >> 16))) * mult;
    }
  } else if constexpr (FMT == FMT_FP8) {
    decode_chunk<FMT_FP8, 8>(Raw<FMT_FP8, 8>{make_uint2(b.w[0], b.w[1])}, ms * mult, v);
    decode_chunk<FMT_FP8, 8>(Raw<FMT_FP8, 8>{make_uint2(b.w[2], b.w[3])}, ms * mult, v + 8);
  } else {
    decode_chunk<FMT_NVFP4, 8>(Raw<FMT_NVFP4, 8>{b.w[0], scode}, ms * mult, v);
    decode_chunk<FMT_NVFP4, 8>(Raw<FMT_NVFP4, 8>{b.w[1], scode}, ms * mult, v + 8);
  }
}

// NVFP4 block scale code of this lane's 16 values (one block), as
// nvfp4_block_code computes it for a block held by two threads.
__device__ __forceinline__ uint32_t nvfp4_scale16(const float* x, float ts) {
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(x[i]));
  return e4m3_code_of(bm / (6.0f * ts));
}

// ----------------------------------------------------------------------------
// loads
// ----------------------------------------------------------------------------
template <int FMT, int NR, int NC>
struct MRaw {
  using T = MTile<NR, NC>;
  static constexpr int CB = kChunkBytes<FMT>;
  Bytes<CB> c[T::RB][T::CG];
  uint32_t s[T::RB][T::CG];   // NVFP4 block scale codes
  float ms;

  // Every load is unconditional (all rows exist). The scheduling barrier keeps
  // the loads written before the tile (buffer records) ahead of it: returns
  // come back in issue order.
  __device__ __forceinline__ void issue(const StateBuf& sb, size_t mat) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < T::RB; ++r)
#pragma unroll
      for (int q = 0; q < T::CG; ++q) {
        const size_t elem = (mat * NR + T::row(r)) * NC + T::col(q);
        c[r][q] = load_bytes<CB>(static_cast<const uint8_t*>(sb.data) + elem * CB / 16);
        if constexpr (FMT == FMT_NVFP4) s[r][q] = sb.nv_scale[elem / 16];
      }
    ms = mat_scale<FMT>(sb, mat);
  }
  // dst = mult * (the stored values)
  __device__ __forceinline__ void decode(T& dst, float mult = 1.0f) const {
#pragma unroll
    for (int r = 0; r < T::RB; ++r)
#pragma unroll
      for (int q = 0; q < T::CG; ++q) {
        float v[16];
        decode16<FMT>(c[r][q], FMT == FMT_NVFP4 ? s[r][q] : 0u, ms, mult, v);
#pragma unroll
        for (int k = 0; k < 16; ++k) dst.set(r, q, k, v[k]);
      }
  }
};

// ----------------------------------------------------------------------------
// rank-m update on the matrix cores
// ----------------------------------------------------------------------------
// M <- M + sum_{e<m} rowv[e][n] colv[e][p] (rowv: m x NR LDS rows of stride
// rs, colv: m x NC LDS rows of stride cs). Entries past m enter as zeros on
// both operands (the LDS rows there are not read into the product), so stale
// LDS contents never reach the result. No barriers.
template <int NR, int NC>
__device__ __forceinline__ void mtile_rank_update(MTile<NR, NC>& M, const float* rowv, int rs, const float* colv,
                                                  int cs, int m) {
  using T = MTile<NR, NC>;
  const int g = static_cast<int>((threadIdx.x >> 4) & 3);
  for (int kc = 0; kc < (m + 3) >> 2; ++kc) {
    const int e = 4 * kc + g;
    const bool live = e < m;
    const int es = live ? e : 0;
    float bop[T::RB];
#pragma unroll
    for (int r = 0; r < T::RB; ++r) bop[r] = live ? rowv[es * rs + T::row(r)] : 0.0f;
#pragma unroll
    for (int q = 0; q < T::CG; ++q)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const float aop = live ? colv[es * cs + T::colv_col(q, cb)] : 0.0f;
#pragma unroll
        for (int r = 0; r < T::RB; ++r)
          M.v[r][q][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, bop[r], M.v[r][q][cb], 0, 0, 0);
      }
  }
}

// ----------------------------------------------------------------------------
// output matvec over rows
// ----------------------------------------------------------------------------
// The value v of the lane whose position in its 16-lane row is this lane's
// under the involution CTRL (row_mirror: j <-> 15 - j, row_half_mirror:
// j <-> 7 - j within each half, quad_perm xor 2 / xor 1). Every source lane
// exists, so the old value is never used.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One butterfly stage over a 16-lane row: the lanes with bit B of their row
// position set keep the upper half of x, the others the lower half, and each
// adds its partner's copy of the half it keeps (the partner, CTRL, has bit B
// flipped and the higher bits used so far unchanged).
template <int N, int CTRL, int B>
__device__ __forceinline__ void butterfly_stage(const float* x, float* out) {
  const bool up = (threadIdx.x >> B) & 1;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = up ? x[N / 2 + i] : x[i];
    const float send = up ? x[i] : x[N / 2 + i];
    out[i] = keep + dpp_partner<CTRL>(send);
  }
}

// Sums of 16 values over the 16 lanes of each row: afterwards lane j of the
// row holds the row's total of x[j]. Partners flip bits 3, 2, 1, 0 of the row
// position in turn (the XOR masks 15, 7, 2, 1 span all sixteen lanes).
__device__ __forceinline__ float row_transpose_sum16(const float* x) {
  float a[8], b[4], c[2], d[1];
  butterfly_stage<16, kDppMirror, 3>(x, a);
  butterfly_stage<8, kDppHalfMirror, 2>(a, b);
  butterfly_stage<4, kDppXor2, 1>(b, c);
  butterfly_stage<2, kDppXor1, 0>(c, d);
  return d[0];
}

// out[p] = sum_n M[n][p] w[n] (w: NR floats of LDS; out: NC floats of LDS;
// red: 4 NC floats of LDS scratch). Barriers inside; all threads must call.
template <int NR, int NC>
__device__ __forceinline__ void mtile_matvec(const MTile<NR, NC>& M, const float* w, float* red, float* out) {
  using T = MTile<NR, NC>;
  float wr[T::RB];
#pragma unroll
  for (int r = 0; r < T::RB; ++r) wr[r] = w[T::row(r)];
  const int wave = static_cast<int>(threadIdx.x >> 6), j = static_cast<int>(threadIdx.x & 15);
#pragma unroll
  for (int q = 0; q < T::CG; ++q) {
    float part[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < T::RB; ++r) acc += M.at(r, q, k) * wr[r];
      part[k] = acc;
    }
    // the 16 lanes of a row hold 16 rows of the same columns; lane j ends with column j of them
    red[wave * NC + T::col(q) + j] = row_transpose_sum16(part);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < NC; p += kThreads) out[p] = (red[p] + red[NC + p]) + (red[2 * NC + p] + red[3 * NC + p]);
  __syncthreads();
}

// out[j][p] = sum_n M[n][p] w[j ws + n] for the two weight rows j = 0, 1 (w:
// LDS; out: 2 NC floats of LDS; red: 8 NC floats of LDS scratch). Barriers
// inside; all threads must call.
template <int NR, int NC>
__device__ __forceinline__ void mtile_matvec2(const MTile<NR, NC>& M, const float* w, int ws, float* red, float* out) {
  using T = MTile<NR, NC>;
  float wr[2][T::RB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < T::RB; ++r) wr[j][r] = w[j * ws + T::row(r)];
  const int wave = static_cast<int>(threadIdx.x >> 6), ln = static_cast<int>(threadIdx.x & 15);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < T::CG; ++q) {
      float part[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < T::RB; ++r) acc += M.at(r, q, k) * wr[j][r];
        part[k] = acc;
      }
      red[(wave * 2 + j) * NC + T::col(q) + ln] = row_transpose_sum16(part);
    }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * NC; idx += kThreads) {
    const int j = idx / NC, c = idx - j * NC;
    out[idx] = (red[j * NC + c] + red[(2 + j) * NC + c]) + (red[(4 + j) * NC + c] + red[(6 + j) * NC + c]);
  }
  __syncthreads();
}

// M <- M Diag-on-rows(f): row n times f[n] (f: NR floats of LDS).
template <int NR, int NC>
__device__ __forceinline__ void mtile_scale_rows(MTile<NR, NC>& M, const float* f) {
  using T = MTile<NR, NC>;
#pragma unroll
  for (int r = 0; r < T::RB; ++r) {
    const float x = f[T::row(r)];
#pragma unroll
    for (int q = 0; q < T::CG; ++q)
#pragma unroll
      for (int b = 0; b < 4; ++b) M.v[r][q][b] *= x;
  }
}

// M <- L M.
template <int NR, int NC>
__device__ __forceinline__ void mtile_scale(MTile<NR, NC>& M, float L) {
  using T = MTile<NR, NC>;
#pragma unroll
  for (int r = 0; r < T::RB; ++r)
#pragma unroll
    for (int q = 0; q < T::CG; ++q)
#pragma unroll
      for (int b = 0; b < 4; ++b) M.v[r][q][b] *= L;
}

// Workgroup max of |M|, in every thread. Barriers inside.
template <int NR, int NC>
__device__ __forceinline__ float mtile_absmax(const MTile<NR, NC>& M, float* scratch4) {
  using T = MTile<NR, NC>;
  float mx = 0.0f;
#pragma unroll
  for (int r = 0; r < T::RB; ++r)
#pragma unroll
    for (int q = 0; q < T::CG; ++q)
#pragma unroll
      for (int k = 0; k < 16; ++k) mx = fmaxf(mx, fabsf(M.at(r, q, k)));
  mx = wave_max(mx);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch4[threadIdx.x >> 6] = mx;
  __syncthreads();
  return fmaxf(fmaxf(scratch4[0], scratch4[1]), fmaxf(scratch4[2], scratch4[3]));
}

// ----------------------------------------------------------------------------
// stores
// ----------------------------------------------------------------------------
// Store M into sb in format FMT (scales of FP8 and NVFP4 from M itself; for
// NVFP4 the matrix max may be passed in as amax >= 0 to skip its reduction).
// Byte-identical to tile_store of the same values. All threads must call.
template <int FMT, int NR, int NC>
__device__ __forceinline__ void mtile_store(const StateBuf& sb, size_t mat, const MTile<NR, NC>& M, float* scratch4,
                                            float amax = -1.0f) {
  using T = MTile<NR, NC>;
  constexpr int CB = kChunkBytes<FMT>;
  float sc = 1.0f;
  if constexpr (FMT == FMT_FP8) sc = fp8_scale_of(mtile_absmax(M, scratch4));
  if constexpr (FMT == FMT_NVFP4) sc = nvfp4_tscale_of(amax >= 0.0f ? amax : mtile_absmax(M, scratch4));
  const float y = 1.0f / sc;
#pragma unroll
  for (int r = 0; r < T::RB; ++r)
#pragma unroll
    for (int q = 0; q < T::CG; ++q) {
      const size_t elem = (mat * NR + T::row(r)) * NC + T::col(q);
      float x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = M.at(r, q, k);
      uint8_t* dst = static_cast<uint8_t*>(sb.data) + elem * CB / 16;
      if constexpr (FMT == FMT_NVFP4) {
        const uint32_t s = nvfp4_scale16(x, sc);
        store_bytes<CB>(encode16<FMT>(x, e4m3_value(s) * sc, 0.0f), dst);
        sb.nv_scale[elem / 16] = static_cast<uint8_t>(s);
      } else {
        store_bytes<CB>(encode16<FMT>(x, sc, y), dst);
      }
    }
  if constexpr (FMT == FMT_FP8 || FMT == FMT_NVFP4)
    if (threadIdx.x == 0) sb.tscale[mat] = sc;
}

// Replace M by the values it reads back as after a store in FMT (scales from M,
// as mtile_store computes them). All threads must call.
template <int FMT, int NR, int NC>
__device__ __forceinline__ void mtile_round_trip(MTile<NR, NC>& M, float* scratch4) {
  using T = MTile<NR, NC>;
  if constexpr (FMT != FMT_F32) {
    float sc = 1.0f;
    if constexpr (FMT == FMT_FP8) sc = fp8_scale_of(mtile_absmax(M, scratch4));
    if constexpr (FMT == FMT_NVFP4) sc = nvfp4_tscale_of(mtile_absmax(M, scratch4));
    const float y = 1.0f / sc;
#pragma unroll
    for (int r = 0; r < T::RB; ++r)
#pragma unroll
      for (int q = 0; q < T::CG; ++q) {
        float x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = M.at(r, q, k);
        uint32_t s = 0u;
        if constexpr (FMT == FMT_NVFP4) s = nvfp4_scale16(x, sc);
        const Bytes<kChunkBytes<FMT>> b = encode16<FMT>(x, FMT == FMT_NVFP4 ? e4m3_value(s) * sc : sc, y);
        decode16<FMT>(b, s, FMT == FMT_F16 ? 1.0f : sc, 1.0f, x);
#pragma unroll
        for (int k = 0; k < 16; ++k) M.set(r, q, k, x[k]);
      }
  }
}

}  // namespace rs

// Device-side helpers shared by the ReplaySSM decode kernels (gfx950).
//
// - element conversion of the input dtypes (fp32, bf16 bit patterns);
// - codecs of the stored-state formats (fp32, fp16, E4M3 with a per-matrix
//   scale, NVFP4 with E4M3 block scales and an fp32 tensor scale); the NVFP4
//   and E4M3 rules are those of the OCP microscaling / 8-bit float formats,
//   the formats the sitech.ge ReplaySSM page ("Bounding quantization error")
//   names for its low-precision reads;
// - the thread -> tile mapping used by every state-streaming kernel: a stored
//   state matrix is rows x cols (cols innermost), a 256-thread workgroup
//   covers it in passes, each thread owns E consecutive columns of one row per
//   pass, so reductions over rows stay in registers and only the final partial
//   sums cross lanes;
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "rs.h"
#include "rs_host.h"

namespace rs {

constexpr int kThreads = 256;

// ----------------------------------------------------------------------------
// input element types
// ----------------------------------------------------------------------------
struct bf16 {
  uint16_t u;
};

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return __uint_as_float(static_cast<uint32_t>(v.u) << 16); }

// Inverse of to_f for values that came from T (exact: no rounding happens).
template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float v) { return bf16{static_cast<uint16_t>(__float_as_uint(v) >> 16)}; }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------------------
// E4M3FN code values (decoding and encoding otherwise use the gfx950
// conversion instructions, with the tile loads and stores)
// ----------------------------------------------------------------------------
// Value of an E4M3FN code (a block scale): the packed FP8 conversion at unit
// scale, exact for every finite code (0x7F and 0xFF are NaN, as the format
// defines them; the encoders here never produce them).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code & 0xFFu, 1.0f, false)[0];
}

// ----------------------------------------------------------------------------
// streaming (nontemporal) vector loads and stores
// ----------------------------------------------------------------------------
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 nt_load(const float4* p) {
  const vf4 v = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const vu4 v = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 nt_load(const uint2* p) {
  const vu2 v = __builtin_nontemporal_load(reinterpret_cast<const vu2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t nt_load(const uint32_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ void nt_store(float4 v, float4* p) {
  vf4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<vf4*>(p));
}
__device__ __forceinline__ void nt_store(uint4 v, uint4* p) {
  vu4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<vu4*>(p));
}
__device__ __forceinline__ void nt_store(uint2 v, uint2* p) {
  vu2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<vu2*>(p));
}
__device__ __forceinline__ void nt_store(uint32_t v, uint32_t* p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store(float v, float* p) { __builtin_nontemporal_store(v, p); }

// ----------------------------------------------------------------------------
// stored-state access
// ----------------------------------------------------------------------------
// Thread -> (row, column chunk) mapping of a rows x cols matrix: each thread
// owns E consecutive columns of one row per pass.
template <int E_, int NR, int NC>
struct TileMap {
  static constexpr int E = E_;                         // consecutive columns per thread
  static constexpr int TPR = NC / E;                   // threads per row
  static constexpr int RPP = kThreads / TPR;           // rows per pass
  static constexpr int PASSES = (NR + RPP - 1) / RPP;
  static_assert(NC % E == 0, "cols must be a multiple of the chunk");
  static_assert(TPR >= 1 && TPR <= 64 && (64 % TPR) == 0, "a row must fit in one wavefront");
};

// Raw (undecoded) chunk of E elements of format FMT. fp32 takes E = 4 or 8;
// the other formats take E = 8 (an NVFP4 block of 16 spans two threads).
template <int FMT, int E>
struct Raw;
template <>
struct Raw<FMT_F32, 4> { float4 v; };
template <>
struct Raw<FMT_F32, 8> { float4 v, w; };
template <>
struct Raw<FMT_F16, 8> { uint4 v; };
template <>
struct Raw<FMT_FP8, 8> { uint2 v; };
template <>
struct Raw<FMT_NVFP4, 8> { uint32_t v; uint32_t s; };

template <int FMT, int E, int NC>
__device__ __forceinline__ Raw<FMT, E> load_chunk(const StateBuf& sb, size_t mat, int NR, int row, int c) {
  Raw<FMT, E> r;
  const size_t elem = (mat * NR + row) * NC + static_cast<size_t>(c) * E;
  if constexpr (FMT == FMT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(sb.data) + elem);
    r.v = nt_load(p);
    if constexpr (E == 8) r.w = nt_load(p + 1);
  } else if constexpr (FMT == FMT_F16) {
    r.v = nt_load(reinterpret_cast<const uint4*>(static_cast<const __half*>(sb.data) + elem));
  } else if constexpr (FMT == FMT_FP8) {
    r.v = nt_load(reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(sb.data) + elem));
  } else {
    r.v = nt_load(reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(sb.data) + elem / 2));
    r.s = sb.nv_scale[elem / 16];
  }
  return r;
}

// Per-matrix scalar needed to decode (FP8 scale, NVFP4 tensor scale).
template <int FMT>
__device__ __forceinline__ float mat_scale(const StateBuf& sb, size_t mat) {
  if constexpr (FMT == FMT_FP8 || FMT == FMT_NVFP4) return sb.tscale[mat];
  return 1.0f;
}

template <int FMT, int E>
__device__ __forceinline__ void decode_chunk(const Raw<FMT, E>& r, float ms, float* v) {
  if constexpr (FMT == FMT_F32) {
    v[0] = r.v.x; v[1] = r.v.y; v[2] = r.v.z; v[3] = r.v.w;
    if constexpr (E == 8) { v[4] = r.w.x; v[5] = r.w.y; v[6] = r.w.z; v[7] = r.w.w; }
  } else if constexpr (FMT == FMT_F16) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
      v[2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
    }
  } else if constexpr (FMT == FMT_FP8) {
    // gfx950 converts two E4M3FN codes per instruction, exactly (the scale operand
    // only contributes its exponent, so it is 1 and the scale is applied after)
    const uint32_t w[2] = {r.v.x, r.v.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[h], 1.0f, false);   // bytes 0, 1
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[h], 1.0f, true);    // bytes 2, 3
      v[4 * h + 0] = lo.x * ms;
      v[4 * h + 1] = lo.y * ms;
      v[4 * h + 2] = hi.x * ms;
      v[4 * h + 3] = hi.y * ms;
    }
  } else {
    // two E2M1 codes per instruction (low nibble first), exactly; block and tensor
    // scale applied after
    const float sd = e4m3_value(r.s) * ms;
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 3);
    v[0] = p0.x * sd; v[1] = p0.y * sd; v[2] = p1.x * sd; v[3] = p1.y * sd;
    v[4] = p2.x * sd; v[5] = p2.y * sd; v[6] = p3.x * sd; v[7] = p3.y * sd;
  }
}

// The chunk's element values before the per-chunk and per-matrix scales (FP8:
// the E4M3 values; NVFP4: the E2M1 values; FP16: the values), and the
// per-chunk scale (NVFP4: the E4M3 block scale; otherwise 1). A reduction
// that weights every element of a chunk by the same factor folds the chunk
// scale into that factor and the matrix scale into its result.
template <int FMT>
__device__ __forceinline__ void decode_codes8(const Raw<FMT, 8>& r, float* v) {
  static_assert(FMT == FMT_F16 || FMT == FMT_FP8 || FMT == FMT_NVFP4, "low-precision chunks");
  if constexpr (FMT == FMT_F16) {
    decode_chunk<FMT_F16, 8>(r, 1.0f, v);
  } else if constexpr (FMT == FMT_FP8) {
    const uint32_t w[2] = {r.v.x, r.v.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[h], 1.0f, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[h], 1.0f, true);
      v[4 * h + 0] = lo.x; v[4 * h + 1] = lo.y; v[4 * h + 2] = hi.x; v[4 * h + 3] = hi.y;
    }
  } else {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.v, 1.0f, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y; v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  }
}
template <int FMT>
__device__ __forceinline__ float chunk_scale(const Raw<FMT, 8>& r) {
  if constexpr (FMT == FMT_NVFP4) return e4m3_value(r.s);
  return 1.0f;
}

// ----------------------------------------------------------------------------
// wavefront helpers
// ----------------------------------------------------------------------------
// Cross-lane reductions without the LDS path: inside a 16-lane row through
// DPP operand modifiers (quad_perm, row rotations and mirrors fold into the
// add), across rows through gfx950's permlane swaps, which exchange rows 0/1
// and 2/3 (permlane16) or the two halves of the wavefront (permlane32).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;       // row_ror:4
constexpr int kDppRor8 = 0x128;       // row_ror:8
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// v of this lane and of lane ^ 16 (respectively ^ 32), as the pair the swap returns
__device__ __forceinline__ f32x2 swap16(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(q[0]), __uint_as_float(q[1])};
}
__device__ __forceinline__ f32x2 swap32(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(q[0]), __uint_as_float(q[1])};
}

// Sum over the lanes that agree on (lane mod FROM); FROM a power of two <= 32.
template <int FROM>
__device__ __forceinline__ float wave_sum_stride(float v) {
  static_assert(FROM >= 1 && FROM <= 32 && (FROM & (FROM - 1)) == 0, "power of two up to 32");
  if constexpr (FROM == 1) v += dpp_mov<kDppXor1>(v);
  if constexpr (FROM <= 2) v += dpp_mov<kDppXor2>(v);
  if constexpr (FROM <= 4) v += dpp_mov<kDppRor4>(v);   // with ror 8: the row's lanes of one residue mod 4
  if constexpr (FROM <= 8) v += dpp_mov<kDppRor8>(v);
  if constexpr (FROM <= 16) {
    const f32x2 p = swap16(v);
    v = p.x + p.y;
  }
  const f32x2 p = swap32(v);
  return p.x + p.y;
}

// One lane's part of a length-N dot of LDS rows held by a 16-lane group: lane
// ln takes the N/16 consecutive elements from ln*N/16, with 16-byte LDS loads
// when that run is a whole number of float4 (rows then 16-byte aligned).
// Optional third row w weights the products. Sum the parts with group_sum16.
template <int N>
__device__ __forceinline__ float lds_dot16(const float* a, const float* b, int ln, const float* w = nullptr) {
  constexpr int R = N / 16;
  float part = 0.0f;
  if constexpr (N % 16 == 0 && R % 4 == 0) {
    const float4* pa = reinterpret_cast<const float4*>(a + ln * R);
    const float4* pb = reinterpret_cast<const float4*>(b + ln * R);
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      float4 x = pa[q];
      const float4 y = pb[q];
      if (w) {
        const float4 z = reinterpret_cast<const float4*>(w + ln * R)[q];
        x.x *= z.x; x.y *= z.y; x.z *= z.z; x.w *= z.w;
      }
      part += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
  } else {
    for (int n = ln; n < N; n += 16) part += (w ? a[n] * w[n] : a[n]) * b[n];
  }
  return part;
}

// Transposing sum over the 8 lanes that share (lane mod 8): each lane brings
// 8 values, and after three exchange-and-add stages (lane bit 5 through the
// half swap, bit 4 through the row-pair swap, bit 3 through a row rotation by
// 8) each lane holds the 8-lane sum of one of them, whose index (0..7) goes to
// `which`; every index is held by exactly one lane of the 8. 7 exchanges and 7
// adds instead of 3 per value. The index is tracked through the same
// exchanges, so it does not depend on which half of a swap moves.
__device__ __forceinline__ float transpose_sum8(const float (&v)[8], int& which) {
  const bool hi3 = (threadIdx.x & 8) != 0;
  float a[4];
  int ia = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
    a[i] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  {
    const auto q = __builtin_amdgcn_permlane32_swap(0u, 4u, false, false);
    ia = static_cast<int>(q[0]);   // 0 or 4: the column offset this lane now holds
  }
  float b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 2]), false, false);
    b[i] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  {
    const auto q = __builtin_amdgcn_permlane16_swap(0u, 2u, false, false);
    ia += static_cast<int>(q[0]);
  }
  const float keep = hi3 ? b[1] : b[0], send = hi3 ? b[0] : b[1];
  which = ia + (hi3 ? 1 : 0);
  return keep + dpp_mov<kDppRor8>(send);
}

// Suffix products inside each aligned group of 16 lanes (a DPP row): lane l
// gets the product of v over the lanes l .. 15 of its row, by four row shifts
// toward lane 0 (row_shl; a lane whose source would lie past the row's end
// reads 1). Every lane of the row must hold a value.
__device__ __forceinline__ float row_suffix_prod16(float v) {
  const int one = __float_as_int(1.0f);
  v *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(v), 0x101, 0xF, 0xF, false));
  v *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(v), 0x102, 0xF, 0xF, false));
  v *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(v), 0x104, 0xF, 0xF, false));
  v *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(v), 0x108, 0xF, 0xF, false));
  return v;
}

// v of lane l + 1 of the same 16-lane row, 1 for the row's last lane.
__device__ __forceinline__ float row_next16(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v), 0x101, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes (a DPP row), in every lane of it.
__device__ __forceinline__ float group_sum16(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  return v;
}

// Maximum over the wavefront, in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppMirror>(v));
  f32x2 p = swap16(v);
  v = fmaxf(p.x, p.y);
  p = swap32(v);
  return fmaxf(p.x, p.y);
}

// Workgroups are handed to the eight XCDs round-robin; give each XCD a
// contiguous range of tiles so the heads of one sequence (which share that
// sequence's B/C or k/q records) meet in the same L2.
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  const int per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace rs

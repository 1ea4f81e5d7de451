// Gated DeltaNet decode kernels for gfx950: conventional read-modify-write
// step, and the ReplaySSM non-flush and flush steps in UT / WY form.
//
// Per sequence b and value head h (key/query head h / (n_v / n_qk)):
//   alpha = exp(g);  S = alpha S (I - beta k k^T) + beta v k^T;  o = S q
// With u_t = beta_t (v_t - alpha_t S_{t-1} k_t), S_t = alpha_t S_{t-1} + u_t k_t^T,
// so over buffer entries 1..j from the checkpoint S0 (gamma_t = prod_{l<=t}
// alpha_l, r_{t,i} = prod_{i<l<=t} alpha_l):
//   u_t = beta_t (v_t - gamma_t S0 k_t) - sum_{i<t} beta_t r_{t,i} (k_t.k_i) u_i
//   o_j = gamma_j S0 q_j + sum_{i<=j} r_{j,i} (k_i.q_j) u_i
//   S_m = gamma_m S0 + sum_i r_{m,i} u_i k_i^T                      (the fold)
// (sitech.ge ReplaySSM page, "How ReplaySSM works": output from checkpoint +
// buffer without a state write; one checkpoint write when the buffer fills.)
//
// The u_t are the rows of the unit lower-triangular system (I + L) U =
// diag(beta)(V - diag(gamma) K S0^T) solved by forward substitution. Row t
// depends only on S0 and entries <= t, so it is solved once, on the step that
// appends entry t, and kept beside that entry in the ring; every step then
// needs just S0 k_j and S0 q_j from its single read of S0, plus length-dv
// vector work over the held rows.
//
// States are stored as [dk][dv] (value index innermost) so that S0 k and S0 q
// are sums over rows held in registers. One 256-thread workgroup per column
// slice of a (sequence, value head) state in the ReplaySSM steps: dv = 128 is
// split into two slices of 64 columns (32 KiB of fp32 each), smaller states
// are one slice; the conventional step takes the whole state.
#include <type_traits>

#include "rs_device.h"
#include "rs_tile.h"
#include "rs_mtile.h"
#include "rs_internal.h"

namespace rs {

namespace {

// Value columns split across NS workgroups: with k, q, g, beta fixed, column v
// of the stored state (row v of S) evolves and is read out on its own, so a
// workgroup owns the columns c0..c0+NVS-1 of one state and repeats the few
// length-dk dots of the other slices.
template <int NV>
constexpr int gdn_slices() { return NV >= 128 ? 2 : 1; }

// Columns that one flush or commit-fold workgroup folds: its own slice, or for
// an FP8 checkpoint the whole state (one scale spans the matrix, and its amax
// needs every folded column in one workgroup).
template <int NV, int CKF>
constexpr int gdn_fold_cols() { return CKF == FMT_FP8 ? NV : NV / gdn_slices<NV>(); }
// Workgroups per state of the flush kernel: one per folded column range. (The
// self-scheduling kernel keeps the non-flush step's slices; there the other
// slices' workgroups of an FP8 flush only count in.)
template <int NV, int CKF>
constexpr int gdn_flush_slices() { return NV / gdn_fold_cols<NV, CKF>(); }

// The state tile a fold holds. Column slices (fp32 and FP16 checkpoints) keep
// the streaming register layout, four columns per thread and pass. A whole FP8
// state whose sides are multiples of 64 is held in the matrix-core
// accumulator layout instead: its rank-m update runs on v_mfma_f32_16x16x4f32
// in fp32, and its loads and stores move 16 codes (one row's 16 consecutive
// columns) per lane.
template <int CKF, int NK, int NV, int NVS>
constexpr bool gdn_mfma_fold() { return CKF == FMT_FP8 && NVS == NV && NK % 64 == 0 && NV % 64 == 0; }

// VG: Kimi Delta Attention, the decay is a vector over the dk key channels
// (a per-channel gate) instead of one scalar per head.
template <int NK, int NVS, bool VG = false>
struct alignas(16) GSmem {
  static constexpr int kNK = NK;
  static constexpr int kNVS = NVS;
  static constexpr bool kVG = VG;
  alignas(16) float K[kRing][NK];    // k of entries 0..m-1
  alignas(16) float W[4][NK];        // matvec weights: k_cur, q, 0, 0
  float U[kRing][NVS];   // u of entries 0..m-1 (the current one computed here), own columns
  float vc[NVS];         // v of the current token, own columns
  float out[4][NVS];     // S0 k_cur, S0 q
  float red[VG ? 1 : 4 * 4 * NVS];   // matvec scratch (VG: lives in A, dead by then)
  float kk[kRing];       // beta_cur r_{cur,i} (k_cur . k_i), i < cur
  float kq[kRing];       // r_{cur,i} (k_i . q), i <= cur
  float rr[kRing];       // r_{cur,i}
  float al[kRing];
  float gam, bet;
  float s4[4];
  // VG: per-channel log decays of entries 0..m-1, then in place the products
  // r_{cur,e} = prod_{e<l<=cur} alpha_l; gv = gamma_cur per channel
  alignas(16) float A[VG ? kRing : 1][NK];
  float gv[VG ? NK : 1];
  static_assert(!VG || 4 * 4 * NVS <= kRing * NK, "matvec scratch fits in the decay table");
  __device__ __forceinline__ float* redp() { if constexpr (VG) return &A[0][0]; else return red; }
};

struct GPtrs {
  size_t st;       // state index b * n_v + h
  int b, h, kh;
  int half, c0;    // column slice and its first column
};

template <int NV, int NS>
__device__ __forceinline__ GPtrs gdn_tile(const GDNArgs& a) {
  GPtrs p;
  const size_t t = static_cast<size_t>(xcd_tile(blockIdx.x, gridDim.x));
  p.st = t / NS;
  p.half = static_cast<int>(t - p.st * NS);
  p.c0 = p.half * (NV / NS);
  p.b = static_cast<int>(p.st / a.nv);
  p.h = static_cast<int>(p.st - static_cast<size_t>(p.b) * a.nv);
  p.kh = p.h / a.vpk;
  return p;
}

__device__ __forceinline__ int slot_of(long long nck, int e) { return static_cast<int>((nck + e) & (kRing - 1)); }

// fp32 columns c0..c0+NVS-1 of state `st` ([NK][NV], value index innermost)
// as a RegTile<4, NK, NVS>: each thread owns 4 consecutive columns of one row
// per pass. Loads are issued unconditionally (rows past NK are clamped and
// dropped when decoding).
template <int NK, int NV, int NVS>
struct GSlice {
  using TM = TileMap<4, NK, NVS>;
  float4 r[TM::PASSES];
  __device__ __forceinline__ static size_t off(size_t st, int c0, int row) {
    return (st * NK + row) * NV + c0 + RegTile<4, NK, NVS>::col0();
  }
  // (loads written before the slice stay ahead of it, as for RawTile::issue)
  __device__ __forceinline__ void issue(const float* base, size_t st, int c0) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      int row = RegTile<4, NK, NVS>::row(k);
      if constexpr (NK % TM::RPP != 0 || TM::RPP > NK) row = row < NK ? row : NK - 1;
      r[k] = nt_load(reinterpret_cast<const float4*>(base + off(st, c0, row)));
    }
  }
  __device__ __forceinline__ void decode(RegTile<4, NK, NVS>& d) const {
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const bool in = (NK % TM::RPP == 0 && TM::RPP <= NK) || RegTile<4, NK, NVS>::row(k) < NK;
      d.v[k][0] = in ? r[k].x : 0.0f;
      d.v[k][1] = in ? r[k].y : 0.0f;
      d.v[k][2] = in ? r[k].z : 0.0f;
      d.v[k][3] = in ? r[k].w : 0.0f;
    }
  }
  __device__ __forceinline__ static void store(float* base, size_t st, int c0, const RegTile<4, NK, NVS>& S) {
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = RegTile<4, NK, NVS>::row(k);
      if (row < NK)
        nt_store(make_float4(S.v[k][0], S.v[k][1], S.v[k][2], S.v[k][3]),
                 reinterpret_cast<float4*>(base + off(st, c0, row)));
    }
  }
  // the checkpoint slice a step reads
  __device__ __forceinline__ void issue_read(const GDNArgs& a, size_t st, int c0) {
    issue(static_cast<const float*>(a.ck.data), st, c0);
  }
};

// The same slice read from the NVFP4 read copy (sitech.ge ReplaySSM page,
// "Bounding quantization error": reads go to a low-precision copy), decoded into
// the same register layout: a thread's four columns are two bytes of E2M1 codes
// and its block's E4M3 scale (the block's 16 columns span four threads), times
// the matrix's tensor scale. The value is e2m1(code) * (e4m3(scale) * tscale),
// the product rounded as the format defines it.
template <int NK, int NV, int NVS>
struct GSliceNv {
  using TM = TileMap<4, NK, NVS>;
  static constexpr bool kWhole = NK % TM::RPP == 0 && TM::RPP <= NK;   // every pass's rows exist
  uint32_t c[TM::PASSES];   // four codes (two bytes)
  uint32_t s[TM::PASSES];   // block scale code
  float ts;
  __device__ __forceinline__ void issue_read(const GDNArgs& a, size_t st, int c0) {
    __builtin_amdgcn_sched_barrier(0);
    // the slice's codes and scales from per-workgroup bases plus one 32-bit lane
    // offset each, so that the passes differ only in the loads' immediate offsets
    const size_t e0 = st * NK * NV + c0;   // the slice's first element
    const uint8_t* cb = static_cast<const uint8_t*>(a.rc.data) + e0 / 2;
    const uint8_t* sb = a.rc.nv_scale + e0 / 16;
    const int r0 = static_cast<int>(threadIdx.x) / TM::TPR;
    const uint32_t lo = static_cast<uint32_t>(r0 * NV + RegTile<4, NK, NVS>::col0());
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      uint32_t off = lo + static_cast<uint32_t>(k * TM::RPP * NV);
      if constexpr (!kWhole) {
        const int row = r0 + k * TM::RPP;
        off = static_cast<uint32_t>((row < NK ? row : NK - 1) * NV + RegTile<4, NK, NVS>::col0());
      }
      c[k] = *reinterpret_cast<const uint16_t*>(cb + off / 2);
      s[k] = sb[off / 16];
    }
    ts = a.rc.tscale[st];
  }
  // out[q][col] = sum_rows S0[row][col] w[q ws + row] for q = 0, 1 straight from
  // the codes: a thread's four columns share a block scale, so the scale joins
  // the two row weights (two multiplies instead of four) and the tensor scale
  // joins the sum; the 4 lanes that share columns add their 8 values by a
  // transposing exchange (each lane ends with 2). `red` is 4 * 2 * NVS floats
  // of LDS, `out` 2 * NVS. Barriers inside; all threads call.
  __device__ __forceinline__ void matvec2(const float* w, int ws, float* red, float* out) const {
    static_assert(TM::TPR == 16, "16 lanes per row of four columns");
    const int r0 = static_cast<int>(threadIdx.x) / TM::TPR;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = r0 + k * TM::RPP;
      if (kWhole || row < NK) {
        const float sd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s[k], 1.0f, false)[0];   // byte 0: the scale
        const float w0 = w[row] * sd, w1 = w[ws + row] * sd;
        const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 0);
        const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 1);
        acc[0] += lo.x * w0; acc[1] += lo.y * w0; acc[2] += hi.x * w0; acc[3] += hi.y * w0;
        acc[4] += lo.x * w1; acc[5] += lo.y * w1; acc[6] += hi.x * w1; acc[7] += hi.y * w1;
      }
    }
    // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same columns: halves (bit 5)
    // split the two weight rows, row pairs (bit 4) the column pairs
    float a4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i + 4]), false, false);
      a4[i] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    }
    const int qr = static_cast<int>(__builtin_amdgcn_permlane32_swap(0u, 1u, false, false)[0]);   // weight row held
    float a2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a4[i]), __float_as_uint(a4[i + 2]), false, false);
      a2[i] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    }
    const int cp = static_cast<int>(__builtin_amdgcn_permlane16_swap(0u, 2u, false, false)[0]);   // column pair held
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    *reinterpret_cast<float2*>(&red[(wave * 2 + qr) * NVS + (lane & 15) * 4 + cp]) = make_float2(a2[0], a2[1]);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 2 * NVS; idx += kThreads)
      out[idx] = ts * ((red[idx] + red[2 * NVS + idx]) + (red[4 * NVS + idx] + red[6 * NVS + idx]));
    __syncthreads();
  }
  __device__ __forceinline__ void decode(RegTile<4, NK, NVS>& d) const {
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const bool in = (NK % TM::RPP == 0 && TM::RPP <= NK) || RegTile<4, NK, NVS>::row(k) < NK;
      const float sd = e4m3_value(s[k]) * ts;
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 0);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[k], 1.0f, 1);
      d.v[k][0] = in ? lo.x * sd : 0.0f;
      d.v[k][1] = in ? lo.y * sd : 0.0f;
      d.v[k][2] = in ? hi.x * sd : 0.0f;
      d.v[k][3] = in ? hi.y * sd : 0.0f;
    }
  }
};

// What the non-flush step and the speculative append read: the checkpoint, or
// its read copy.
// The slice of a checkpoint stored in format CKF (fp32, FP16, or E4M3 codes with
// one fp32 scale per matrix), in GSlice's register layout: four columns per
// thread and pass, i.e. 16, 8 or 4 bytes per load and store.
template <int CKF, int NK, int NV, int NVS>
struct GSliceF {
  static_assert(CKF == FMT_F32 || CKF == FMT_F16 || CKF == FMT_FP8, "fp32, FP16 or FP8 checkpoints");
  using TM = TileMap<4, NK, NVS>;
  using Word = typename std::conditional<CKF == FMT_F32, float4,
                                         typename std::conditional<CKF == FMT_F16, uint2, uint32_t>::type>::type;
  using Elem = typename std::conditional<CKF == FMT_F32, float,
                                         typename std::conditional<CKF == FMT_F16, uint16_t, uint8_t>::type>::type;
  Word r[TM::PASSES];
  float ms;   // FP8: the matrix scale
  __device__ __forceinline__ static size_t off(size_t st, int c0, int row) {
    return (st * NK + row) * NV + c0 + RegTile<4, NK, NVS>::col0();
  }
  // (loads written before the slice stay ahead of it, as for RawTile::issue)
  __device__ __forceinline__ void issue(const StateBuf& sb, size_t st, int c0) {
    __builtin_amdgcn_sched_barrier(0);
    const Elem* base = static_cast<const Elem*>(sb.data);
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      int row = RegTile<4, NK, NVS>::row(k);
      if constexpr (NK % TM::RPP != 0 || TM::RPP > NK) row = row < NK ? row : NK - 1;
      r[k] = nt_load(reinterpret_cast<const Word*>(base + off(st, c0, row)));
    }
    ms = CKF == FMT_FP8 ? sb.tscale[st] : 1.0f;
  }
  __device__ __forceinline__ void issue_read(const GDNArgs& a, size_t st, int c0) { issue(a.ck, st, c0); }
  __device__ __forceinline__ void decode(RegTile<4, NK, NVS>& d) const {
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const bool in = (NK % TM::RPP == 0 && TM::RPP <= NK) || RegTile<4, NK, NVS>::row(k) < NK;
      float t[4];
      if constexpr (CKF == FMT_F32) {
        t[0] = r[k].x; t[1] = r[k].y; t[2] = r[k].z; t[3] = r[k].w;
      } else if constexpr (CKF == FMT_F16) {
        const uint32_t w[2] = {r[k].x, r[k].y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          t[2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
          t[2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
        }
      } else {
        // two E4M3FN codes per conversion, exactly; the scale applied after
        const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, false);
        const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, true);
        t[0] = lo.x * ms; t[1] = lo.y * ms; t[2] = hi.x * ms; t[3] = hi.y * ms;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) d.v[k][i] = in ? t[i] : 0.0f;
    }
  }
  // FP8: the E4M3 values of the codes without the matrix scale (ms), for a
  // caller that applies it to sums instead.
  __device__ __forceinline__ void decode_values(RegTile<4, NK, NVS>& d) const {
    static_assert(CKF == FMT_FP8, "FP8 codes");
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const bool in = (NK % TM::RPP == 0 && TM::RPP <= NK) || RegTile<4, NK, NVS>::row(k) < NK;
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r[k], 1.0f, true);
      d.v[k][0] = in ? lo.x : 0.0f;
      d.v[k][1] = in ? lo.y : 0.0f;
      d.v[k][2] = in ? hi.x : 0.0f;
      d.v[k][3] = in ? hi.y : 0.0f;
    }
  }
  // Store S (FP8: codes under the matrix scale sc, y = RN(1/sc), which the
  // caller derived from the whole matrix's |max|; the scale itself is the
  // caller's to write).
  __device__ __forceinline__ static void store(const StateBuf& sb, size_t st, int c0, const RegTile<4, NK, NVS>& S,
                                               float sc = 1.0f, float y = 1.0f) {
    Elem* base = static_cast<Elem*>(sb.data);
#pragma unroll
    for (int k = 0; k < TM::PASSES; ++k) {
      const int row = RegTile<4, NK, NVS>::row(k);
      if (row >= NK) continue;
      Word* dst = reinterpret_cast<Word*>(base + off(st, c0, row));
      if constexpr (CKF == FMT_F32) {
        nt_store(make_float4(S.v[k][0], S.v[k][1], S.v[k][2], S.v[k][3]), dst);
      } else if constexpr (CKF == FMT_F16) {
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          w[i] = static_cast<uint32_t>(__half_as_ushort(__float2half_rn(S.v[k][2 * i]))) |
                 (static_cast<uint32_t>(__half_as_ushort(__float2half_rn(S.v[k][2 * i + 1]))) << 16);
        nt_store(make_uint2(w[0], w[1]), dst);
      } else {
        uint32_t w;
        fp8_codes<4>(S.v[k], sc, y, &w);
        nt_store(w, dst);
      }
    }
  }
};

template <bool RC, int CKF, int NK, int NV, int NVS>
using ReadSlice = typename std::conditional<RC, GSliceNv<NK, NV, NVS>, GSliceF<CKF, NK, NV, NVS>>::type;

template <bool MF, int CKF, int NK, int NV, int NVS>
struct GFoldTypes {
  using Tile = RegTile<4, NK, NVS>;
  using Raw = GSliceF<CKF, NK, NV, NVS>;
};
template <int CKF, int NK, int NV, int NVS>
struct GFoldTypes<true, CKF, NK, NV, NVS> {
  using Tile = MTile<NK, NV>;
  using Raw = MRaw<FMT_FP8, NK, NV>;
};
template <int CKF, int NK, int NV, int NVS>
using GFoldTile = typename GFoldTypes<gdn_mfma_fold<CKF, NK, NV, NVS>(), CKF, NK, NV, NVS>::Tile;
template <int CKF, int NK, int NV, int NVS>
using GFoldRaw = typename GFoldTypes<gdn_mfma_fold<CKF, NK, NV, NVS>(), CKF, NK, NV, NVS>::Raw;

// The fold's loads and output matvec on either layout: issue the checkpoint's
// columns c0.., and the matvec against the two weight rows.
template <int CKF, int NK, int NV, int NVS>
__device__ __forceinline__ void fold_issue(GSliceF<CKF, NK, NV, NVS>& r, const StateBuf& sb, size_t st, int c0) {
  r.issue(sb, st, c0);
}
template <int NK, int NV>
__device__ __forceinline__ void fold_issue(MRaw<FMT_FP8, NK, NV>& r, const StateBuf& sb, size_t st, int) {
  r.issue(sb, st);
}
template <int NK, int NVS>
__device__ __forceinline__ void fold_matvec2(const RegTile<4, NK, NVS>& S, const float* w, int ws, float* red, float* out) {
  tile_matvec<2>(S, w, ws, red, out);
}
template <int NK, int NV>
__device__ __forceinline__ void fold_matvec2(const MTile<NK, NV>& S, const float* w, int ws, float* red, float* out) {
  mtile_matvec2(S, w, ws, red, out);
}

// Stage the window's entries 0..m-1 (entry m-1 is the current token, the
// others come from the ring): k rows, the own columns of the held entries' u
// rows, the decays, and the current v (own columns), beta, and the matvec
// weights [k_cur, q, 0, 0]. Loads go to registers first (load), so the caller
// can issue the state tile after them and still have the records while the
// tile streams in (vector loads return in order); store moves them to LDS.
template <typename TIN, int NK, int NV, int NVS, bool VG = false>
struct GStage {
  static constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NK % VK == 0 && NVS % VK == 0 && NVS % 4 == 0, "records are whole 16-byte chunks");
  static constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  static constexpr int CU = (kRing * NVS / 4 + kThreads - 1) / kThreads;
  static constexpr int CQ = (NK / VK + kThreads - 1) / kThreads;
  static constexpr int CV = (NVS / VK + kThreads - 1) / kThreads;
  static constexpr int CG = VG ? (kRing * NK / 4 + kThreads - 1) / kThreads : 1;
  RegChunks<TIN, CK> k;
  RegChunks<float, CU> u;
  RegChunks<TIN, CQ> q, kc;
  RegChunks<TIN, CV> v;
  RegChunks<float, CG> gr;   // VG: per-channel gate rows of entries 0..m-1
  float g, beta;

  __device__ __forceinline__ void load(const GDNArgs& a, const GPtrs& p, long long nck, int m) {
    const int held = m - 1;
    const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
    const TIN* rk = static_cast<const TIN*>(a.rk) + bk * kRing * NK;
    const float* ru = static_cast<const float*>(a.ru) + p.st * kRing * NV + p.c0;
    const float* rg = static_cast<const float*>(a.rg) + p.st * kRing;
    const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
    const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
    const TIN* iv = static_cast<const TIN*>(a.v) + p.st * NV + p.c0;
    k.load(EntrySrc<TIN>{rk, ik, 0, nck, held, NK}, m, NK);
    // u rows are NV apart, NVS of them are ours; with no held entry every lane
    // reads the ring's first row and stores nothing
    u.load(EntrySrc<float>{ru, ru, 0, nck, held, NV}, held, NVS);
    q.load(EntrySrc<TIN>{iq, iq, 0, 0, 0, NK}, 1, NK);
    kc.load(EntrySrc<TIN>{ik, ik, 0, 0, 0, NK}, 1, NK);
    v.load(EntrySrc<TIN>{iv, iv, 0, 0, 0, NVS}, 1, NVS);
    if constexpr (VG) {
      const float* rgv = static_cast<const float*>(a.rg) + p.st * kRing * NK;
      gr.load(EntrySrc<float>{rgv, a.g + p.st * NK, 0, nck, held, NK}, m, NK);
      g = 0.0f;
    } else {
      const int e = static_cast<int>(threadIdx.x) < m ? static_cast<int>(threadIdx.x) : m - 1;
      g = *(e < held ? rg + slot_of(nck, e) : a.g + p.st);
    }
    beta = a.beta[p.st];
  }
  __device__ __forceinline__ void store(GSmem<NK, NVS, VG>& s, int m) const {
    const int held = m - 1;
    k.to_lds(&s.K[0][0], NK, m, NK);
    u.to_lds(&s.U[0][0], NVS, held, NVS);
    kc.to_lds(&s.W[0][0], NK, 1, NK);
    q.to_lds(&s.W[1][0], NK, 1, NK);
    v.to_lds(s.vc, NVS, 1, NVS);
    for (int n = threadIdx.x; n < NK; n += kThreads) {
      s.W[2][n] = 0.0f;
      s.W[3][n] = 0.0f;
    }
    if constexpr (VG) gr.to_lds(&s.A[0][0], NK, m, NK);
    else if (static_cast<int>(threadIdx.x) < m) s.al[threadIdx.x] = expf(g);
    if (threadIdx.x == 0) s.bet = beta;
  }
};

// A KDA channel decay alpha = exp(g), as 2^(g log2 e) on the hardware
// exponential: a relative error of about |g| 2^-24 per factor, |log r| 2^-24 on
// a product r of them, at a fraction of the library exp's instructions. A
// window takes 16 decays per key channel; every KDA kernel (the conventional
// baselines included) forms them this way.
__device__ __forceinline__ float kda_alpha(float g) { return __expf(g); }

// VG only, after staging is visible: per key channel c, the decay products
// r_{cur,e}[c] = prod_{e<l<=cur} alpha_l[c] replace the staged log decays (the
// same descending order as the definition's direct products), gamma_cur[c] goes
// to gv, and the matvec weights become gamma * k_cur and gamma * q (the plain q
// is kept in W[2] for the dots). The scalar gamma of the common code is 1.
template <typename SM>
__device__ __forceinline__ void kda_decays(SM& s, int m) {
  const int cur = m - 1;
  for (int c = threadIdx.x; c < SM::kNK; c += kThreads) {
    float acc = 1.0f;
#pragma unroll
    for (int e = kRing - 1; e >= 0; --e) {
      if (e <= cur) {
        const float al = kda_alpha(s.A[e][c]);
        s.A[e][c] = acc;
        acc *= al;
      }
    }
    s.gv[c] = acc;
    const float qv = s.W[1][c];
    s.W[2][c] = qv;
    s.W[0][c] *= acc;
    s.W[1][c] = qv * acc;
  }
  if (threadIdx.x == 0) s.gam = 1.0f;
}

// Dots and decays for the current entry cur = m-1 (after staging is visible):
//   kk[i] = beta_cur r_{cur,i} (k_cur . k_i) for i < cur
//   kq[i] = r_{cur,i} (k_i . q) for i <= cur;  rr[i] = r_{cur,i};  gam = gamma_cur
// VG: the decays are per channel and weight the dots instead (r = 1):
//   kk[i] = beta_cur <k_cur, r_{cur,i} * k_i>,  kq[i] = <q, r_{cur,i} * k_i>
template <typename SM>
__device__ __forceinline__ void gdn_dots(SM& s, int m) {
  constexpr int NK = SM::kNK;
  const int cur = m - 1;
  const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
  for (int pr = grp; pr < 2 * m - 1; pr += kThreads / 16) {
    const bool isq = pr >= cur;
    const int i = isq ? pr - cur : pr;
    const float* other = isq ? &s.W[SM::kVG ? 2 : 1][0] : &s.K[cur][0];
    float part = lds_dot16<NK>(&s.K[i][0], other, ln, SM::kVG ? &s.A[i][0] : nullptr);
    part = group_sum16(part);
    if (ln == 0) {
      float r = 1.0f;
      if constexpr (!SM::kVG) {
#pragma unroll
        for (int l = 1; l < kRing; ++l) r *= (l > i && l <= cur) ? s.al[l] : 1.0f;
      }
      if (isq) {
        s.kq[i] = r * part;
        s.rr[i] = r;
      } else {
        s.kk[i] = s.bet * r * part;
      }
    }
  }
  if constexpr (!SM::kVG) {
    if (threadIdx.x == 0) {
      float gm = 1.0f;
#pragma unroll
      for (int e = 0; e < kRing; ++e) gm *= e <= cur ? s.al[e] : 1.0f;
      s.gam = gm;
    }
  }
}

// The held entries' part of row cur and of the output for column v: it needs
// no state, so it is summed while the state tile streams in.
//   hu = sum_{i<cur} kk[i] u_i[v],  ho = sum_{i<cur} kq[i] u_i[v]
template <typename SM>
__device__ __forceinline__ void gdn_held_sums(const SM& s, int m, int v, float& hu, float& ho) {
  const int cur = m - 1;
  hu = 0.0f;
  ho = 0.0f;
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) {   // selects keep every LDS load unconditional
    const float ui = s.U[i][v];
    hu += i < cur ? s.kk[i] * ui : 0.0f;
    ho += i < cur ? s.kq[i] * ui : 0.0f;
  }
}

// After the matvec: u_cur[v] = beta (v_cur - gamma S0 k_cur) - hu, stored in
// U[cur]; returns o[v] = gamma S0 q + ho + kq[cur] u_cur. ms: a scale of the
// matvec's sums (an FP8 matrix scale the matvec left out), else 1.
template <typename SM>
__device__ __forceinline__ float gdn_finish_row(SM& s, int m, int v, float hu, float ho, float ms = 1.0f) {
  const int cur = m - 1;
  const float sk = ms * s.out[0][v], sq = ms * s.out[1][v];
  const float u = s.bet * (s.vc[v] - s.gam * sk) - hu;
  s.U[cur][v] = u;
  return s.gam * sq + ho + s.kq[cur] * u;
}

// S <- S Diag(f) for a [dk][dv] tile: row r (key channel r) times f[r].
template <int NK, int NVS>
__device__ __forceinline__ void tile_scale_rows(RegTile<4, NK, NVS>& S, const float* f) {
#pragma unroll
  for (int k = 0; k < RegTile<4, NK, NVS>::P; ++k) {
    const int row = RegTile<4, NK, NVS>::row(k);
    const float x = f[row < NK ? row : NK - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) S.v[k][i] *= x;
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// conventional step (baseline). VG (KDA): S <- S Diag(alpha) first, then the
// delta update with no further decay.
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_conv_kernel(GDNArgs a) {
  constexpr int NVS = NV;   // whole state per workgroup (measured faster for read + write)
  __shared__ GSmem<NK, NVS> s;
  const GPtrs p = gdn_tile<NV, 1>(a);
  float* ck = static_cast<float*>(a.ck.data);
  static_assert(NK <= kThreads && NVS <= kThreads, "one input element per thread");
  // the token's inputs into registers first, then the state (returns come back
  // in issue order), then the inputs to LDS while the state streams in
  const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
  const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
  const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
  const TIN* iv = static_cast<const TIN*>(a.v) + p.st * NV + p.c0;
  const int ti = static_cast<int>(threadIdx.x);
  const int ik_ = ti < NK ? ti : 0, iv_ = ti < NVS ? ti : 0;
  const float kv = to_f(ik[ik_]), qv = to_f(iq[ik_]), vv = to_f(iv[iv_]);
  const float gvv = VG ? a.g[p.st * NK + ik_] : 0.0f;
  const float gs = VG ? 0.0f : a.g[p.st], beta = a.beta[p.st];
  GSlice<NK, NV, NVS> raw;
  raw.issue(ck, p.st, p.c0);
  if (ti < NK) {
    s.W[0][ti] = kv;
    s.W[1][ti] = qv;
    s.W[2][ti] = VG ? kda_alpha(gvv) : 0.0f;   // VG: the channel decays
    s.W[3][ti] = 0.0f;
  }
  if (ti < NVS) s.vc[ti] = vv;
  __syncthreads();
  // k . q (one 16-lane group)
  if (threadIdx.x < 16) {
    float part = 0.0f;
    for (int n = threadIdx.x; n < NK; n += 16) part += s.W[0][n] * s.W[1][n];
    part = group_sum16(part);
    if (threadIdx.x == 0) s.kq[0] = part;
  }
  const float alpha = VG ? 1.0f : expf(gs);
  RegTile<4, NK, NVS> S;
  raw.decode(S);
  if constexpr (VG) tile_scale_rows(S, &s.W[2][0]);
  tile_matvec<2>(S, &s.W[0][0], NK, s.red, &s.out[0][0]);   // out[0] = S k, out[1] = S q
  for (int v = threadIdx.x; v < NVS; v += kThreads) s.U[0][v] = beta * (s.vc[v] - alpha * s.out[0][v]);
  __syncthreads();
  tile_rank_update(S, alpha, &s.W[0][0], NK, &s.U[0][0], NVS, 1);
  GSlice<NK, NV, NVS>::store(ck, p.st, p.c0, S);
  const float kq = s.kq[0];
  for (int v = threadIdx.x; v < NVS; v += kThreads)
    a.o[p.st * NV + p.c0 + v] = alpha * s.out[1][v] + kq * s.U[0][v];
}

// ----------------------------------------------------------------------------
// non-flush step: o from checkpoint + buffer, append (with its u row), no state write
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV, bool VG, bool RC, int CKF = FMT_F32, int NS = gdn_slices<NV>()>
__device__ __forceinline__ void gdn_nonflush_body(const GDNArgs& a, GSmem<NK, NV / NS, VG>& s) {
  constexpr int NVS = NV / NS;
  const GPtrs p = gdn_tile<NV, NS>(a);
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * NS + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * NS) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 2 ? RS_ERR_FULL : 0);
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, wg, nck, len, nd);
  } else {
    const int j = len + 1;
    GStage<TIN, NK, NV, NVS, VG> stg;
    stg.load(a, p, nck, j);            // records first, then the state tile
    ReadSlice<RC, CKF, NK, NV, NVS> raw;   // the checkpoint slice, or the read copy's
    raw.issue_read(a, p.st, p.c0);
    arr.arrive(actr, wg, nck, len, nd);
    stg.store(s, j);
    __syncthreads();
    if constexpr (VG) {
      kda_decays(s, j);
      __syncthreads();
    }
    gdn_dots(s, j);
    __syncthreads();   // dots visible; VG: the decay table becomes matvec scratch
    static_assert(NVS <= kThreads, "one thread per column");
    const int v = threadIdx.x;
    float hu = 0.0f, ho = 0.0f;
    if (v < NVS) gdn_held_sums(s, j, v, hu, ho);
    // FP8: the matvec runs on the codes' values and the one matrix scale goes
    // on its two sums, not on every element
    float ms = 1.0f;
    if constexpr (RC && NVS == 64) {
      raw.matvec2(&s.W[0][0], NK, s.redp(), &s.out[0][0]);
    } else {
      RegTile<4, NK, NVS> S;
      if constexpr (!RC && CKF == FMT_FP8) {
        raw.decode_values(S);
        ms = raw.ms;
      } else {
        raw.decode(S);
      }
      tile_matvec<2>(S, &s.W[0][0], NK, s.redp(), &s.out[0][0]);
    }
    const int slot = slot_of(nck, len);
    float* ru = static_cast<float*>(a.ru) + (p.st * kRing + slot) * NV + p.c0;
    if (v < NVS) {
      a.o[p.st * NV + p.c0 + v] = gdn_finish_row(s, j, v, hu, ho, ms);
      ru[v] = s.U[j - 1][v];
    }
    // append the current record (bit copies); each slice its own v columns
    TIN* rv = static_cast<TIN*>(a.rv) + (p.st * kRing + slot) * NV + p.c0;
    const TIN* iv = static_cast<const TIN*>(a.v) + p.st * NV + p.c0;
    for (int v = threadIdx.x; v < NVS; v += kThreads) rv[v] = iv[v];
    if (p.half == 0) {
      if constexpr (VG) {
        float* rgv = static_cast<float*>(a.rg) + (p.st * kRing + slot) * NK;
        for (int n = threadIdx.x; n < NK; n += kThreads) rgv[n] = a.g[p.st * NK + n];
      } else if (threadIdx.x == 0) {
        static_cast<float*>(a.rg)[p.st * kRing + slot] = a.g[p.st];
      }
      if (threadIdx.x == 0) static_cast<float*>(a.rbeta)[p.st * kRing + slot] = a.beta[p.st];
      if (p.h % a.vpk == 0) {
        const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
        TIN* rk = static_cast<TIN*>(a.rk) + bk * kRing * NK;
        TIN* rq = static_cast<TIN*>(a.rq) + bk * kRing * NK;
        const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
        const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
        for (int n = threadIdx.x; n < NK; n += kThreads) {
          rk[slot * NK + n] = ik[n];
          rq[slot * NK + n] = iq[n];
        }
      }
    }
  }
  arr.finish(mp, actr, wg, a.nv * NS, MetaOp::NonFlush, 0, nck, len, nd);
}

// Workgroups per state of the non-flush kernel: column slices for fp32 states
// and their read copies; FP16 / FP8 states are small enough for one workgroup,
// which then stages the records and forms the dots once.
template <int NV, bool RC, int CKF>
constexpr int gdn_nonflush_slices() { return RC || CKF != FMT_F32 ? 1 : gdn_slices<NV>(); }

template <typename TIN, int NK, int NV, bool VG, bool RC, int CKF = FMT_F32>
__global__ __launch_bounds__(kThreads) void gdn_nonflush_kernel(GDNArgs a) {
  constexpr int NS = gdn_nonflush_slices<NV, RC, CKF>();
  __shared__ GSmem<NK, NV / NS, VG> s;
  gdn_nonflush_body<TIN, NK, NV, VG, RC, CKF, NS>(a, s);
}

// ----------------------------------------------------------------------------
// flush step: fold the len held entries and the current token, write once, o
// ----------------------------------------------------------------------------
// A flush of the NVS columns c0.. of one state (a column slice, or the whole
// state): the window staged for those columns, the checkpoint's columns read,
// the dots, the matvec, the current row, o, and the rank-m update into S. The
// workgroup counts in through arr once its loads are issued.
template <typename TIN, int CKF, int NK, int NV, int NVS, bool VG>
__device__ __forceinline__ void gdn_flush_cols(const GDNArgs& a, const GPtrs& p, GSmem<NK, NVS, VG>& s, int m,
                                               long long nck, Arrival& arr, uint32_t* actr, int wg, int len, int nd,
                                               GFoldTile<CKF, NK, NV, NVS>& S) {
  GStage<TIN, NK, NV, NVS, VG> stg;
  stg.load(a, p, nck, m);            // records first, then the state tile
  GFoldRaw<CKF, NK, NV, NVS> raw;
  fold_issue(raw, a.ck, p.st, p.c0);
  arr.arrive(actr, wg, nck, len, nd);
  stg.store(s, m);
  __syncthreads();
  if constexpr (VG) {
    kda_decays(s, m);
    __syncthreads();
  }
  gdn_dots(s, m);
  if constexpr (VG) {
    // the fold's decayed k rows r_{m,i} * k_i, made now so that the decay table
    // can serve as matvec scratch
    __syncthreads();
    for (int idx = threadIdx.x; idx < m * NK; idx += kThreads) {
      const int i = idx / NK, c = idx - i * NK;
      s.K[i][c] *= s.A[i][c];
    }
    __syncthreads();
  }
  if constexpr (!VG) __syncthreads();   // dots visible (VG: the barrier above)
  static_assert(NVS <= kThreads, "one thread per column");
  const int v = threadIdx.x;
  float hu = 0.0f, ho = 0.0f;
  if (v < NVS) gdn_held_sums(s, m, v, hu, ho);
  raw.decode(S);
  fold_matvec2(S, &s.W[0][0], NK, s.redp(), &s.out[0][0]);
  if (v < NVS) {
    a.o[p.st * NV + p.c0 + v] = gdn_finish_row(s, m, v, hu, ho);
    if constexpr (!VG) {
      // fold columns r_{cur,i} u_i (same thread, same column v)
#pragma unroll
      for (int i = 0; i < kRing; ++i)
        if (i < m) s.U[i][v] *= s.rr[i];
    }
  }
  __syncthreads();
  // VG: S0 Diag(gamma_m) + sum_i u_i (r_{m,i} * k_i)^T (k rows decayed above)
  if constexpr (gdn_mfma_fold<CKF, NK, NV, NVS>()) {
    if constexpr (VG) mtile_scale_rows(S, s.gv);
    else mtile_scale(S, s.gam);
    mtile_rank_update(S, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  } else if constexpr (VG) {
    tile_scale_rows(S, s.gv);
    tile_rank_update(S, 1.0f, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  } else {
    tile_rank_update(S, s.gam, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  }
}

// Store a whole folded state (held by this workgroup as one tile) into an FP8
// checkpoint with one scale from its |max|. Barriers inside.
template <int NK, int NV, bool VG>
__device__ __forceinline__ void gdn_store_fp8(const GDNArgs& a, size_t st, GSmem<NK, NV, VG>& s,
                                              const RegTile<4, NK, NV>& S) {
  const float sc = fp8_scale_of(tile_absmax(S, s.s4)), y = 1.0f / sc;
  GSliceF<FMT_FP8, NK, NV, NV>::store(a.ck, st, 0, S, sc, y);
  if (threadIdx.x == 0) a.ck.tscale[st] = sc;
}
template <int NK, int NV, bool VG>
__device__ __forceinline__ void gdn_store_fp8(const GDNArgs& a, size_t st, GSmem<NK, NV, VG>& s,
                                              const MTile<NK, NV>& S) {
  mtile_store<FMT_FP8>(a.ck, st, S, s.s4);
}

// flush step: fold the len held entries and the current token, write once, o.
// FP8 checkpoints: one scale spans the matrix, so one workgroup folds the whole
// state in one pass (staged once, one matvec and one rank update over every
// column). NS: workgroups per state in the launch; where it exceeds the
// folding ones (an FP8 flush inside the self-scheduling step), the others only
// count in.
template <typename TIN, int NK, int NV, bool VG, int CKF = FMT_F32, int NS = gdn_slices<NV>()>
__device__ __forceinline__ void gdn_flush_body(const GDNArgs& a, GSmem<NK, gdn_fold_cols<NV, CKF>(), VG>& s) {
  constexpr int NF = gdn_fold_cols<NV, CKF>();
  const GPtrs p = gdn_tile<NV, NS>(a);
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * NS + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * NS) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 1 ? RS_ERR_FULL : 0);
  const int m = len + 1;
  Arrival arr;
  if (errbit != 0 || (NF == NV && p.half != 0)) {
    arr.arrive(actr, wg, nck, len, nd);
  } else {
    // (a whole-state fold runs in the slice-0 workgroup, whose columns start at 0)
    GFoldTile<CKF, NK, NV, NF> S;
    gdn_flush_cols<TIN, CKF, NK, NV, NF, VG>(a, p, s, m, nck, arr, actr, wg, len, nd, S);
    if constexpr (CKF == FMT_FP8) gdn_store_fp8(a, p.st, s, S);
    else GSliceF<CKF, NK, NV, NF>::store(a.ck, p.st, p.c0, S);
  }
  arr.finish(mp, actr, wg, a.nv * NS, MetaOp::Flush, 0, nck, len, nd);
}

template <typename TIN, int NK, int NV, bool VG, int CKF = FMT_F32>
__global__ __launch_bounds__(kThreads) void gdn_flush_kernel(GDNArgs a) {
  __shared__ GSmem<NK, gdn_fold_cols<NV, CKF>(), VG> s;
  gdn_flush_body<TIN, NK, NV, VG, CKF, gdn_flush_slices<NV, CKF>()>(a, s);
}

template <int NK, int NV, bool VG, int CKF>
union GAutoSmem {
  GSmem<NK, NV / gdn_slices<NV>(), VG> nf;
  GSmem<NK, gdn_fold_cols<NV, CKF>(), VG> fl;
};

// self-scheduling step (continuous batching): a sequence whose buffer is full
// takes the flush, every other one a non-flush step, in one launch (the branch
// is uniform per workgroup)
template <typename TIN, int NK, int NV, bool VG, int CKF = FMT_F32>
__global__ __launch_bounds__(kThreads) void gdn_auto_kernel(GDNArgs a) {
  __shared__ GAutoSmem<NK, NV, VG, CKF> s;
  const GPtrs p = gdn_tile<NV, gdn_slices<NV>()>(a);
  if (a.meta[p.b].len == kRing - 1) gdn_flush_body<TIN, NK, NV, VG, CKF>(a, s.fl);
  else gdn_nonflush_body<TIN, NK, NV, VG, false, CKF>(a, s.nf);
}

// ----------------------------------------------------------------------------
// speculative append (ReplaySSM): K drafts at window entries len..len+K-1. Each
// draft's u row is solved in order (it depends on S0 and the entries before
// it), its output read from the checkpoint and the buffer, and the drafts are
// written to the ring with their u rows; no state is written. Because a u row
// depends only on S0 and earlier entries, the rows of an accepted prefix stay
// valid after the commit (sitech.ge ReplaySSM page, "Reducing state traffic
// and simplifying rollback": drafts are appended until verification, the
// verification outputs need no intermediate state).
// ----------------------------------------------------------------------------
namespace {

template <int NK, int NVS, int KQ, bool VG>
struct alignas(16) GSpecSmem {
  // k of window entries 0..n-1 (held, then drafts) for the dots; once they are
  // done, the same space is the matvec scratch (4 KQ NVS floats), and after the
  // matvecs the held-entry sums HU, HO (KQ NVS floats each)
  static constexpr int KROWS = (4 * KQ * NVS + NK - 1) / NK > kRing ? (4 * KQ * NVS + NK - 1) / NK : kRing;
  alignas(16) float K[KROWS][NK];
  alignas(16) float W[2 * KQ][NK];         // matvec weights k_d, q_d per draft (zero past K)
  float U[kRing][NVS];         // u rows, own columns (held from the ring, drafts solved here)
  float kk[KQ][kRing];         // beta_d r_{e,i} (k_e . k_i) for i < e = len + d
  float kq[KQ][kRing];         // r_{e,i} (k_i . q_d) for i <= e
  float rt[KQ][kRing];         // r_{e,i} for i <= e
  float al[kRing];             // alpha of window entry e
  float gam[KQ];               // gamma of draft d's entry (VG: 1, the decays weight the dots)
  float bet[KQ];
  // VG (per-channel decays, e = len + d): WS = k_e * P_d and q_d * P_d with
  // P_d = prod_{len<=l<=e} alpha_l; DW[d(d-1)/2 + j] = prod_{len+j<l<=e} alpha_l
  // (the decay between draft j and draft d > j). They live only while the dots
  // are taken; the drafts' v rows and the matvec outputs are written after
  // that (with VG the v rows wait in registers), so the two share space.
  struct Dots {
    alignas(16) float WS[VG ? 2 * KQ : 1][NK];
    alignas(16) float DW[VG && KQ > 1 ? KQ * (KQ - 1) / 2 : 1][NK];
  };
  struct Mv {
    float V[KQ][NVS];          // v of the drafts, own columns
    float out[2 * KQ][NVS];    // S0 k_d, S0 q_d
  };
  union {
    Dots dots;
    Mv mv;
  };
};

// The dots of a speculative round on the matrix cores, for bf16 records (their
// products are exact in fp32; only the accumulation order differs from the
// lane-group dots). One wavefront forms G = A Bt^T with A's rows 0..K-1 the
// drafts' k (window entries len + d), rows 8..8+K-1 their q, the rest zero, and
// Bt's rows the window's 16 k rows, in steps of 32 of v_mfma_f32_16x16x32_bf16
// (a short last step zero-padded). Operand lane layout of that instruction: lane l
// holds row l % 16 of A (of Bt) at k = 8 (l / 16) .. + 7 of each 32-wide step;
// the result lane l holds column l % 16, rows 4 (l / 16) .. + 3 (checked against
// a host product before use). Then kk[d][i] = beta_d r_{e,i} (k_e . k_i) for
// i < e and kq[d][i] = r_{e,i} (k_i . q_d) for i <= e, e = len + d; entries past
// the window are garbage in G and never read. Called by lanes 0..63 only.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t bf16x8_of(const float* p) {
  const float4 u = *reinterpret_cast<const float4*>(p), v = *reinterpret_cast<const float4*>(p + 4);
  const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i)   // the values are bf16 already: keep the upper half
    r[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(__float_as_uint(f[i]) >> 16));
  return r;
}

template <int NK, int KQ, typename SM>
__device__ __forceinline__ void spec_gram_bf16(SM& s, int K, int len) {
  static_assert(NK % 8 == 0 && KQ <= 8, "8-element lane chunks; at most 8 drafts");
  const int l = threadIdx.x, row = l & 15, k8 = 8 * (l >> 4);
  const bool isk = row < 8;
  const int d = isk ? row : row - 8;
  const bool live = d < K;
  const float* arow = isk ? &s.K[(len + d) & (kRing - 1)][0] : &s.W[2 * (d < KQ ? d : 0) + 1][0];
  const float* brow = &s.K[row][0];
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8_t zero;
#pragma unroll
  for (int i = 0; i < 8; ++i) zero[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
#pragma unroll
  for (int st = 0; st < (NK + 31) / 32; ++st) {
    const bool in = 32 * st + k8 < NK;   // a short last step is zero-padded
    const bf16x8_t av = live && in ? bf16x8_of(arow + 32 * st + k8) : zero;
    const bf16x8_t bv = in ? bf16x8_of(brow + 32 * st + k8) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
  const int i = l & 15;           // window entry (column)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * (l >> 4) + j;  // A row
    if (m < 8) {
      if (m < K && i < len + m) s.kk[m][i] = s.bet[m] * s.rt[m][i] * acc[j];
    } else if (m - 8 < K && i <= len + m - 8) {
      s.kq[m - 8][i] = s.rt[m - 8][i] * acc[j];
    }
  }
}

// out[m][col] = sum_rows S[row][col] * w[m * ws + row] for m < Q <= 16, the
// state slice held as RegTile<4, NK, 64> (16 threads per row, four columns
// each), on the matrix cores: in a wavefront, lane l holds rows
// 4 wave + l / 16 + 16 k and columns 4 (l % 16) + c, which is, for each pass k
// and column offset c, the B operand of v_mfma_f32_16x16x4f32 (B[l / 16][l % 16]);
// the A operand is w[l % 16][that row]. Each wavefront sums its 32 rows inside
// the instruction; the four wavefronts' partials meet in `red` (4 Q 64 floats of
// LDS). fp32 products and sums: only the order of the additions differs from
// tile_matvec. Barriers inside; all threads must call.
template <int Q, int NK, int NVS, bool HALF_RED = false, bool W_IN_RED = false>
__device__ __forceinline__ void tile_matvec_mfma(const RegTile<4, NK, NVS>& S, const float* w, int ws, float* red,
                                                 float* out) {
  static_assert(NVS == 64 && Q <= 16, "16 lanes per row of four columns; at most 16 weight rows");
  constexpr int P = RegTile<4, NK, NVS>::P;
  const int l = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = l & 15;
  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int row = RegTile<4, NK, NVS>::row(k);
    const float a = (m < Q && row < NK) ? w[m * ws + row] : 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, row < NK ? S.v[k][c] : 0.0f,
                                                                              acc[c], 0, 0, 0);
  }
  // lane l: column 4 (l % 16) + c, rows 4 (l / 16) + i of the wavefront's partial
  if constexpr (HALF_RED) {
    // in two steps through 2 Q NVS floats of scratch: waves 2, 3 leave their
    // partials, waves 0, 1 add theirs, then the two halves meet (W_IN_RED: the
    // weight rows share the scratch, so every wave has read them first)
    if constexpr (W_IN_RED) __syncthreads();
    if (wave >= 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = 4 * (l >> 4) + i;
        if (mr < Q)
          *reinterpret_cast<float4*>(red + ((wave - 2) * Q + mr) * NVS + 4 * (l & 15)) =
              make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      }
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = 4 * (l >> 4) + i;
        if (mr < Q) {
          float4* dst = reinterpret_cast<float4*>(red + (wave * Q + mr) * NVS + 4 * (l & 15));
          const float4 o = *dst;
          *dst = make_float4(acc[0][i] + o.x, acc[1][i] + o.y, acc[2][i] + o.z, acc[3][i] + o.w);
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Q * NVS; idx += kThreads) out[idx] = red[idx] + red[Q * NVS + idx];
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mr = 4 * (l >> 4) + i;
      if (mr < Q) {
        float* dst = red + (wave * Q + mr) * NVS + 4 * (l & 15);
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Q * NVS; idx += kThreads)
      out[idx] = (red[idx] + red[Q * NVS + idx]) + (red[2 * Q * NVS + idx] + red[3 * Q * NVS + idx]);
    __syncthreads();
  }
}

}  // namespace

// The K drafts' records of one speculative round in one set of register
// chunks: thread chunk q < K NK / VK is a chunk of the drafts' q, the next K NK
// / VK are their k, then K NVS / VK of their v (this slice's columns), so that
// threads hold at most ceil((2 KQ NK + KQ NVS) / VK / 256) chunks instead of one
// set per record kind. Chunks past the round's records load the first q chunk
// (a valid address) and are never stored.
template <typename TIN, int NK, int NVS, int KQ>
struct DraftChunks {
  static constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  static constexpr int CH = ((2 * KQ * NK + KQ * NVS) / VK + kThreads - 1) / kThreads;
  uint4 c[CH];
  __device__ __forceinline__ void load(const TIN* iq, const TIN* ik, size_t kstride, const TIN* iv, size_t vstride,
                                       int K) {
    const int qn = K * (NK / VK), vn = K * (NVS / VK);
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      int q = static_cast<int>(threadIdx.x) + r * kThreads;
      const TIN* src;
      if (q < 2 * qn) {
        const int part = q < qn ? 0 : 1;
        q -= part * qn;
        const int e = q / (NK / VK), k = q - e * (NK / VK);
        src = (part ? ik : iq) + e * kstride + k * VK;
      } else if (q < 2 * qn + vn) {
        q -= 2 * qn;
        const int e = q / (NVS / VK), k = q - e * (NVS / VK);
        src = iv + e * vstride + k * VK;
      } else {
        src = iq;
      }
      c[r] = *reinterpret_cast<const uint4*>(src);
    }
  }
  // q of draft d to row 2 d + 1 of W, its k to row 2 d (rows of NK floats)
  __device__ __forceinline__ void qk_to_lds(float* W, int K) const {
    const int qn = K * (NK / VK);
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      int q = static_cast<int>(threadIdx.x) + r * kThreads;
      if (q < 2 * qn) {
        const int part = q < qn ? 0 : 1;
        q -= part * qn;
        const int e = q / (NK / VK), k = q - e * (NK / VK);
        float t[VK];
        unpack16(c[r], static_cast<const TIN*>(nullptr), t);
#pragma unroll
        for (int i = 0; i < VK; ++i) W[(2 * e + 1 - part) * NK + k * VK + i] = t[i];
      }
    }
  }
  // The records into the ring as they came (bit copies), draft d at slot
  // slot(d): q and k (rows of NK) when qk is set, v (this slice's NVS
  // columns of rows of NV) always.
  template <int NV, typename SLOT>
  __device__ __forceinline__ void to_ring(TIN* rq, TIN* rk, TIN* rv, bool qk, int K, SLOT slot) const {
    const int qn = K * (NK / VK), vn = K * (NVS / VK);
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      int q = static_cast<int>(threadIdx.x) + r * kThreads;
      TIN* dst = nullptr;
      if (q < 2 * qn) {
        const int part = q < qn ? 0 : 1;
        q -= part * qn;
        const int e = q / (NK / VK), k = q - e * (NK / VK);
        if (qk) dst = (part ? rk : rq) + static_cast<size_t>(slot(e)) * NK + k * VK;
      } else if (q < 2 * qn + vn) {
        q -= 2 * qn;
        const int e = q / (NVS / VK), k = q - e * (NVS / VK);
        dst = rv + static_cast<size_t>(slot(e)) * NV + k * VK;
      }
      if (dst) *reinterpret_cast<uint4*>(dst) = c[r];
    }
  }
  // v of draft d to row d of V (rows of NVS floats)
  __device__ __forceinline__ void v_to_lds(float* V, int K) const {
    const int qn = K * (NK / VK), vn = K * (NVS / VK);
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      int q = static_cast<int>(threadIdx.x) + r * kThreads - 2 * qn;
      if (q >= 0 && q < vn) {
        const int e = q / (NVS / VK), k = q - e * (NVS / VK);
        float t[VK];
        unpack16(c[r], static_cast<const TIN*>(nullptr), t);
#pragma unroll
        for (int i = 0; i < VK; ++i) V[e * NVS + k * VK + i] = t[i];
      }
    }
  }
};

// Without the per-channel gate and up to 4 drafts: 7 waves per SIMD with the
// matrix-core accumulators, the register budget the VALU dots and matvecs had;
// otherwise the compiler puts the accumulators in separate registers and
// occupancy drops.
template <typename TIN, int NK, int NV, int KQ, bool VG, bool RC, int CKF = FMT_F32>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu((!VG && KQ <= 4) ? 7 : 1, 8)))
void gdn_spec_append_kernel(GDNArgs a) {
  constexpr int NS = gdn_slices<NV>();
  constexpr int NVS = NV / NS;
  constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NK % VK == 0 && NVS % VK == 0, "records are whole 16-byte chunks");
  constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  constexpr int CU = (kRing * NVS / 4 + kThreads - 1) / kThreads;
  __shared__ GSpecSmem<NK, NVS, KQ, VG> s;
  const GPtrs p = gdn_tile<NV, NS>(a);
  const int K = a.K;
  static_assert(!VG || 2 * NK <= kThreads, "two threads per key channel");
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * NS + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * NS) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = (nd != 0 || len + K > kRing) ? RS_ERR_OVERFLOW : 0;
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, wg, nck, len, nd);
  } else {
    const int n = len + K;
    const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
    const size_t kstride = static_cast<size_t>(a.batch) * a.nqk * NK;   // between drafts (q, k)
    const size_t vstride = static_cast<size_t>(a.batch) * a.nv * NV;    // between drafts (v, o)
    const size_t gstride = static_cast<size_t>(a.batch) * a.nv;         // between drafts (g, beta)
    const TIN* rk = static_cast<const TIN*>(a.rk) + bk * kRing * NK;
    const float* ru = static_cast<const float*>(a.ru) + p.st * kRing * NV + p.c0;
    const float* rg = static_cast<const float*>(a.rg) + p.st * kRing;
    const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
    const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
    const TIN* iv = static_cast<const TIN*>(a.v) + p.st * NV + p.c0;
    // records into registers, then the state slice, then records to LDS
    RegChunks<TIN, CK> ck;
    RegChunks<float, CU> cu;
    DraftChunks<TIN, NK, NVS, KQ> cdr;
    ck.load(EntrySrc<TIN>{rk, ik, kstride, nck, len, NK}, n, NK);
    cu.load(EntrySrc<float>{ru, ru, 0, nck, len, NV}, len, NVS);
    cdr.load(iq, ik, kstride, iv, vstride, K);
    float gv = 0.0f;
    float lg[kRing];   // VG: the log decays of window entries 0..n-1 of this thread's key channel
    if constexpr (VG) {
      const int c = static_cast<int>(threadIdx.x) % NK;
      const float* rgc = static_cast<const float*>(a.rg) + p.st * kRing * NK + c;
      const float* igc = a.g + p.st * NK + c;
#pragma unroll
      for (int e = 0; e < kRing; ++e) {
        const int ee = e < n ? e : n - 1;
        lg[e] = ee < len ? rgc[slot_of(nck, ee) * NK] : igc[static_cast<size_t>(ee - len) * gstride * NK];
      }
    } else {
      const int e = static_cast<int>(threadIdx.x) < n ? static_cast<int>(threadIdx.x) : n - 1;
      gv = *(e < len ? rg + slot_of(nck, e) : a.g + static_cast<size_t>(e - len) * gstride + p.st);
    }
    const int dd = static_cast<int>(threadIdx.x) < K ? static_cast<int>(threadIdx.x) : K - 1;
    const float bv = a.beta[static_cast<size_t>(dd) * gstride + p.st];
    ReadSlice<RC, CKF, NK, NV, NVS> raw;   // the checkpoint slice, or the read copy's
    raw.issue_read(a, p.st, p.c0);
    arr.arrive(actr, wg, nck, len, nd);
    ck.to_lds(&s.K[0][0], NK, n, NK);
    cu.to_lds(&s.U[0][0], NVS, len, NVS);
    cdr.qk_to_lds(&s.W[0][0], K);
    for (int idx = 2 * K * NK + threadIdx.x; idx < 2 * KQ * NK; idx += kThreads) (&s.W[0][0])[idx] = 0.0f;
    if constexpr (!VG) cdr.v_to_lds(&s.mv.V[0][0], K);
    // the drafts' records into the ring now, from the registers (this launch reads
    // none of those slots; q and k rows are shared by the value heads of a
    // key head, one slice of one of which writes them)
    const auto dslot = [&](int d) { return slot_of(nck, len + d); };
    cdr.template to_ring<NV>(static_cast<TIN*>(a.rq) + bk * kRing * NK, static_cast<TIN*>(a.rk) + bk * kRing * NK,
                             static_cast<TIN*>(a.rv) + p.st * kRing * NV + p.c0, p.half == 0 && p.h % a.vpk == 0,
                             K, dslot);
    if constexpr (VG) {
      // the raw log decays, each from its own register (an index that is not
      // a constant would make the wait before these stores one for every
      // load in flight, the state tile's included)
      if (p.half == 0 && static_cast<int>(threadIdx.x) < NK) {
        float* rgw = static_cast<float*>(a.rg) + p.st * kRing * NK + threadIdx.x;
#pragma unroll
        for (int e = 0; e < kRing; ++e)
          if (e >= len && e < n) rgw[static_cast<size_t>(slot_of(nck, e)) * NK] = lg[e];
      }
    }
    if constexpr (!VG)
      if (static_cast<int>(threadIdx.x) < n) s.al[threadIdx.x] = expf(gv);
    if (static_cast<int>(threadIdx.x) < K) s.bet[threadIdx.x] = bv;
    __syncthreads();
    if constexpr (VG) {
      // The decay from entry i to draft entry e = len + d factors at the first
      // draft: r_{e,i} = Rh_i * P_d for a held entry (Rh_i = prod_{i<l<len}
      // alpha_l), and DW for a pair of drafts. Two threads per key channel hold
      // its window decays in registers: thread c scales the held k rows by Rh
      // in place (and keeps Gam = prod_{l<len} alpha_l), thread NK + c writes
      // WS and DW. Then every dot of every draft in one pass:
      //   kk[d][i] = beta_d <k_e, r_{e,i} * k_i>,  kq[d][i] = <q_d, r_{e,i} * k_i>.
      // gamma_e = Gam * P_d.
      const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
      float gam_c = 1.0f;
      if (static_cast<int>(threadIdx.x) < NK) {
        const int c = threadIdx.x;
        float acc = 1.0f;
#pragma unroll
        for (int i = kRing - 1; i >= 0; --i) {
          if (i < len) {
            s.K[i][c] *= acc;
            acc *= kda_alpha(lg[i]);
          }
        }
        gam_c = acc;
      } else if (static_cast<int>(threadIdx.x) < 2 * NK) {
        const int c = threadIdx.x - NK;
        float pd = 1.0f;
        for (int d = 0; d < K; ++d) {
          pd *= kda_alpha(lg[len + d]);           // len + d < 16; wave-uniform index
          s.dots.WS[2 * d][c] = s.W[2 * d][c] * pd;
          s.dots.WS[2 * d + 1][c] = s.W[2 * d + 1][c] * pd;
          float q = 1.0f;
          for (int j = d - 1; j >= 0; --j) {
            q *= kda_alpha(lg[len + j + 1]);
            s.dots.DW[d * (d - 1) / 2 + j][c] = q;
          }
        }
      }
      if (static_cast<int>(threadIdx.x) < K) s.gam[threadIdx.x] = 1.0f;
      __syncthreads();
      // Held entry i: one 16-lane group takes its dots with all 2 K rows of WS
      // (row 2 d + isq; the k row, already scaled by Rh_i, is read once). Then
      // for each draft d its d draft kk and d + 1 draft kq pairs, K^2 in all.
      for (int i = grp; i < len; i += kThreads / 16) {
        float part[2 * KQ];
#pragma unroll
        for (int row = 0; row < 2 * KQ; ++row)
          part[row] = row < 2 * K ? lds_dot16<NK>(&s.K[i][0], &s.dots.WS[row][0], ln) : 0.0f;
#pragma unroll
        for (int row = 0; row < 2 * KQ; ++row) {
          if (row < 2 * K) {
            const float v = group_sum16(part[row]);
            if (ln == 0) {
              if (row & 1) s.kq[row >> 1][i] = v;
              else s.kk[row >> 1][i] = s.bet[row >> 1] * v;
            }
          }
        }
      }
      for (int t = grp; t < K * K; t += kThreads / 16) {
        const int d = static_cast<int>(sqrtf(static_cast<float>(t) + 0.5f));   // t in [d^2, (d + 1)^2)
        const int r = t - d * d;
        const bool isq = r >= d;                  // earlier draft j (kk: j < d; kq: j <= d)
        const int j = isq ? r - d : r;
        const int i = len + j, ee = len + d;
        const float* w = j < d ? &s.dots.DW[d * (d - 1) / 2 + j][0] : nullptr;
        const float part = group_sum16(lds_dot16<NK>(&s.K[i][0], isq ? &s.W[2 * d + 1][0] : &s.K[ee][0], ln, w));
        if (ln == 0) {
          if (isq) s.kq[d][i] = part;
          else s.kk[d][i] = s.bet[d] * part;
        }
      }
      __syncthreads();
      // matvec weights gamma_e * k_e and gamma_e * q_d (owners: their channel)
      if (static_cast<int>(threadIdx.x) < NK) {
        for (int d = 0; d < K; ++d) {
          s.W[2 * d][threadIdx.x] = s.dots.WS[2 * d][threadIdx.x] * gam_c;
          s.W[2 * d + 1][threadIdx.x] = s.dots.WS[2 * d + 1][threadIdx.x] * gam_c;
        }
      }
    } else {
      // decays r_{e,i} = prod_{i<l<=e} alpha_l and gamma_e = prod_{l<=e} alpha_l for
      // draft d (e = len + d): thread 16 d + i holds alpha_i (1 past e), and the
      // suffix products over its 16-lane row give both (every lane takes part)
      static_assert(KQ * kRing <= kThreads, "one thread per (draft, entry)");
      {
        const int d = static_cast<int>(threadIdx.x) / kRing, i = static_cast<int>(threadIdx.x) % kRing;
        const int ee = len + d;
        const float ai = d < K && i <= ee ? s.al[i] : 1.0f;
        const float suf = row_suffix_prod16(ai);
        const float r = row_next16(suf);
        if (d < K && i <= ee) {
          s.rt[d][i] = r;
          if (i == 0) s.gam[d] = suf;
        }
      }
      __syncthreads();
      if constexpr (sizeof(TIN) == 2) {
        // bf16 records: all the round's dots are one 16 x 16 block of a small
        // GEMM, [k of the drafts; q of the drafts] times the window's k rows,
        // taken by one wavefront on the matrix cores
        if (threadIdx.x < 64) spec_gram_bf16<NK, KQ>(s, K, len);
      } else {
      // dots per draft d (entry e = len + d), 16-lane groups
      const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
      for (int pr = grp; pr < K * 2 * kRing; pr += kThreads / 16) {
        const int d = pr / (2 * kRing), rem = pr - d * 2 * kRing;
        const bool isq = rem >= kRing;
        const int i = isq ? rem - kRing : rem;
        const int ee = len + d;
        if (isq ? i > ee : i >= ee) continue;   // uniform over the group
        const float* other = isq ? &s.W[2 * d + 1][0] : &s.K[ee][0];
        float part = lds_dot16<NK>(&s.K[i][0], other, ln);
        part = group_sum16(part);
        if (ln == 0) {
          if (isq) s.kq[d][i] = s.rt[d][i] * part;
          else s.kk[d][i] = s.bet[d] * s.rt[d][i] * part;
        }
      }
      }
    }
    float* red = &s.K[0][0];
    float* HU = red;                 // [KQ][NVS], after the matvecs
    float* HO = red + KQ * NVS;      // [KQ][NVS]
    __syncthreads();                 // dots done: the k rows become scratch
    if constexpr (VG) cdr.v_to_lds(&s.mv.V[0][0], K);   // over WS (the matvec's barriers publish it)
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    // S0 [k_d, q_d]: all 2 KQ weight rows in one pass on the matrix cores where the
    // slice has 64 columns and the scratch holds it (without the per-channel gate:
    // with it the accumulators cost a wave of occupancy); otherwise on the VALU, rows
    // 0..KQ-1, then KQ..2KQ-1 if drafts reach them (fewer accumulator registers and
    // half the scratch of one 2KQ-row pass). Barriers inside publish the dots.
    constexpr bool kMfmaMv = NVS == 64 && 4 * 2 * KQ * NVS <= GSpecSmem<NK, NVS, KQ, VG>::KROWS * NK;
    if constexpr (kMfmaMv) {
      tile_matvec_mfma<2 * KQ>(S, &s.W[0][0], NK, red, &s.mv.out[0][0]);
    } else {
      tile_matvec<KQ>(S, &s.W[0][0], NK, red, &s.mv.out[0][0]);
      if (2 * K > KQ) tile_matvec<KQ>(S, &s.W[KQ][0], NK, red, &s.mv.out[KQ][0]);
    }
    // every (draft, column) pair at once: the parts of the draft's row and output
    // that do not involve other drafts (checkpoint and held entries)
    for (int idx = threadIdx.x; idx < K * NVS; idx += kThreads) {
      const int d = idx / NVS, v = idx - d * NVS;
      float hu = 0.0f, ho = 0.0f;
#pragma unroll 4
      for (int i = 0; i < len; ++i) {
        const float ui = s.U[i][v];
        hu += s.kk[d][i] * ui;
        ho += s.kq[d][i] * ui;
      }
      HU[d * NVS + v] = s.bet[d] * (s.mv.V[d][v] - s.gam[d] * s.mv.out[2 * d][v]) - hu;
      HO[d * NVS + v] = s.gam[d] * s.mv.out[2 * d + 1][v] + ho;
    }
    __syncthreads();
    // the drafts' rows in order (each depends on the drafts before it), one
    // thread per column with the earlier rows in registers
    float* ruw = static_cast<float*>(a.ru) + p.st * kRing * NV + p.c0;
    for (int v = threadIdx.x; v < NVS; v += kThreads) {
      float ur[KQ];
#pragma unroll
      for (int d = 0; d < KQ; ++d) {
        if (d < K) {
          float u = HU[d * NVS + v];
#pragma unroll
          for (int j = 0; j < d; ++j) u -= s.kk[d][len + j] * ur[j];   // len + j < len + K <= 16
          ur[d] = u;
          s.U[len + d][v] = u;
          ruw[slot_of(nck, len + d) * NV + v] = u;
        }
      }
    }
    __syncthreads();
    // outputs, every (draft, column) pair at once
    for (int idx = threadIdx.x; idx < K * NVS; idx += kThreads) {
      const int d = idx / NVS, v = idx - d * NVS;
      float o = HO[d * NVS + v];
#pragma unroll
      for (int j = 0; j < KQ; ++j)   // drafts up to this one: entries len .. len + d
        o += j <= d ? s.kq[d][len + j < kRing ? len + j : kRing - 1] * s.U[len + j < kRing ? len + j : kRing - 1][v]
                    : 0.0f;
      a.o[d * vstride + p.st * NV + p.c0 + v] = o;
    }
    // the drafts' gates and betas into the ring (the records went earlier)
    if (p.half == 0 && static_cast<int>(threadIdx.x) < K) {
      const int d = threadIdx.x, sl = slot_of(nck, len + d);
      if constexpr (!VG) static_cast<float*>(a.rg)[p.st * kRing + sl] = a.g[d * gstride + p.st];
      static_cast<float*>(a.rbeta)[p.st * kRing + sl] = a.beta[d * gstride + p.st];
    }
  }
  arr.finish(mp, actr, wg, a.nv * NS, MetaOp::Append, K, nck, len, nd);
}

// ----------------------------------------------------------------------------
// Folds with a read copy. The non-flush steps and appends solved their rows u
// from the read copy, so a fold re-solves the rows of its m entries from the
// fp32 checkpoint before folding (sitech.ge ReplaySSM page, "Bounding
// quantization error": the read error must not enter the recurrence):
//   (I + L) U = diag(beta) (V - diag(gamma) K S0^T),  L_{t,i} = beta_t r_{t,i} (k_t . k_i)
// (KDA: the per-channel decays weight the dots, L_{t,i} = beta_t <k_t, r_{t,i} * k_i>,
// and the matvec rows, S0 (gamma_t * k_t)). S0 times all the rows in one pass
// (on the matrix cores for 64-column slices), forward substitution per column,
// then the fold as in the steps without a copy.
// ----------------------------------------------------------------------------
namespace {

// NVS: the columns of one matvec; NU: the columns held (NU = 2 NVS when one
// workgroup folds a whole state as two 64-column halves).
template <int NK, int NVS, bool VG, int NU = NVS>
struct alignas(16) GRcSmem {
  static constexpr bool kWtInRed = NVS == 64 && NU == NVS;   // the matvec reads its rows once
  alignas(16) float K[kRing][NK];            // k rows of entries 0..m-1 (VG: then times r_{m-1,i})
  alignas(16) float q[NK];                   // flush: q of the current token
  float U[kRing][NU];                        // v rows, then the solved rows u (own columns)
  // matvec scratch (the matrix-core matvec adds in two steps), and over its
  // start the result: each output element is written by the thread that last
  // reads the scratch at that index
  union {
    alignas(16) float red[(NVS == 64 ? 2 : 4) * kRing * NVS];
    alignas(16) float out[kRing][NVS];       // S0 times the matvec rows
    alignas(16) float Wt[VG && kWtInRed ? kRing : 1][NK];   // VG: matvec rows gamma_t * k_t, until the matvec reads them
  };
  alignas(16) float Wt2[VG && !kWtInRed ? kRing : 1][NK];  // VG, otherwise: the rows apart
  __device__ __forceinline__ float* wt() {
    if constexpr (kWtInRed) return &Wt[0][0];
    else return &Wt2[0][0];
  }
  float kk[kRing][kRing];                    // L_{t,i}, i < t
  float al[kRing], bt[kRing], gam[kRing], rr[kRing];
  alignas(16) float A[VG ? kRing : 1][NK];   // VG: alpha of entry e on channel c
  float gv[VG ? NK : 1];                     // VG: gamma_{m-1} per channel
  float s4[4];
};

// The entries of a fold in registers, then LDS: entries 0..held-1 from the
// ring, and, with cur, entry held the current token. Own columns of v.
template <typename TIN, int NK, int NV, int NVS, bool VG>
struct GRcStage {
  static constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  static constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  static constexpr int CV = (kRing * NVS / VK + kThreads - 1) / kThreads;
  static constexpr int CQ = (NK / VK + kThreads - 1) / kThreads;
  static constexpr int CG = VG ? (kRing * NK / 4 + kThreads - 1) / kThreads : 1;
  RegChunks<TIN, CK> k;
  RegChunks<TIN, CV> v;
  RegChunks<TIN, CQ> q;
  RegChunks<float, CG> gr;
  float g = 0.0f, beta = 0.0f;

  __device__ __forceinline__ void load(const GDNArgs& a, size_t st, int b, int kh, int c0, long long nck, int held,
                                       bool cur) {
    const int m = held + (cur ? 1 : 0);
    const size_t bk = static_cast<size_t>(b) * a.nqk + kh;
    const TIN* rk = static_cast<const TIN*>(a.rk) + bk * kRing * NK;
    const TIN* rv = static_cast<const TIN*>(a.rv) + st * kRing * NV + c0;
    const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
    const TIN* iv = static_cast<const TIN*>(a.v) + st * NV + c0;
    k.load(EntrySrc<TIN>{rk, ik, 0, nck, held, NK}, m, NK);
    v.load(EntrySrc<TIN>{rv, iv, 0, nck, held, NV}, m, NVS);
    const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
    if (cur) q.load(EntrySrc<TIN>{iq, iq, 0, 0, 0, NK}, 1, NK);
    const int e = static_cast<int>(threadIdx.x) < m ? static_cast<int>(threadIdx.x) : m - 1;
    if constexpr (VG) {
      const float* rgv = static_cast<const float*>(a.rg) + st * kRing * NK;
      gr.load(EntrySrc<float>{rgv, a.g + st * NK, 0, nck, held, NK}, m, NK);
    } else {
      g = e < held ? static_cast<const float*>(a.rg)[st * kRing + slot_of(nck, e)] : a.g[st];
    }
    beta = e < held ? static_cast<const float*>(a.rbeta)[st * kRing + slot_of(nck, e)] : a.beta[st];
  }
  template <typename SM>
  __device__ __forceinline__ void store(SM& s, int m, bool cur) const {
    k.to_lds(&s.K[0][0], NK, m, NK);
    v.to_lds(&s.U[0][0], NVS, m, NVS);
    if (cur) q.to_lds(s.q, NK, 1, NK);
    if constexpr (VG) gr.to_lds(&s.A[0][0], NK, m, NK);
    if (static_cast<int>(threadIdx.x) < m) {
      if constexpr (!VG) s.al[threadIdx.x] = expf(g);
      s.bt[threadIdx.x] = beta;
    }
  }
};

// After the staging is visible: gates, the matvec rows and L. Rows past m are
// zeroed (the matvec takes all 16). Barrier at the end.
template <int NK, int NVS, bool VG, int NU>
__device__ __forceinline__ void rc_gates_and_gram(GRcSmem<NK, NVS, VG, NU>& s, int m) {
  if constexpr (VG) {
    // alpha per entry and channel, then gamma_t * k_t (direct products in entry order)
    for (int idx = threadIdx.x; idx < m * NK; idx += kThreads) (&s.A[0][0])[idx] = kda_alpha((&s.A[0][0])[idx]);
    __syncthreads();
    for (int c = threadIdx.x; c < NK; c += kThreads) {
      float acc = 1.0f;
      for (int t = 0; t < m; ++t) {
        acc *= s.A[t][c];
        s.wt()[t * NK + c] = acc * s.K[t][c];
      }
      s.gv[c] = acc;
    }
    for (int idx = m * NK + threadIdx.x; idx < kRing * NK; idx += kThreads) s.wt()[idx] = 0.0f;
  } else {
    if (static_cast<int>(threadIdx.x) < m) {
      const int t = threadIdx.x;
      float g = 1.0f, r = 1.0f;
      for (int l = 0; l < m; ++l) {
        if (l <= t) g *= s.al[l];
        if (l > t) r *= s.al[l];
      }
      s.gam[t] = g;
      s.rr[t] = r;   // r_{m-1,t}
    }
    for (int idx = m * NK + threadIdx.x; idx < kRing * NK; idx += kThreads) (&s.K[0][0])[idx] = 0.0f;
  }
  const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
  if constexpr (VG) {
    // L_{t,i} for i < t < m, one row t per 16-lane group: walking i down from
    // t - 1, each lane keeps the decays r_{t,i} = prod_{i<l<=t} alpha_l of its
    // channels ln + 16 j as running products (one multiply per pair and channel)
    static_assert(NK % 16 == 0, "16 lanes over the key channels");
    constexpr int CPL = NK / 16;
    for (int t = grp; t < m; t += kThreads / 16) {
      float kt[CPL], r[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        kt[j] = s.K[t][ln + 16 * j];
        r[j] = 1.0f;
      }
      for (int i = t - 1; i >= 0; --i) {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          r[j] *= s.A[i + 1][ln + 16 * j];
          part += kt[j] * (r[j] * s.K[i][ln + 16 * j]);
        }
        part = group_sum16(part);
        if (ln == 0) s.kk[t][i] = s.bt[t] * part;
      }
    }
  } else {
    // L_{t,i} for i < t < m, one pair per 16-lane group
    const int npairs = m * (m - 1) / 2;
    for (int pr = grp; pr < npairs; pr += kThreads / 16) {
      // pair pr = t (t - 1) / 2 + i, i < t, in closed form (the float root is
      // exact enough below 120 pairs; the two steps fix a rounding either way)
      int t = static_cast<int>((1.0f + sqrtf(8.0f * static_cast<float>(pr) + 1.0f)) * 0.5f);
      int i = pr - t * (t - 1) / 2;
      if (i >= t) {
        i -= t;
        ++t;
      }
      if (i < 0) {
        --t;
        i += t;
      }
      float part = lds_dot16<NK>(&s.K[t][0], &s.K[i][0], ln);
      part = group_sum16(part);
      if (ln == 0) {
        float r = 1.0f;
        for (int l = i + 1; l <= t; ++l) r *= s.al[l];
        s.kk[t][i] = s.bt[t] * r * part;
      }
    }
  }
  __syncthreads();
}

// S0 times the matvec rows, the forward substitution per own column, and the
// fold into S. Barriers inside; all threads call.
template <int NK, int NVS, bool VG>
__device__ __forceinline__ void rc_solve_and_fold(RegTile<4, NK, NVS>& S, GRcSmem<NK, NVS, VG>& s, int m) {
  const float* W = VG ? s.wt() : &s.K[0][0];
  if constexpr (NVS == 64) tile_matvec_mfma<kRing, NK, NVS, true, VG>(S, W, NK, s.red, &s.out[0][0]);
  else tile_matvec<kRing>(S, W, NK, s.red, &s.out[0][0]);
  for (int v = threadIdx.x; v < NVS; v += kThreads) {
    float ur[kRing];
#pragma unroll
    for (int t = 0; t < kRing; ++t) {
      if (t < m) {
        float u = VG ? s.bt[t] * (s.U[t][v] - s.out[t][v]) : s.bt[t] * (s.U[t][v] - s.gam[t] * s.out[t][v]);
#pragma unroll
        for (int i = 0; i < t; ++i) u -= s.kk[t][i] * ur[i];
        ur[t] = u;
        s.U[t][v] = VG ? u : u * s.rr[t];   // fold columns: r_{m-1,t} u_t (VG: the decay goes on k)
      }
    }
  }
  if constexpr (VG) {
    // fold rows r_{m-1,i} * k_i (descending direct products)
    for (int c = threadIdx.x; c < NK; c += kThreads) {
      float acc = 1.0f;
      for (int i = m - 1; i >= 0; --i) {
        s.K[i][c] *= acc;
        acc *= s.A[i][c];
      }
    }
  }
  __syncthreads();
  if constexpr (VG) {
    tile_scale_rows(S, s.gv);
    tile_rank_update(S, 1.0f, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  } else {
    tile_rank_update(S, s.gam[m - 1], &s.K[0][0], NK, &s.U[0][0], NVS, m);
  }
}

// A whole state held as two 64-column halves: S0 times the matvec rows for the
// half of columns c0.. and the forward substitution of those columns (as in
// rc_solve_and_fold). The weight rows stay in LDS for the other half.
// Barriers inside; all threads call.
template <int NK, int NU, bool VG>
__device__ __forceinline__ void rc_solve_half(const RegTile<4, NK, 64>& S, GRcSmem<NK, 64, VG, NU>& s, int m,
                                              int c0) {
  const float* W = VG ? s.wt() : &s.K[0][0];
  tile_matvec_mfma<kRing, NK, 64, true, false>(S, W, NK, s.red, &s.out[0][0]);
  for (int v = threadIdx.x; v < 64; v += kThreads) {
    float ur[kRing];
#pragma unroll
    for (int t = 0; t < kRing; ++t) {
      if (t < m) {
        float u = VG ? s.bt[t] * (s.U[t][c0 + v] - s.out[t][v])
                     : s.bt[t] * (s.U[t][c0 + v] - s.gam[t] * s.out[t][v]);
#pragma unroll
        for (int i = 0; i < t; ++i) u -= s.kk[t][i] * ur[i];
        ur[t] = u;
        s.U[t][c0 + v] = VG ? u : u * s.rr[t];
      }
    }
  }
  __syncthreads();   // out read before the scratch is reused
}

// NVFP4 codes and block scales of the 64 columns c0.. of state st held as
// RegTile<4, NK, 64>, under the tensor scale ts of the whole matrix: the bytes
// the whole-matrix quantizer writes for those columns (its blocks are the same
// four threads' 16 columns of one row).
template <int NK, int NV>
__device__ __forceinline__ void rc_store_nvfp4_half(const StateBuf& sb, size_t st, int c0, const RegTile<4, NK, 64>& M,
                                                    float ts) {
  using TM = TileMap<4, NK, 64>;
  const int c = static_cast<int>(threadIdx.x % TM::TPR);
  uint8_t* base = static_cast<uint8_t*>(sb.data) + st * NK * NV / 2;
  uint8_t* sbase = sb.nv_scale + st * NK * NV / 16;
#pragma unroll
  for (int k = 0; k < TM::PASSES; ++k) {
    const int row = RegTile<4, NK, 64>::row(k);
    const uint32_t sc = nvfp4_block_code<4>(M.v[k], ts);
    const uint32_t w = nvfp4_codes4(M.v[k], e4m3_value(sc) * ts);
    if (row < NK) {
      const int e = row * NV + c0 + 4 * c;
      *reinterpret_cast<uint16_t*>(base + e / 2) = static_cast<uint16_t>(w);
      if ((c & 3) == 0) sbase[e / 16] = static_cast<uint8_t>(sc);
    }
  }
}

}  // namespace

// flush step with a read copy: the rows of the len held entries and the
// current token re-solved from the checkpoint, the fold, one write, o = S q.
// COPY (states held whole, one workgroup per state): the NVFP4 read copy of the
// new state from the same registers; otherwise a requant launch follows.
template <typename TIN, int NK, int NV, bool VG, bool COPY>
__device__ __forceinline__ void gdn_flush_rc_body(const GDNArgs& a, GRcSmem<NK, NV / gdn_slices<NV>(), VG>& s) {
  static_assert(!COPY || gdn_slices<NV>() == 1, "the copy needs the whole state");
  constexpr int NVS = NV / gdn_slices<NV>();
  const GPtrs p = gdn_tile<NV, gdn_slices<NV>()>(a);
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * gdn_slices<NV>() + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * gdn_slices<NV>()) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 1 ? RS_ERR_FULL : 0);
  const int m = len + 1;
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, wg, nck, len, nd);
  } else {
    float* ck = static_cast<float*>(a.ck.data);
    GRcStage<TIN, NK, NV, NVS, VG> stg;
    stg.load(a, p.st, p.b, p.kh, p.c0, nck, len, true);   // records first, then the state tile
    GSlice<NK, NV, NVS> raw;
    raw.issue(ck, p.st, p.c0);
    arr.arrive(actr, wg, nck, len, nd);
    stg.store(s, m, true);
    __syncthreads();
    rc_gates_and_gram(s, m);
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    rc_solve_and_fold(S, s, m);
    GSlice<NK, NV, NVS>::store(ck, p.st, p.c0, S);
    tile_matvec<1>(S, s.q, NK, s.red, &s.out[0][0]);   // o = S_m q (barriers inside)
    for (int v = threadIdx.x; v < NVS; v += kThreads) a.o[p.st * NV + p.c0 + v] = s.out[0][v];
    if constexpr (COPY) tile_store_nvfp4(a.rc, p.st, S, tile_absmax(S, s.s4));
  }
  arr.finish(mp, actr, wg, a.nv * gdn_slices<NV>(), MetaOp::Flush, 0, nck, len, nd);
}

// A whole state of two 64-column halves folded with a read copy by one
// workgroup: the entries staged once (held entries, and with cur the current
// token), each half's rows re-solved against its own columns, both halves
// folded into S and written to the checkpoint. counted_in() runs between the
// loads and the staging (a step counts its workgroup in there). Barriers inside.
template <typename TIN, int NK, int NV, bool VG, typename F>
__device__ __forceinline__ void rc_fold_whole(const GDNArgs& a, GRcSmem<NK, 64, VG, NV>& s, size_t st, int b, int kh,
                                              long long nck, int held, bool cur, RegTile<4, NK, 64> (&S)[2],
                                              F counted_in) {
  static_assert(NV == 128, "two 64-column halves");
  const int m = held + (cur ? 1 : 0);
  float* ck = static_cast<float*>(a.ck.data);
  GRcStage<TIN, NK, NV, NV, VG> stg;
  stg.load(a, st, b, kh, 0, nck, held, cur);   // records first, then the state
  GSlice<NK, NV, 64> raw[2];
  raw[0].issue(ck, st, 0);
  raw[1].issue(ck, st, 64);
  counted_in();
  stg.store(s, m, cur);
  __syncthreads();
  rc_gates_and_gram(s, m);
  raw[0].decode(S[0]);
  raw[1].decode(S[1]);
  rc_solve_half(S[0], s, m, 0);
  rc_solve_half(S[1], s, m, 64);
  if constexpr (VG) {
    // fold rows r_{m-1,i} * k_i (descending direct products)
    for (int c = threadIdx.x; c < NK; c += kThreads) {
      float acc = 1.0f;
      for (int i = m - 1; i >= 0; --i) {
        s.K[i][c] *= acc;
        acc *= s.A[i][c];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (VG) {
      tile_scale_rows(S[h], s.gv);
      tile_rank_update(S[h], 1.0f, &s.K[0][0], NK, &s.U[0][64 * h], NV, m);
    } else {
      tile_rank_update(S[h], s.gam[m - 1], &s.K[0][0], NK, &s.U[0][64 * h], NV, m);
    }
    GSlice<NK, NV, 64>::store(ck, st, 64 * h, S[h]);
  }
}

// The NVFP4 read copy of a whole state held as two 64-column halves: one
// tensor scale from both halves' |max|. Barriers inside.
template <int NK, int NV, bool VG>
__device__ __forceinline__ void rc_copy_whole(const GDNArgs& a, GRcSmem<NK, 64, VG, NV>& s, size_t st,
                                              const RegTile<4, NK, 64> (&S)[2]) {
  float mx = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < RegTile<4, NK, 64>::P; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(S[h].v[k][i]));
  mx = wave_max(mx);
  __syncthreads();   // earlier readers of s4 are done
  if ((threadIdx.x & 63) == 0) s.s4[threadIdx.x >> 6] = mx;
  __syncthreads();
  const float ts = nvfp4_tscale_of(fmaxf(fmaxf(s.s4[0], s.s4[1]), fmaxf(s.s4[2], s.s4[3])));
  rc_store_nvfp4_half<NK, NV>(a.rc, st, 0, S[0], ts);
  rc_store_nvfp4_half<NK, NV>(a.rc, st, 64, S[1], ts);
  if (threadIdx.x == 0) a.rc.tscale[st] = ts;
}

// The read-copy flush of a state of two 64-column halves, folded by one
// workgroup with o = S_m q and the copy written from the same registers. NS:
// workgroups per state in the launch (any beyond the first only count in).
template <typename TIN, int NK, int NV, bool VG, int NS>
__device__ __forceinline__ void gdn_flush_rc_whole_body(const GDNArgs& a, GRcSmem<NK, 64, VG, NV>& s) {
  const GPtrs p = gdn_tile<NV, NS>(a);
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * NS + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * NS) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 1 ? RS_ERR_FULL : 0);
  Arrival arr;
  if (errbit != 0 || p.half != 0) {
    arr.arrive(actr, wg, nck, len, nd);
  } else {
    RegTile<4, NK, 64> S[2];
    rc_fold_whole<TIN, NK, NV, VG>(a, s, p.st, p.b, p.kh, nck, len, true, S,
                                   [&] { arr.arrive(actr, wg, nck, len, nd); });
    tiles_matvec<2>(S, s.q, s.red, &s.out[0][0]);   // o = S_m q: out[h][v] for column 64 h + v
    for (int v = threadIdx.x; v < NV; v += kThreads) a.o[p.st * NV + v] = (&s.out[0][0])[v];
    rc_copy_whole(a, s, p.st, S);
  }
  arr.finish(mp, actr, wg, a.nv * NS, MetaOp::Flush, 0, nck, len, nd);
}

// One workgroup per state, the read copy written in the same launch.
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_flush_rc_kernel(GDNArgs a) {
  if constexpr (gdn_slices<NV>() == 1) {
    __shared__ GRcSmem<NK, NV, VG> s;
    gdn_flush_rc_body<TIN, NK, NV, VG, true>(a, s);
  } else {
    __shared__ GRcSmem<NK, 64, VG, NV> s;
    gdn_flush_rc_whole_body<TIN, NK, NV, VG, 1>(a, s);
  }
}

// The LDS of a read-copy flush that folds the whole state: one tile, or two
// 64-column halves.
template <int NK, int NV, bool VG>
using GRcWholeSmem = typename std::conditional<gdn_slices<NV>() == 1, GRcSmem<NK, NV, VG>, GRcSmem<NK, 64, VG, NV>>::type;

template <int NK, int NV, bool VG>
union GAutoRcSmem {
  GSmem<NK, NV / gdn_slices<NV>(), VG> nf;
  GRcSmem<NK, NV / gdn_slices<NV>(), VG> fl;
};

// self-scheduling step with a read copy: the flushes fold in column slices, on
// the non-flush steps' grid, and a requant launch follows. (A whole-state flush
// here was measured slower: the non-flush steps pay its registers, and on the
// slice grid the second slice's workgroups would only count in.)
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_auto_rc_kernel(GDNArgs a) {
  __shared__ GAutoRcSmem<NK, NV, VG> s;
  const GPtrs p = gdn_tile<NV, gdn_slices<NV>()>(a);
  if (a.meta[p.b].len == kRing - 1) gdn_flush_rc_body<TIN, NK, NV, VG, false>(a, s.fl);
  else gdn_nonflush_body<TIN, NK, NV, VG, true>(a, s.nf);
}

// speculative commit with a read copy, fold part: as gdn_commit_fold_kernel,
// with the rows of the m committed entries re-solved from the checkpoint. One
// work item per state: the new checkpoint and its NVFP4 read copy are written
// from the same registers.
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_commit_fold_rc_kernel(GDNArgs a) {
  __shared__ GRcWholeSmem<NK, NV, VG> s;
  const int total = *a.work_count * a.nv;
  float* ckp = static_cast<float*>(a.ck.data);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const FoldItem it = a.work[item / a.nv];
    const int h = item - (item / a.nv) * a.nv, m = it.m;
    const size_t st = static_cast<size_t>(it.b) * a.nv + h;
    if constexpr (gdn_slices<NV>() == 1) {
      GRcStage<TIN, NK, NV, NV, VG> stg;
      stg.load(a, st, it.b, h / a.vpk, 0, it.nck, m, false);
      GSlice<NK, NV, NV> raw;
      raw.issue(ckp, st, 0);
      stg.store(s, m, false);
      __syncthreads();
      rc_gates_and_gram(s, m);
      RegTile<4, NK, NV> S;
      raw.decode(S);
      rc_solve_and_fold(S, s, m);
      GSlice<NK, NV, NV>::store(ckp, st, 0, S);
      tile_store_nvfp4(a.rc, st, S, tile_absmax(S, s.s4));
    } else {
      RegTile<4, NK, 64> S[2];
      rc_fold_whole<TIN, NK, NV, VG>(a, s, st, it.b, h / a.vpk, it.nck, m, false, S, [] {});
      rc_copy_whole(a, s, st, S);
    }
    __syncthreads();
  }
}

// The NVFP4 read copy of whole states from the fp32 checkpoint, one workgroup
// per state: every state, or (folded) those of sequences whose buffer is empty
// and holds no drafts. Bytes identical to the Mamba-2 quantizer's for the same
// matrix (same tile layout and encoder), and to what the folds that write the
// copy themselves store.
template <int NK, int NV>
__global__ __launch_bounds__(kThreads) void gdn_requant_kernel(GDNArgs a, int folded) {
  __shared__ float s4[4];
  const int mat = xcd_tile(blockIdx.x, gridDim.x);
  if (folded) {
    const rs_meta* mp = a.meta + mat / a.nv;
    if (mp->len != 0 || mp->nd != 0) return;   // uniform over the workgroup
  }
  RawTile<FMT_F32, 4, NK, NV> raw;   // four columns per thread: loads that cover whole rows
  raw.issue(a.ck, mat);
  RegTile<4, NK, NV> H;
  raw.decode(H);
  tile_store<FMT_NVFP4>(a.rc, mat, H, s4);
}

// ----------------------------------------------------------------------------
// speculative commit: the fold of the committed entries
// ----------------------------------------------------------------------------
// The NVS columns c0.. (a column slice, or the whole state) of a commit fold
// of state st over its m committed entries, into S (the checkpoint's columns
// read first).
template <typename TIN, int CKF, int NK, int NV, int NVS, bool VG>
__device__ __forceinline__ void gdn_commit_cols(const GDNArgs& a, const FoldItem& it, int h, int c0,
                                                GSmem<NK, NVS, VG>& s, GFoldTile<CKF, NK, NV, NVS>& S) {
  constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  constexpr int CU = (kRing * NVS / 4 + kThreads - 1) / kThreads;
  const int m = it.m;
  const size_t st = static_cast<size_t>(it.b) * a.nv + h;
  const size_t bk = static_cast<size_t>(it.b) * a.nqk + h / a.vpk;
  const TIN* rk = static_cast<const TIN*>(a.rk) + bk * kRing * NK;
  const float* ru = static_cast<const float*>(a.ru) + st * kRing * NV + c0;
  RegChunks<TIN, CK> ck;
  RegChunks<float, CU> cu;
  ck.load(EntrySrc<TIN>{rk, rk, 0, it.nck, m, NK}, m, NK);
  cu.load(EntrySrc<float>{ru, ru, 0, it.nck, m, NV}, m, NVS);
  float gv = 0.0f;
  float lg[VG ? kRing : 1];   // VG: log decays of the m entries, this thread's key channel
  if constexpr (VG) {
    const int c = static_cast<int>(threadIdx.x) < NK ? static_cast<int>(threadIdx.x) : NK - 1;
    const float* rgc = static_cast<const float*>(a.rg) + st * kRing * NK + c;
#pragma unroll
    for (int e = 0; e < kRing; ++e) lg[e] = rgc[slot_of(it.nck, e < m ? e : m - 1) * NK];
  } else {
    const int e = static_cast<int>(threadIdx.x) < m ? static_cast<int>(threadIdx.x) : m - 1;
    gv = static_cast<const float*>(a.rg)[st * kRing + slot_of(it.nck, e)];
  }
  GFoldRaw<CKF, NK, NV, NVS> raw;
  fold_issue(raw, a.ck, st, c0);
  ck.to_lds(&s.K[0][0], NK, m, NK);
  cu.to_lds(&s.U[0][0], NVS, m, NVS);
  if constexpr (!VG)
    if (static_cast<int>(threadIdx.x) < m) s.al[threadIdx.x] = expf(gv);
  __syncthreads();
  if constexpr (VG) {
    // channel owners: k rows times r_{m,i} (descending direct products), gamma_m
    if (static_cast<int>(threadIdx.x) < NK) {
      float acc = 1.0f;
#pragma unroll
      for (int i = kRing - 1; i >= 0; --i) {
        if (i < m) {
          s.K[i][threadIdx.x] *= acc;
          acc *= kda_alpha(lg[i]);
        }
      }
      s.gv[threadIdx.x] = acc;
    }
  } else {
    if (static_cast<int>(threadIdx.x) < m) {
      float w = 1.0f;
#pragma unroll
      for (int l = 1; l < kRing; ++l) w *= (l > static_cast<int>(threadIdx.x) && l < m) ? s.al[l] : 1.0f;
      s.rr[threadIdx.x] = w;
    }
    if (threadIdx.x == 0) {
      float gm = 1.0f;
#pragma unroll
      for (int l = 0; l < kRing; ++l) gm *= l < m ? s.al[l] : 1.0f;
      s.gam = gm;
    }
    __syncthreads();
    for (int v = threadIdx.x; v < NVS; v += kThreads)
#pragma unroll
      for (int i = 0; i < kRing; ++i)
        if (i < m) s.U[i][v] *= s.rr[i];
  }
  __syncthreads();
  raw.decode(S);
  if constexpr (gdn_mfma_fold<CKF, NK, NV, NVS>()) {
    if constexpr (VG) mtile_scale_rows(S, s.gv);
    else mtile_scale(S, s.gam);
    mtile_rank_update(S, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  } else if constexpr (VG) {
    tile_scale_rows(S, s.gv);
    tile_rank_update(S, 1.0f, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  } else {
    tile_rank_update(S, s.gam, &s.K[0][0], NK, &s.U[0][0], NVS, m);
  }
}

// speculative commit (ReplaySSM), fold part: for each sequence listed by
// commit_meta, S <- gamma_m S0 + sum_i r_{m,i} u_i k_i^T over its m committed
// entries (u rows from the ring), one column slice per work item, over a
// fixed grid (every workgroup leaves when the list is done). VG (KDA):
// S <- S0 Diag(gamma_m) + sum_i u_i (r_{m,i} * k_i)^T with per-channel decays.
// FP8 checkpoints: one item per state, folding every column (one scale spans
// the matrix).
template <typename TIN, int NK, int NV, bool VG, int CKF = FMT_F32>
__global__ __launch_bounds__(kThreads) void gdn_commit_fold_kernel(GDNArgs a) {
  constexpr int NVS = gdn_fold_cols<NV, CKF>();
  constexpr int NS = NV / NVS;
  static_assert(!VG || NK <= kThreads, "one thread per key channel");
  __shared__ GSmem<NK, NVS, VG> s;
  const int per = a.nv * NS;
  const int total = *a.work_count * per;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const FoldItem it = a.work[item / per];
    const int r = item - (item / per) * per;
    const int h = r / NS, half = r - h * NS;
    const size_t st = static_cast<size_t>(it.b) * a.nv + h;
    GFoldTile<CKF, NK, NV, NVS> S;
    gdn_commit_cols<TIN, CKF, NK, NV, NVS, VG>(a, it, h, half * NVS, s, S);
    if constexpr (CKF == FMT_FP8) gdn_store_fp8(a, st, s, S);
    else GSliceF<CKF, NK, NV, NVS>::store(a.ck, st, half * NVS, S);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// snapshot baseline: step the live state through K drafts, write each state to
// snap[d] and each output; the live state is not written here (the restore
// below makes the snapshot after the last accepted draft live)
// ----------------------------------------------------------------------------
namespace {

template <int NK, int NVS, int KQ, bool VG>
struct GConvSpecSmem {
  float AL[VG ? KQ : 1][NK];   // VG: the channel decays of each draft
  float W[2 * KQ][NK];   // k_d, q_d
  float V[KQ][NVS];      // v_d, own columns
  float out[2][NVS];     // S k_d, S q_d
  float red[4 * 2 * NVS];
  float U[NVS];
  float kq[KQ], al[KQ], bet[KQ];
};

}  // namespace

// One workgroup per column slice, as in the replay kernels (the delta rule is
// column-independent in the stored layout): the whole 128 x 128 state in one
// workgroup needs 132 registers per lane here and runs at 3 waves per SIMD.
template <typename TIN, int NK, int NV, int KQ, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_conv_spec_kernel(GDNArgs a) {
  constexpr int NS = gdn_slices<NV>();
  constexpr int NVS = NV / NS;
  constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  constexpr int CD = (KQ * NK / VK + kThreads - 1) / kThreads;
  constexpr int CV = (KQ * NVS / VK + kThreads - 1) / kThreads;
  constexpr int CA = VG ? (KQ * NK / 4 + kThreads - 1) / kThreads : 1;
  __shared__ GConvSpecSmem<NK, NVS, KQ, VG> s;
  const GPtrs p = gdn_tile<NV, NS>(a);
  const int K = a.K;
  const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
  const size_t kstride = static_cast<size_t>(a.batch) * a.nqk * NK;
  const size_t vstride = static_cast<size_t>(a.batch) * a.nv * NV;
  const size_t gstride = static_cast<size_t>(a.batch) * a.nv;
  const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
  const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
  const TIN* iv = static_cast<const TIN*>(a.v) + p.st * NV + p.c0;
  RegChunks<TIN, CD> cq, cd;
  RegChunks<TIN, CV> cv;
  cq.load(EntrySrc<TIN>{iq, iq, kstride, 0, 0, NK}, K, NK);
  cd.load(EntrySrc<TIN>{ik, ik, kstride, 0, 0, NK}, K, NK);
  cv.load(EntrySrc<TIN>{iv, iv, vstride, 0, 0, NVS}, K, NVS);
  RegChunks<float, CA> ca;
  if constexpr (VG) {
    const float* ig = a.g + p.st * NK;
    ca.load(EntrySrc<float>{ig, ig, gstride * NK, 0, 0, NK}, K, NK);
  }
  const int dd = static_cast<int>(threadIdx.x) < K ? static_cast<int>(threadIdx.x) : K - 1;
  const float gv = VG ? 0.0f : a.g[dd * gstride + p.st], bv = a.beta[dd * gstride + p.st];
  float* ck = static_cast<float*>(a.ck.data);
  GSlice<NK, NV, NVS> raw;
  raw.issue(ck, p.st, p.c0);
  cd.to_lds(&s.W[0][0], 2 * NK, K, NK);
  cq.to_lds(&s.W[1][0], 2 * NK, K, NK);
  cv.to_lds(&s.V[0][0], NVS, K, NVS);
  if constexpr (VG) ca.to_lds(&s.AL[0][0], NK, K, NK);
  if (static_cast<int>(threadIdx.x) < K) {
    s.al[threadIdx.x] = VG ? 1.0f : expf(gv);   // VG: the decay is applied to the rows
    s.bet[threadIdx.x] = bv;
  }
  __syncthreads();
  if constexpr (VG) {
    for (int idx = threadIdx.x; idx < K * NK; idx += kThreads) (&s.AL[0][0])[idx] = kda_alpha((&s.AL[0][0])[idx]);
    __syncthreads();
  }
  {
    const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
    for (int d = grp; d < K; d += kThreads / 16) {
      float part = 0.0f;
      for (int c = ln; c < NK; c += 16) part += s.W[2 * d][c] * s.W[2 * d + 1][c];
      part = group_sum16(part);
      if (ln == 0) s.kq[d] = part;
    }
  }
  RegTile<4, NK, NVS> S;
  raw.decode(S);
  for (int d = 0; d < K; ++d) {
    if constexpr (VG) tile_scale_rows(S, &s.AL[d][0]);        // S Diag(alpha_d)
    tile_matvec<2>(S, &s.W[2 * d][0], NK, s.red, &s.out[0][0]);   // S k_d, S q_d (barriers inside)
    const float al = s.al[d], be = s.bet[d], kq = s.kq[d];
    for (int v = threadIdx.x; v < NVS; v += kThreads) {
      const float u = be * (s.V[d][v] - al * s.out[0][v]);
      s.U[v] = u;
      a.o[d * vstride + p.st * NV + p.c0 + v] = al * s.out[1][v] + kq * u;
    }
    __syncthreads();
    tile_rank_update(S, al, &s.W[2 * d][0], NK, s.U, NVS, 1);
    GSlice<NK, NV, NVS>::store(a.snap + d * vstride * NK, p.st, p.c0, S);
    __syncthreads();
  }
}

// snapshot baseline commit: the snapshot after draft k[b] becomes the live state
template <int NK, int NV>
__global__ __launch_bounds__(kThreads) void gdn_restore_kernel(GDNArgs a) {
  const GPtrs p = gdn_tile<NV, 1>(a);
  const int k = a.accepted[p.b];
  if (k < 1 || k > a.kmax) return;
  const size_t mat = static_cast<size_t>(NK) * NV;
  const float4* src = reinterpret_cast<const float4*>(
      a.snap + (static_cast<size_t>(k - 1) * a.batch * a.nv + p.st) * mat);
  float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.ck.data) + p.st * mat);
  for (size_t i = threadIdx.x; i < mat / 4; i += kThreads) nt_store(nt_load(src + i), dst + i);
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
namespace {

template <int NK, int NV, bool VG, bool RC, int CKF>
struct gdn_step_kernels {
  static void conv(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_conv_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_conv_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
  static void nonflush(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_nonflush_kernel<bf16, NK, NV, VG, RC, CKF><<<grid, kThreads, 0, st>>>(a);
    else gdn_nonflush_kernel<float, NK, NV, VG, RC, CKF><<<grid, kThreads, 0, st>>>(a);
  }
  static void flush(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if constexpr (RC) {
      if (bf) gdn_flush_rc_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
      else gdn_flush_rc_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    } else {
      if (bf) gdn_flush_kernel<bf16, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
      else gdn_flush_kernel<float, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
    }
  }
  static void auto_step(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if constexpr (RC) {
      if (bf) gdn_auto_rc_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
      else gdn_auto_rc_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    } else {
      if (bf) gdn_auto_kernel<bf16, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
      else gdn_auto_kernel<float, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
    }
  }
};

template <typename TIN, int NK, int NV, bool VG, bool RC, int CKF>
void gdn_spec_append(const GDNArgs& a, int grid, hipStream_t st) {
  if (a.K <= 2) gdn_spec_append_kernel<TIN, NK, NV, 2, VG, RC, CKF><<<grid, kThreads, 0, st>>>(a);
  else if (a.K <= 4) gdn_spec_append_kernel<TIN, NK, NV, 4, VG, RC, CKF><<<grid, kThreads, 0, st>>>(a);
  else gdn_spec_append_kernel<TIN, NK, NV, 8, VG, RC, CKF><<<grid, kThreads, 0, st>>>(a);
}

template <typename TIN, int NK, int NV, bool VG>
void gdn_conv_spec(const GDNArgs& a, int grid, hipStream_t st) {
  if (a.K <= 2) gdn_conv_spec_kernel<TIN, NK, NV, 2, VG><<<grid, kThreads, 0, st>>>(a);
  else if (a.K <= 4) gdn_conv_spec_kernel<TIN, NK, NV, 4, VG><<<grid, kThreads, 0, st>>>(a);
  else gdn_conv_spec_kernel<TIN, NK, NV, 8, VG><<<grid, kThreads, 0, st>>>(a);
}

template <int NK, int NV, bool VG, bool RC, int CKF>
void gdn_spec_kernels(GDNOp op, bool bf, const GDNArgs& a, int grid, hipStream_t st) {
  if (op == GDNOp::SpecAppend) {
    if (bf) gdn_spec_append<bf16, NK, NV, VG, RC, CKF>(a, grid, st);
    else gdn_spec_append<float, NK, NV, VG, RC, CKF>(a, grid, st);
  } else if (op == GDNOp::ConvSpec) {
    if (bf) gdn_conv_spec<bf16, NK, NV, VG>(a, grid, st);
    else gdn_conv_spec<float, NK, NV, VG>(a, grid, st);
  } else if constexpr (RC) {
    if (bf) gdn_commit_fold_rc_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_commit_fold_rc_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  } else {
    if (bf) gdn_commit_fold_kernel<bf16, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
    else gdn_commit_fold_kernel<float, NK, NV, VG, CKF><<<grid, kThreads, 0, st>>>(a);
  }
}

template <int NK, int NV, bool VG, bool RC, int CKF>
void gdn_launch_kind(GDNOp op, const GDNArgs& a, GDNLaunch l, hipStream_t st) {
  const bool bf = l.in_bf16;
  using Steps = gdn_step_kernels<NK, NV, VG, RC, CKF>;
  switch (op) {
    case GDNOp::Conv: Steps::conv(bf, a, l.grid, st); break;
    case GDNOp::NonFlush: Steps::nonflush(bf, a, l.grid, st); break;
    case GDNOp::Flush: Steps::flush(bf, a, l.grid, st); break;
    case GDNOp::Auto: Steps::auto_step(bf, a, l.grid, st); break;
    case GDNOp::SpecAppend:
    case GDNOp::ConvSpec: gdn_spec_kernels<NK, NV, VG, RC, CKF>(op, bf, a, l.grid, st); break;
    case GDNOp::CommitFold: {
      const int items = l.grid * gdn_slices<NV>();   // upper bound of listed work items
      gdn_spec_kernels<NK, NV, VG, RC, CKF>(op, bf, a, items < 2048 ? items : 2048, st);
      break;
    }
    case GDNOp::Restore: gdn_restore_kernel<NK, NV><<<l.grid, kThreads, 0, st>>>(a); break;
    case GDNOp::Requant: gdn_requant_kernel<NK, NV><<<l.grid, kThreads, 0, st>>>(a, 0); break;
    case GDNOp::RequantFolded: gdn_requant_kernel<NK, NV><<<l.grid, kThreads, 0, st>>>(a, 1); break;
  }
}

template <int NK, int NV>
void gdn_launch_shape(GDNOp op, const GDNArgs& a, GDNLaunch l, hipStream_t st) {
  // replay steps and appends: one workgroup per column slice of each state
  // (the flush of an FP8 checkpoint or with a read copy: one per state)
  if ((op == GDNOp::Flush && (l.rc || l.ckf == FMT_FP8)) || (op == GDNOp::NonFlush && (l.rc || l.ckf != FMT_F32)))
    l.grid *= 1;
  else if (op == GDNOp::NonFlush || op == GDNOp::Flush || op == GDNOp::Auto || op == GDNOp::SpecAppend ||
           op == GDNOp::ConvSpec)
    l.grid *= gdn_slices<NV>();
  if (l.rc) {   // the read copy sits beside an fp32 checkpoint
    if (l.vg) gdn_launch_kind<NK, NV, true, true, FMT_F32>(op, a, l, st);
    else gdn_launch_kind<NK, NV, false, true, FMT_F32>(op, a, l, st);
    return;
  }
  if constexpr (NK != 64) {   // FP16 / FP8 checkpoints: the 16 x 16 and 128 x 128 states
    if (l.ckf == FMT_F16) {
      if (l.vg) gdn_launch_kind<NK, NV, true, false, FMT_F16>(op, a, l, st);
      else gdn_launch_kind<NK, NV, false, false, FMT_F16>(op, a, l, st);
      return;
    }
    if (l.ckf == FMT_FP8) {
      if (l.vg) gdn_launch_kind<NK, NV, true, false, FMT_FP8>(op, a, l, st);
      else gdn_launch_kind<NK, NV, false, false, FMT_FP8>(op, a, l, st);
      return;
    }
  }
  if (l.vg) gdn_launch_kind<NK, NV, true, false, FMT_F32>(op, a, l, st);
  else gdn_launch_kind<NK, NV, false, false, FMT_F32>(op, a, l, st);
}

}  // namespace

// The compiled shapes are the ones gdn_shape_supported (rs_host.cpp) accepts.
void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (l.dk == 16 && l.dv == 16) gdn_launch_shape<16, 16>(op, a, l, st);
  else if (l.dk == 64 && l.dv == 64) gdn_launch_shape<64, 64>(op, a, l, st);
  else if (l.dk == 128 && l.dv == 128) gdn_launch_shape<128, 128>(op, a, l, st);
}

}  // namespace rs
